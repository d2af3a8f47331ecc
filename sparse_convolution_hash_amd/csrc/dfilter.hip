// Weight and bias gradients of the sparse convolution.
//
//   dW[k] = sum over the pairs (i, o) of offset k of x[i]^T dy[o]   [cin, cout]
//   dbias = sum over rows o of dy[o]                                 [cout]
//
// (the Hygon spconv-das README's dfilter, "Public Interface Support").  The
// contraction runs over pairs.  The CSR pair list is cut into one segment of
// equal length per workgroup; a workgroup walks its segment in steps of up
// to 64 pairs (a step never straddles two offsets), gathers each step's rows
// and transposes them in registers into channel-major LDS tiles (the MFMA
// fragments need 16 bytes of consecutive pairs per channel), accumulates
// fp32 on MFMA, and writes one partial tile per offset it touches.  Pair
// indices are fetched two steps ahead and rows one step ahead.  A second
// kernel sums each offset's partials in segment order, so the result does
// not depend on scheduling.
#include <algorithm>
#include <mutex>

#include "common.h"

namespace spc {
namespace {

constexpr int DT = 256;          // threads per workgroup (2 x 2 waves)
constexpr int PS = 64;           // pairs staged per step
constexpr int TMAX = 128;        // channel tile edge
constexpr int MAX_WG = 512;           // segments (workgroups) over all channel tiles
constexpr int MAX_K = 343;            // offsets (pair_ptr is staged in LDS)

struct DfArgs {
    const void* x;        // [n_in, cin]
    const void* dy;       // [n_out, cout]
    const int32_t* ptr;   // [K+1] or NULL (identity pairs, K == 1)
    const int32_t* pin;
    const int32_t* pout;
    float* part;          // [nseg + K, cin, cout] partial tiles
    int32_t n_in, n_out, cin, cout, K;
    int32_t nseg;         // segments of the pair list (workgroups per channel tile)
};

// Pair ranges.  Segment b is [b*seg, (b+1)*seg) of the pair list, with seg a
// multiple of PS and about P / nseg; the same numbers are derived from
// pair_ptr by every workgroup and by the reduction.
__device__ __forceinline__ int64_t pairs_total(const DfArgs& a) { return a.ptr ? a.ptr[a.K] : a.n_in; }
__device__ __forceinline__ int64_t off_beg(const DfArgs& a, int k) { return a.ptr ? a.ptr[k] : 0; }
__device__ __forceinline__ int64_t off_end(const DfArgs& a, int k) { return a.ptr ? a.ptr[k + 1] : a.n_in; }

// pair_ptr (or the identity's [0, n_in]) in LDS: the step walk reads it
// there, so it never waits on the vector memory counter of the prefetches.
__device__ __forceinline__ void stage_ptr(int32_t* sptr, const DfArgs& a) {
    for (int k = threadIdx.x; k <= a.K; k += blockDim.x) sptr[k] = a.ptr ? a.ptr[k] : (k == 0 ? 0 : a.n_in);
    __syncthreads();
}
__device__ __forceinline__ int64_t seg_len(const DfArgs& a, int64_t P) {
    const int64_t s = (P + a.nseg - 1) / a.nseg;
    return s < PS ? PS : (s + PS - 1) / PS * PS;
}

// One step: pairs [b, e) of offset k (e > b), or none (k < 0).
struct Step {
    int64_t b, e;
    int k;
};

// The step starting at pair p of segment end s1, from offset k on (sptr:
// pair_ptr staged in LDS).
__device__ __forceinline__ Step step_at(const int32_t* sptr, int64_t p, int k, int64_t s1) {
    if (p >= s1) return Step{0, 0, -1};
    while (sptr[k + 1] <= p) ++k;  // p < s1 <= P: ends inside the offsets
    const int64_t e0 = sptr[k + 1], e1 = p + PS;
    return Step{p, min(min(e0, e1), s1), k};
}

// Row stride (bytes) of a channel-major LDS tile: PS pairs plus 16 bytes of
// padding so that consecutive channels fall in different banks.
template <typename TT>
constexpr int lds_row() { return PS * int(sizeof(typename TT::storage)) + 16; }

// One staging item: E consecutive pairs x E consecutive channels of one operand.
template <typename TT>
struct Item {
    u32x4 in[TT::E];
    uint32_t ok;  // bit e: slot e holds a real row (else it is zeroed when stored)
};

// Item geometry: item j of a step is E consecutive pairs (group pg) x E
// consecutive channels (block ch) of x (j < xi_items) or of dy.
struct ItemGeo {
    bool is_x;
    int pg, ch;
    __device__ ItemGeo(int item, int xi_items, int E) {
        is_x = item < xi_items;
        const int j = is_x ? item : item - xi_items;
        pg = j % (PS / E);
        ch = j / (PS / E);
    }
};

// Pair indices (rows of x or dy) of an item's pairs in step st: unguarded
// loads from clamped, valid positions of the step.
template <typename TT, bool IDENT>
__device__ __forceinline__ void load_idx(int32_t (&r)[TT::E], const DfArgs& a, const ItemGeo& g, const Step& st) {
    constexpr int E = TT::E;
    const int32_t* idx = g.is_x ? a.pin : a.pout;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int64_t p = st.b + g.pg * E + e;
        const int64_t pc = p < st.e ? p : st.e - 1;
        if constexpr (IDENT)
            r[e] = int32_t(pc);
        else
            r[e] = idx[pc];
    }
}

// The item's rows for step st, from indices r: unguarded loads (an invalid
// slot reads row 0 and is zeroed when stored, not here: a select right after
// the loads would wait for them).
template <typename TT>
__device__ __forceinline__ void load_rows(Item<TT>& it, const int32_t (&r)[TT::E], const DfArgs& a, const ItemGeo& g,
                                          int ci0, int co0, const Step& st) {
    using S = typename TT::storage;
    constexpr int E = TT::E;
    const S* src = g.is_x ? static_cast<const S*>(a.x) : static_cast<const S*>(a.dy);
    const int C = g.is_x ? a.cin : a.cout;
    const int c0 = (g.is_x ? ci0 : co0) + g.ch * E;
    const int32_t lim = g.is_x ? a.n_in : a.n_out;
    it.ok = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const bool ok = st.b + g.pg * E + e < st.e && (unsigned)r[e] < (unsigned)lim;
        it.in[e] = ld16(src + int64_t(ok ? r[e] : 0) * C + c0);
        it.ok |= uint32_t(ok) << e;
    }
}

// Writes a loaded item transposed: lds[channel][pair], 16 bytes of
// consecutive pairs per channel.
template <typename TT>
__device__ __forceinline__ void store_item(char* xt, char* gt, const Item<TT>& it, int item, int xi_items) {
    constexpr int E = TT::E;
    constexpr int PG = PS / E;
    const bool is_x = item < xi_items;
    const int j = is_x ? item : item - xi_items;
    const int pg = j % PG, ch = j / PG;
    char* dst = (is_x ? xt : gt) + (ch * E) * lds_row<TT>() + pg * 16;
    u32x4 in[E];
#pragma unroll
    for (int e = 0; e < E; ++e) in[e] = (it.ok >> e) & 1u ? it.in[e] : zero4();
    if constexpr (E == 8) {
        typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
        u16x8 v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = __builtin_bit_cast(u16x8, in[e]);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            u16x8 o = {v[0][c], v[1][c], v[2][c], v[3][c], v[4][c], v[5][c], v[6][c], v[7][c]};
            st16(dst + c * lds_row<TT>(), __builtin_bit_cast(u32x4, o));
        }
    } else {
        const uint32_t m[4][4] = {{in[0].x, in[0].y, in[0].z, in[0].w},
                                  {in[1].x, in[1].y, in[1].z, in[1].w},
                                  {in[2].x, in[2].y, in[2].z, in[2].w},
                                  {in[3].x, in[3].y, in[3].z, in[3].w}};
#pragma unroll
        for (int c = 0; c < 4; ++c) st16(dst + c * lds_row<TT>(), u32x4{m[0][c], m[1][c], m[2][c], m[3][c]});
    }
}

// Staging with transposing reads (16-bit full tiles): a step's rows stay
// pair-major in LDS, as they were loaded, and each MFMA fragment (8
// consecutive pairs of one channel) comes from two ds_read_b64_tr_b16 reads
// (within a 16-lane group, lane i receives element i & 3 of the rows that
// lanes 4q + (i >> 2) point at).  Slot q of thread t holds 16-byte chunk
// t + DT*q of the step: the x chunks first (TI / 8 per pair), then the dy
// chunks (TO / 8 per pair), so 16 consecutive lanes read whole rows and a
// load instruction touches a few rows, not one row per lane.
template <int MIM, int NOM>
struct TrGeo {
    static constexpr int TI = 32 * MIM, TO = 32 * NOM;     // the full tile's channels
    static constexpr int XC = PS * TI / 8;                 // x chunks of a step (a multiple of DT)
    static constexpr int NQ = PS * (TI + TO) / 8 / DT;     // slots per thread
    static constexpr int RSX = TI * 2 + 32, RSG = TO * 2 + 32;  // LDS row strides (bytes), padded against bank conflicts
    static_assert(XC % DT == 0 && NQ * DT * 8 == PS * (TI + TO) && NQ <= 8, "whole slots per thread");
    __device__ static constexpr bool is_x(int q) { return q * DT < XC; }
    __device__ static constexpr int cpr(int q) { return is_x(q) ? TI / 8 : TO / 8; }
    // chunk index of slot q within its operand's part of the step
    __device__ static int slot(int q) { return int(threadIdx.x) + DT * (is_x(q) ? q : q - XC / DT); }
    __device__ static int pair(int q) { return slot(q) / cpr(q); }
    __device__ static int chunk(int q) { return slot(q) % cpr(q); }
};

template <typename TT, bool IDENT, int MIM, int NOM>
__device__ __forceinline__ void load_idx_tr(int32_t (&r)[TT::E], const DfArgs& a, const Step& st) {
    using G = TrGeo<MIM, NOM>;
#pragma unroll
    for (int q = 0; q < G::NQ; ++q) {
        const int64_t p = st.b + G::pair(q);
        int64_t pc = p < st.e ? p : st.e - 1;
        pc = pc < 0 ? 0 : pc;  // a step past the end (b = e = 0) reads entry 0 and drops it
        if constexpr (IDENT)
            r[q] = int32_t(pc);
        else
            r[q] = (G::is_x(q) ? a.pin : a.pout)[pc];
    }
}

template <typename TT, int MIM, int NOM>
__device__ __forceinline__ void load_rows_tr(Item<TT>& it, const int32_t (&r)[TT::E], const DfArgs& a, int ci0,
                                             int co0, const Step& st) {
    using S = typename TT::storage;
    using G = TrGeo<MIM, NOM>;
    it.ok = 0;
#pragma unroll
    for (int q = 0; q < G::NQ; ++q) {
        const bool x = G::is_x(q);
        const S* src = x ? static_cast<const S*>(a.x) : static_cast<const S*>(a.dy);
        const int C = x ? a.cin : a.cout;
        const int32_t lim = x ? a.n_in : a.n_out;
        const bool ok = st.b + G::pair(q) < st.e && (unsigned)r[q] < (unsigned)lim;
        it.in[q] = ld16(src + int64_t(ok ? r[q] : 0) * C + (x ? ci0 : co0) + G::chunk(q) * 8);
        it.ok |= uint32_t(ok) << q;
    }
}

template <typename TT, int MIM, int NOM>
__device__ __forceinline__ void store_item_tr(char* xt, char* gt, const Item<TT>& it) {
    using G = TrGeo<MIM, NOM>;
#pragma unroll
    for (int q = 0; q < G::NQ; ++q) {
        const bool x = G::is_x(q);
        char* dst = (x ? xt : gt) + G::pair(q) * (x ? G::RSX : G::RSG) + G::chunk(q) * 16;
        st16(dst, (it.ok >> q) & 1u ? it.in[q] : zero4());
    }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// One MFMA fragment from the pair-major tile: channel n0 + (lane & 15), pairs
// k0 .. k0 + 7 with k0 = 8 * (lane >> 4) + 32 * ks
__device__ __forceinline__ u32x4 tr_fragment(const char* tile, int rs, int n0, int ks, int lr, int lg) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const char* p0 = tile + ((ks * 4 + lg) * 8 + (lr >> 2)) * rs + n0 * 2 + 8 * (lr & 3);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 4 * rs));
    const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
    return u32x4{l2.x, l2.y, h2.x, h2.y};
}

// Workgroup b walks segment b of the pair list in steps; each offset it
// touches gets one partial tile, part[b + k] (b + k is distinct for every
// (segment, offset) pair a walk can meet, as both only grow along it).
// IDENT: K == 1 with the identity pairs (i, i), no pair lists.  MIM x NOM:
// the most 16x16 blocks a wave holds (channel tiles of up to 32*MIM x
// 32*NOM).  DEPTH: steps of rows in flight (2 fits the registers only with
// small accumulator tiles); pair indices are fetched one step earlier still.
// FULL: every channel tile is exactly 2 x MIM by 2 x NOM blocks of 16, so no
// block needs a bound check (the checks would split the MFMA loop into one
// branch per block, each waiting for every LDS read before it)
template <typename TT, bool IDENT, int MIM, int NOM, int DEPTH, bool FULL>
__global__ __launch_bounds__(DT) __attribute__((amdgpu_waves_per_eu(2))) void k_dfilter(DfArgs a) {
    static_assert(DEPTH == 1 || DEPTH == 2, "one or two steps of rows in flight");
    constexpr int E = TT::E;
    constexpr int ROW = lds_row<TT>();
    __shared__ __attribute__((aligned(16))) char xt[TMAX * ROW];  // [ci][pairs]
    __shared__ __attribute__((aligned(16))) char gt[TMAX * ROW];  // [co][pairs]
    __shared__ int32_t sptr[MAX_K + 1];

    const int tiles_o = (a.cout + TMAX - 1) / TMAX;
    const int ci0 = (blockIdx.y / tiles_o) * TMAX, co0 = (blockIdx.y % tiles_o) * TMAX;
    const int TI = min(TMAX, a.cin - ci0), TO = min(TMAX, a.cout - co0);
    const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
    const int lr = lane & 15, lg = lane >> 4;
    const int wi = wave >> 1, wo = wave & 1;
    const int MI = FULL ? MIM : (TI / 16 + 1) / 2, NO = FULL ? NOM : (TO / 16 + 1) / 2;  // 16x16 blocks per wave (<= MIM, NOM)
    constexpr int PG = PS / E;
    const int xi_items = PG * (TI / E), items = xi_items + PG * (TO / E);

    const int64_t P = pairs_total(a), seg = seg_len(a, P);
    const int64_t s0 = int64_t(blockIdx.x) * seg, s1 = min(P, s0 + seg);
    if (s0 >= s1 || a.n_in == 0 || a.n_out == 0) return;  // (no rows: no valid pair either)
    stage_ptr(sptr, a);

    // this thread's pipelined item (threads beyond the items load a copy of
    // the last one and do not store it)
    const int my = threadIdx.x;
    const bool has_item = my < items;
    const ItemGeo geo(has_item ? my : items - 1, xi_items, E);
    // 16-bit full tiles stage rows pair-major and read fragments transposed
    constexpr bool TR = FULL && E == 8;
    // with accumulators of up to 2 x 2 blocks per wave the step's loads are
    // branch-free and spread among its MFMAs (larger tiles have no registers
    // to spare for it: the 4 x 4 one did not get faster, the 3 x 3 one lost
    // a wave per SIMD)
    constexpr bool SPREAD = TR && MIM <= 2 && NOM <= 2;
    auto idx_of = [&](int32_t (&r)[E], const Step& st) {
        if constexpr (TR)
            load_idx_tr<TT, IDENT, MIM, NOM>(r, a, st);
        else
            load_idx<TT, IDENT>(r, a, geo, st);
    };
    auto rows_of = [&](Item<TT>& it, const int32_t (&r)[E], const Step& st) {
        if constexpr (TR)
            load_rows_tr<TT, MIM, NOM>(it, r, a, ci0, co0, st);
        else
            load_rows<TT>(it, r, a, geo, ci0, co0, st);
    };

    f32x4_t acc[MIM][NOM];
#pragma unroll
    for (int mi = 0; mi < MIM; ++mi)
#pragma unroll
        for (int no = 0; no < NOM; ++no) acc[mi][no] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // the step pipeline: cur (rows landed or landing), then DEPTH - 1 more
    // steps of rows in flight, then one step of pair indices in flight
    Step cur = step_at(sptr, s0, 0, s1);
    Step nxt = step_at(sptr, cur.e, cur.k, s1);
    Step nx2 = (DEPTH == 2 && nxt.k >= 0) ? step_at(sptr, nxt.e, nxt.k, s1) : Step{0, 0, -1};
    Item<TT> ra, rb;       // rows (rb only for DEPTH 2)
    int32_t ia[E], ib[E];  // pair indices of the step whose rows are loaded next
    {
        int32_t r0[E], r1[E];
        idx_of(r0, cur);
        if (DEPTH == 2 && nxt.k >= 0) idx_of(r1, nxt);
        const Step& ahead = DEPTH == 2 ? nx2 : nxt;
        if (ahead.k >= 0) idx_of(ia, ahead);
        rows_of(ra, r0, cur);
        if (DEPTH == 2 && nxt.k >= 0) rows_of(rb, r1, nxt);
    }

    // one step: cur's rows are in `mine`, which is then refilled with the
    // rows of the step DEPTH ahead (indices in `use`); the indices of the
    // step after that go to `fill`
    auto step = [&](Item<TT>& mine, const int32_t (&use)[E], int32_t (&fill)[E]) {
        const Step& ahead = DEPTH == 2 ? nx2 : nxt;
        const Step after = ahead.k >= 0 ? step_at(sptr, ahead.e, ahead.k, s1) : Step{0, 0, -1};
        // LDS-only barriers: the rows of the steps ahead stay in flight across them
        lds_barrier();  // the previous step's tiles are consumed
        if constexpr (TR) store_item_tr<TT, MIM, NOM>(xt, gt, mine);
        else if (has_item) store_item<TT>(xt, gt, mine, my, xi_items);
        for (int it = my + DT; !TR && it < items; it += DT) {  // more items than threads (fp32): not pipelined
            const ItemGeo g2(it, xi_items, E);
            int32_t r2[E];
            Item<TT> tmp;
            load_idx<TT, IDENT>(r2, a, g2, cur);
            load_rows<TT>(tmp, r2, a, g2, ci0, co0, cur);
            store_item<TT>(xt, gt, tmp, it, xi_items);
        }
        lds_barrier();
        if constexpr (SPREAD) {
            // branch-free, so that these loads share one scheduling region
            // with the MFMAs below, which spread them among themselves (a
            // step past the end reads clamped, valid addresses and keeps
            // nothing: its rows' ok bits are clear)
            rows_of(mine, use, ahead);
            idx_of(fill, after);
        } else if (ahead.k >= 0) {
            rows_of(mine, use, ahead);
            if (after.k >= 0) idx_of(fill, after);
        }
#pragma unroll
        for (int ks = 0; ks < PS / (4 * E); ++ks) {
            const int poff = (ks * 4 + lg) * 16;
            u32x4 gf[NOM], xf[MIM];
            if constexpr (TR) {
                using G = TrGeo<MIM, NOM>;
#pragma unroll
                for (int no = 0; no < NOM; ++no) gf[no] = tr_fragment(gt, G::RSG, (wo * NOM + no) * 16, ks, lr, lg);
#pragma unroll
                for (int mi = 0; mi < MIM; ++mi) xf[mi] = tr_fragment(xt, G::RSX, (wi * MIM + mi) * 16, ks, lr, lg);
            } else {
#pragma unroll
            for (int no = 0; no < NOM; ++no)
                if (FULL || (no < NO && (wo * NO + no) * 16 < TO))
                    gf[no] = ld16(gt + ((wo * NO + no) * 16 + lr) * ROW + poff);
#pragma unroll
            for (int mi = 0; mi < MIM; ++mi)
                if (FULL || (mi < MI && (wi * MI + mi) * 16 < TI))
                    xf[mi] = ld16(xt + ((wi * MI + mi) * 16 + lr) * ROW + poff);
            }
#pragma unroll
            for (int mi = 0; mi < MIM; ++mi)
#pragma unroll
                for (int no = 0; no < NOM; ++no)
                    if (FULL || (mi < MI && no < NO && (wi * MI + mi) * 16 < TI && (wo * NO + no) * 16 < TO))
                        acc[mi][no] = mfma16<TT>(gf[no], xf[mi], acc[mi][no]);
        }
        if constexpr (SPREAD) {
            // one of the step's NV loads after every SP-th MFMA, so that a
            // wave issues its loads between MFMAs instead of stalling on the
            // load path before the first of them
            constexpr int KS = PS / (4 * E), NMB = MIM * NOM, NM = NMB * KS;
            constexpr int NV = TrGeo<MIM, NOM>::NQ * (IDENT ? 1 : 2);
            constexpr int SP = NM / NV > 1 ? NM / NV : 1;
#pragma unroll
            for (int i = 0; i < NM; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i % SP == 0 && i / SP < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
        }
        if (nxt.k != cur.k) {
            // last step of offset cur.k in this segment: D[co][ci] per 16x16
            // tile, this lane holds co = lg*4 .. +3 of ci = lr
            float* part = a.part + (int64_t(blockIdx.x) + cur.k) * a.cin * a.cout;
#pragma unroll
            for (int mi = 0; mi < MIM; ++mi)
#pragma unroll
                for (int no = 0; no < NOM; ++no) {
                    if (!FULL && !(mi < MI && no < NO && (wi * MI + mi) * 16 < TI && (wo * NO + no) * 16 < TO)) continue;
                    const int ci = ci0 + (wi * MI + mi) * 16 + lr;
                    const int co = co0 + (wo * NO + no) * 16 + lg * 4;
                    *reinterpret_cast<f32x4_t*>(part + int64_t(ci) * a.cout + co) = acc[mi][no];
                    acc[mi][no] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
        }
        cur = nxt;
        if (DEPTH == 2) {
            nxt = nx2;
            nx2 = after;
        } else {
            nxt = after;
        }
    };
    if constexpr (DEPTH == 1) {
        while (cur.k >= 0) {
            step(ra, ia, ib);
            if (cur.k < 0) break;
            step(ra, ib, ia);
        }
    } else {
        while (cur.k >= 0) {
            step(ra, ia, ib);
            if (cur.k < 0) break;
            step(rb, ib, ia);
        }
    }
}

// dw[k] = sum of offset k's partials, in segment order (zero if the offset
// has no pairs).  A block takes 256 floats of one offset; its four thread
// groups sum every fourth segment, and the groups are combined in order.
__global__ __launch_bounds__(256) void k_reduce_segs(DfArgs a, float* __restrict__ dw) {
    __shared__ f32x4_t red[4][64];
    const int k = blockIdx.y;
    const int64_t L = int64_t(a.cin) * a.cout;  // a multiple of 256
    const int q = threadIdx.x & 63, g = threadIdx.x >> 6;
    const int64_t e0 = int64_t(blockIdx.x) * 256 + q * 4;
    const int64_t P = pairs_total(a), seg = seg_len(a, P);
    const int64_t beg = off_beg(a, k), end = off_end(a, k);
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    if (end > beg && a.n_in > 0 && a.n_out > 0) {
        const int64_t bf = beg / seg, bl = (end - 1) / seg;
        constexpr int QB = 8;
        for (int64_t b0 = bf + g; b0 <= bl; b0 += 4 * QB) {
            f32x4_t v[QB];
#pragma unroll
            for (int u = 0; u < QB; ++u) {
                const int64_t b = b0 + 4 * u <= bl ? b0 + 4 * u : bl;
                v[u] = *reinterpret_cast<const f32x4_t*>(a.part + (b + k) * L + e0);
            }
#pragma unroll
            for (int u = 0; u < QB; ++u)
                if (b0 + 4 * u <= bl) acc += v[u];
        }
    }
    red[g][q] = acc;
    __syncthreads();
    if (g == 0) *reinterpret_cast<f32x4_t*>(dw + int64_t(k) * L + e0) = ((red[0][q] + red[1][q]) + red[2][q]) + red[3][q];
}

constexpr int COLSUM_BLOCKS = 256;  // dbias partials (one per block, fixed row ranges)

// part[blk][c] = sum of dy rows of block blk's range in column c (fp32).  A
// thread owns one 16-byte column chunk and a row lane; lanes step through
// the rows with batched loads, then combine in lane order through LDS, so
// the result does not depend on scheduling.
template <typename TT>
__global__ __launch_bounds__(256) void k_colsum(const typename TT::storage* __restrict__ dy, int32_t n, int32_t C,
                                                float* __restrict__ part) {
    using S = typename TT::storage;
    constexpr int E = TT::E;
    __shared__ float red[256][8];
    const int CC = C / E;                    // 16-byte chunks per row (C is a multiple of 16)
    const int64_t per = (int64_t(n) + gridDim.x - 1) / gridDim.x;
    const int64_t lo = min<int64_t>(n, per * blockIdx.x), hi = min<int64_t>(n, lo + per);
    float* outp = part + int64_t(blockIdx.x) * C;
    for (int c0 = 0; c0 < CC; c0 += 256) {   // column chunks handled by this pass
        const int nch = min(256, CC - c0);
        const int lanes = 256 / nch;         // row lanes
        const int ch = threadIdx.x % nch, lane = threadIdx.x / nch;
        float acc[E];
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = 0.f;
        if (lane < lanes) {
            constexpr int QB = 4;
            for (int64_t r0 = lo + lane; r0 < hi; r0 += int64_t(lanes) * QB) {
                u32x4 v[QB];
#pragma unroll
                for (int u = 0; u < QB; ++u) {
                    const int64_t r = r0 + int64_t(u) * lanes;
                    v[u] = ld16(dy + (r < hi ? r : lo) * C + (c0 + ch) * E);
                }
#pragma unroll
                for (int u = 0; u < QB; ++u) {
                    if (r0 + int64_t(u) * lanes >= hi) continue;
                    const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        if constexpr (TT::id == SPC_F32) {
                            acc[e] += __uint_as_float(w[e]);
                        } else {
                            const uint16_t h = uint16_t(w[e / 2] >> (16 * (e & 1)));
                            if constexpr (TT::id == SPC_BF16)
                                acc[e] += __uint_as_float(uint32_t(h) << 16);
                            else
                                acc[e] += float(__builtin_bit_cast(_Float16, h));
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int e = 0; e < E; ++e) red[threadIdx.x][e] = acc[e];
        __syncthreads();
        if (threadIdx.x < nch) {  // lane order
            float t[E];
#pragma unroll
            for (int e = 0; e < E; ++e) t[e] = 0.f;
            for (int l = 0; l < lanes; ++l)
#pragma unroll
                for (int e = 0; e < E; ++e) t[e] += red[l * nch + threadIdx.x][e];
#pragma unroll
            for (int e = 0; e < E; ++e) outp[(c0 + threadIdx.x) * E + e] = t[e];
        }
        __syncthreads();
    }
}

// out[j] = sum over s < S (in order) of part[s*L + j], batched loads.
__global__ __launch_bounds__(256) void k_reduce_parts(const float* __restrict__ part, int S, int64_t L,
                                                      float* __restrict__ out) {
    const int64_t j = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (j >= L) return;
    constexpr int QB = 8;
    float acc = 0.f;
    for (int s0 = 0; s0 < S; s0 += QB) {
        float v[QB];
#pragma unroll
        for (int u = 0; u < QB; ++u) v[u] = part[int64_t(s0 + u < S ? s0 + u : S - 1) * L + j];
#pragma unroll
        for (int u = 0; u < QB; ++u)
            if (s0 + u < S) acc += v[u];
    }
    out[j] = acc;
}

struct DfLayout {
    int64_t max_chunks;
    int64_t rparts;  // dbias partial rows
    size_t off_dbias, total;
};

// Partial slots: b + k over segments b < nseg <= MAX_WG and offsets k < K.
DfLayout df_layout(int64_t n_in, int64_t n_out, int32_t cin, int32_t cout, int32_t K, bool dbias) {
    DfLayout l;
    l.max_chunks = MAX_WG + K;
    l.rparts = dbias ? COLSUM_BLOCKS : 0;
    l.off_dbias = align_up(size_t(l.max_chunks) * cin * cout * 4, 256);
    l.total = align_up(l.off_dbias + size_t(l.rparts) * cout * 4, 256);
    return l;
}

template <typename TT>
spc_status launch_dfilter(const DfArgs& a, float* dw, float* dbias, float* bias_part, int64_t rparts,
                          hipStream_t stream) {
    const unsigned tiles = unsigned(ceil_div(a.cin, TMAX) * ceil_div(a.cout, TMAX));
    DfArgs b = a;
    b.nseg = int32_t(std::max<int64_t>(64, MAX_WG / tiles));
    // accumulator extent per wave: 2 or 4 blocks of 16 per dimension (a
    // 128-channel tile needs 4); two steps of rows in flight fit the
    // registers next to the smaller accumulators, and next to the 4 x 4 ones
    // only in the full-tile variant
    const int mim = std::min<int64_t>(a.cin, TMAX) > 64 ? 4 : 2, nom = std::min<int64_t>(a.cout, TMAX) > 64 ? 4 : 2;
    const dim3 grid(unsigned(b.nseg), tiles);
    // every tile full: 64 channels for 2 blocks per wave, multiples of 128 for 4
    const bool full = (mim == 2 ? a.cin == 64 : a.cin % TMAX == 0) && (nom == 2 ? a.cout == 64 : a.cout % TMAX == 0);
#define SPC_DFILTER_F(MIM_, NOM_, DEPTH_, FULL_)                                                                 \
    do {                                                                                                        \
        if (a.ptr)                                                                                              \
            hipLaunchKernelGGL((k_dfilter<TT, false, MIM_, NOM_, DEPTH_, FULL_>), grid, dim3(DT), 0, stream, b); \
        else                                                                                                    \
            hipLaunchKernelGGL((k_dfilter<TT, true, MIM_, NOM_, DEPTH_, FULL_>), grid, dim3(DT), 0, stream, b);  \
    } while (0)
#define SPC_DFILTER(MIM_, NOM_, DEPTH_)                                   \
    do {                                                                  \
        if (full)                                                         \
            SPC_DFILTER_F(MIM_, NOM_, DEPTH_, true);                      \
        else                                                              \
            SPC_DFILTER_F(MIM_, NOM_, DEPTH_, false);                     \
    } while (0)
    if (mim == 2 && nom == 2)
        SPC_DFILTER(2, 2, 2);
    else if (mim == 2)
        SPC_DFILTER(2, 4, 2);
    else if (nom == 2)
        SPC_DFILTER(4, 2, 2);
    else if (full)  // two steps of rows in flight fit two waves per SIMD only without the bound checks
        SPC_DFILTER_F(4, 4, 2, true);
    else if (TT::E == 8 && a.cin == 96 && a.cout == 96) {
        // 96-channel 16-bit layers: full tiles of 2 x 3 blocks, with the transposing reads
        if constexpr (TT::E == 8) SPC_DFILTER_F(3, 3, 2, true);
    }
    else
        SPC_DFILTER_F(4, 4, 1, false);
#undef SPC_DFILTER
#undef SPC_DFILTER_F
    SPC_LAUNCHED("k_dfilter");
    const int64_t L = int64_t(a.cin) * a.cout;
    hipLaunchKernelGGL(k_reduce_segs, dim3(unsigned(L / 256), unsigned(a.K)), dim3(256), 0, stream, b, dw);
    SPC_LAUNCHED("k_reduce_segs");
    if (dbias) {
        hipLaunchKernelGGL(k_colsum<TT>, dim3(unsigned(rparts)), dim3(256), 0, stream,
                           static_cast<const typename TT::storage*>(a.dy), a.n_out, a.cout, bias_part);
        SPC_LAUNCHED("k_colsum");
        hipLaunchKernelGGL(k_reduce_parts, dim3(unsigned(ceil_div(a.cout, 256))), dim3(256), 0, stream, bias_part,
                           int(rparts), int64_t(a.cout), dbias);
        SPC_LAUNCHED("k_reduce_parts");
    }
    return SPC_OK;
}

}  // namespace
}  // namespace spc

using namespace spc;

extern "C" spc_status spc_conv_bwd_filter_workspace(int64_t n_in, int64_t n_out, int32_t cin, int32_t cout,
                                                    int32_t K, int32_t want_dbias, size_t* bytes) {
    clear_error();
    if (!bytes) return fail(SPC_ERR_ARG, "bytes is NULL");
    if (n_in < 0 || n_out < 0 || cin <= 0 || cout <= 0 || K <= 0) return fail(SPC_ERR_ARG, "invalid sizes");
    *bytes = df_layout(n_in, n_out, cin, cout, K, want_dbias != 0).total;
    return SPC_OK;
}

// Scratch of spc_conv_bwd_filter_noalloc: one static array per GPU, held
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: kernels get the device address that hipGetSymbolAddress
// returns for the current device (dfilter_scratch), never the array's name.
static __device__ __align__(256) char scratch[SPC_DFILTER_SCRATCH_BYTES];

namespace spc {
namespace {

std::mutex scratch_mu;
void* scratch_ptr[64];  // per device, guarded by scratch_mu

// The device address of `scratch` on the current device, looked up on the
// first call on that device.
spc_status dfilter_scratch(void** out) {
    int dev = 0;
    SPC_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= 64) return fail(SPC_ERR_UNSUPPORTED, "device %d", dev);
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        SPC_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p || !aligned16(p)) return fail(SPC_ERR_HIP, "scratch symbol address %p", p);
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return SPC_OK;
}

// Checks of spc_conv_bwd_filter's arguments other than the workspace; the
// workspace layout on success.
spc_status dfilter_checks(spc_dtype dtype, const void* feats, int64_t n_in, int32_t cin, const void* dout,
                          int64_t n_out, int32_t cout, int32_t K, const int32_t* pair_ptr, const int32_t* pair_in,
                          const int32_t* pair_out, const float* dw, const float* dbias, DfLayout& l) {
    if (dtype != SPC_F32 && dtype != SPC_F16 && dtype != SPC_BF16) return fail(SPC_ERR_ARG, "unknown dtype %d", int(dtype));
    if (n_in < 0 || n_out < 0 || n_in >= (int64_t(1) << 31) || n_out >= (int64_t(1) << 31))
        return fail(SPC_ERR_ARG, "row counts out of range");
    if (cin <= 0 || cout <= 0 || cin % 16 || cout % 16)
        return fail(SPC_ERR_UNSUPPORTED, "cin=%d cout=%d: channel counts must be positive multiples of 16", cin, cout);
    if (K <= 0 || K > 343) return fail(SPC_ERR_ARG, "K=%d must be in 1..343", K);
    const bool identity = !pair_ptr && !pair_in && !pair_out;
    if (identity && (K != 1 || n_in != n_out))
        return fail(SPC_ERR_ARG, "pair lists are required unless K == 1 and n_in == n_out");
    if (!identity && !(pair_ptr && pair_in && pair_out)) return fail(SPC_ERR_ARG, "pair_ptr/pair_in/pair_out must be all set or all NULL");
    if (!dw) return fail(SPC_ERR_ARG, "dw is NULL");
    if ((n_in > 0 && !feats) || (n_out > 0 && !dout)) return fail(SPC_ERR_ARG, "feats or dout is NULL");
    const void* ptrs[] = {feats, dout, pair_ptr, pair_in, pair_out, dw, dbias};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(SPC_ERR_ARG, "device pointers must be 16-byte aligned");
    l = df_layout(n_in, n_out, cin, cout, K, dbias != nullptr);
    return SPC_OK;
}

spc_status dfilter_run(spc_dtype dtype, const void* feats, int64_t n_in, int32_t cin, const void* dout,
                       int64_t n_out, int32_t cout, int32_t K, const int32_t* pair_ptr, const int32_t* pair_in,
                       const int32_t* pair_out, float* dw, float* dbias, void* ws, const DfLayout& l,
                       hipStream_t stream) {
    DfArgs a{feats, dout, pair_ptr, pair_in, pair_out, static_cast<float*>(ws), int32_t(n_in), int32_t(n_out),
             cin, cout, K, 0};
    float* bias_part = reinterpret_cast<float*>(static_cast<char*>(ws) + l.off_dbias);
    switch (dtype) {
        case SPC_F32: return launch_dfilter<F32>(a, dw, dbias, bias_part, l.rparts, stream);
        case SPC_F16: return launch_dfilter<F16>(a, dw, dbias, bias_part, l.rparts, stream);
        case SPC_BF16: return launch_dfilter<BF16>(a, dw, dbias, bias_part, l.rparts, stream);
    }
    return fail(SPC_ERR_ARG, "unknown dtype %d", int(dtype));
}

}  // namespace
}  // namespace spc

extern "C" spc_status spc_conv_bwd_filter(spc_dtype dtype, const void* feats, int64_t n_in, int32_t cin,
                                          const void* dout, int64_t n_out, int32_t cout, int32_t K,
                                          const int32_t* pair_ptr, const int32_t* pair_in, const int32_t* pair_out,
                                          float* dw, float* dbias, void* ws, size_t ws_bytes, hipStream_t stream) {
    clear_error();
    DfLayout l;
    spc_status st = dfilter_checks(dtype, feats, n_in, cin, dout, n_out, cout, K, pair_ptr, pair_in, pair_out, dw,
                                   dbias, l);
    if (st != SPC_OK) return st;
    if (!ws) return fail(SPC_ERR_ARG, "workspace is NULL");
    if (!aligned16(ws)) return fail(SPC_ERR_ARG, "device pointers must be 16-byte aligned");
    if (ws_bytes < l.total) return fail(SPC_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, l.total);
    return dfilter_run(dtype, feats, n_in, cin, dout, n_out, cout, K, pair_ptr, pair_in, pair_out, dw, dbias, ws, l,
                       stream);
}

extern "C" spc_status spc_conv_bwd_filter_noalloc(spc_dtype dtype, const void* feats, int64_t n_in, int32_t cin,
                                                  const void* dout, int64_t n_out, int32_t cout, int32_t K,
                                                  const int32_t* pair_ptr, const int32_t* pair_in,
                                                  const int32_t* pair_out, float* dw, float* dbias,
                                                  hipStream_t stream) {
    clear_error();
    DfLayout l;
    spc_status st = dfilter_checks(dtype, feats, n_in, cin, dout, n_out, cout, K, pair_ptr, pair_in, pair_out, dw,
                                   dbias, l);
    if (st != SPC_OK) return st;
    if (l.total > SPC_DFILTER_SCRATCH_BYTES)
        return fail(SPC_ERR_UNSUPPORTED,
                    "cin=%d cout=%d K=%d needs %zu bytes of scratch; the allocation-free call holds %zu "
                    "(use spc_conv_bwd_filter with a workspace)",
                    cin, cout, K, l.total, size_t(SPC_DFILTER_SCRATCH_BYTES));
    void* ws = nullptr;
    if ((st = dfilter_scratch(&ws)) != SPC_OK) return st;
    return dfilter_run(dtype, feats, n_in, cin, dout, n_out, cout, K, pair_ptr, pair_in, pair_out, dw, dbias, ws, l,
                       stream);
}
