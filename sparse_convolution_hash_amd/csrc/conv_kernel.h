// Fused implicit-GEMM sparse convolution: gather -> MFMA -> output-stationary
// accumulate, one kernel per call.
//
//   y[r, :] = bias + sum_k  x[map[k][r], :] @ B_k          (map[k][r] >= 0)
//
// covers the submanifold and strided forward (B_k = W[k], the MLX
// sparse/conv.py page's formula), the per-voxel k=1 layer (identity map) and
// dinput (B_k = W[k]^T or W[K-1-k]^T, gathered from dout through the
// input-stationary map).  Absent neighbours contribute nothing, like the MLX
// page's appended zero row, but here a missing row is a predicated-off load
// that leaves a zero fragment.
//
// Work split (CDNA4, 64-lane waves): a workgroup of 4 waves owns BM = 4*RB*16
// output rows and BN = NB*16 output channels.  For each offset that has at
// least one hit among its rows it stages B_k's [CK x BN] slab in LDS (in the
// 16-byte MFMA fragment layout, transposing W on the fly when needed), and
// every wave multiplies its gathered rows, loaded straight from global memory
// into registers as 16-byte fragments, with v_mfma_f32_16x16x32_{bf16,f16}
// (or v_mfma_f32_16x16x4_f32).  The fp32 accumulators stay in registers for
// the whole offset loop; each output row is written once, with the bias added
// and one rounding, so there are no atomics and the result is deterministic.
// The identity map of a k = 1 layer has one offset and equal tiles: there a
// workgroup stages its slab once and walks several tiles (PERSIST).
//
// This header holds the kernel and its launchers; the per-dtype translation
// units conv_f32.hip, conv_f16.hip and conv_bf16.hip instantiate them (one
// each, so that the many variants compile in parallel), and conv.hip holds
// the C entry points.
#pragma once

#include <algorithm>
#include <type_traits>

#include "common.h"

namespace spc {

struct ConvArgs {
    const void* x;       // gathered operand [n_src, CK]
    const void* w;       // weights [K, cin, cout]
    const float* bias;   // [CN] or NULL
    const int32_t* map;  // [n_rows, K] row-major, or NULL (identity, K == 1)
    const int32_t* order;  // processing order of the rows, or NULL (natural order)
    void* y;             // [n_rows, CN]
    int32_t n_rows, n_src, K;
    int32_t CK, CN;      // contraction / output channels
    int32_t cin, cout;   // weight dims
    int32_t w_rev;       // slab of offset k is W[K-1-k]
    int32_t kch;         // 16-byte chunks along CK, padded to a multiple of 4
    const void* res;     // residual [n_rows, CN] added before the activation, or NULL (may alias y)
    int32_t relu;        // ReLU on the final fp32 value
    int32_t xbuf;        // x and the weights lie within 2 GiB (buffer loads can address them)
    const int32_t* n_rows_dev;  // live row count in device memory (n_rows is then the capacity), or NULL
};

// Launch of the convolution for one storage type: trans selects the forward's
// weight staging (B_k = W[k], weights [K, CK, CN]) over dinput's (B_k =
// W[k]^T, weights [K, CN, CK], contraction-contiguous).
spc_status run_conv_f32(ConvArgs& a, bool trans, hipStream_t stream);
spc_status run_conv_f16(ConvArgs& a, bool trans, hipStream_t stream);
spc_status run_conv_bf16(ConvArgs& a, bool trans, hipStream_t stream);

#ifdef SPC_CONV_KERNELS
namespace {

constexpr int CT = 256;          // threads per workgroup
constexpr int NW = CT / WAVE;    // waves per workgroup
// s_waitcnt vmcnt(0) with expcnt / lgkmcnt left at their maxima (gfx9 encoding)
constexpr int WAIT_VMCNT0 = 0x0F70;
constexpr int KTILE = 28;        // offsets whose map rows are staged at once (a 3x3x3 kernel in one go)
// weight fragments read ahead of their MFMAs in the 16-bit step loops
constexpr int BLOOK = 4;

// Buffer loads (CDNA buffer addressing): a 16-byte load through a buffer
// resource whose offset lies past the resource's range returns zeros without
// a memory access, so a masked lane costs nothing and needs no branch.
constexpr int BUF_FLAGS = 0x00020000;        // raw buffer, 32-bit elements (gfx9 family)
constexpr uint32_t BUF_OOB = 0x80000000u;    // past any range below 2 GiB

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, int(bytes), BUF_FLAGS);
}

__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 0));
}




// LDS slab layout: chunk row kb (16 bytes of CK per output channel) has BN
// entries of 16 bytes plus 16 bytes of padding, which keeps both the staging
// writes and the fragment reads free of bank conflicts.
template <int BN>
__device__ __forceinline__ int slab_off(int kb, int n) {
    return kb * (BN * 16 + 16) + n * 16;
}

// The 16-bit forward keeps W's own layout in LDS instead: row kk holds the
// BN output channels of contraction index kk (2 bytes each) plus 32 bytes of
// padding, and the MFMA fragments are read with gfx950's transposing LDS
// reads (ds_read_b64_tr_b16).  Within each 16-lane group, lane j points at 4
// consecutive 16-bit values M[j][0..3]; lane i receives M[4q + (i >> 2)][i & 3]
// for q = 0..3.  So when lane j points at row k0 + (j >> 2), channels
// n0 + 4 (j & 3) .. +3, lane i receives channel n0 + i at k0 .. k0 + 3: half
// of its 8-value fragment, the second read (rows k0 + 4 ..) the other half.
// Staging is then plain 16-byte copies of W rows, with no transposes.  It
// pays for contractions of up to 64 channels (2 MFMA steps), where staging
// dominates an offset's work (LiDAR SubM forward 34.4 -> 30.5 us); longer
// contractions are bound by their LDS reads, and two 8-byte transposing reads
// per fragment instead of one 16-byte read made them slower (shell-set SubM
// forward 281 -> 312 us), so they keep the transposed layout.
template <int BN>
constexpr int row_stride() { return BN * 2 + 32; }

template <typename TT, bool TRANS, int KCMAX>
constexpr bool rows_layout() { return TRANS && TT::E == 8 && KCMAX <= 2; }

// Bytes of one weight slab in LDS for a contraction of kch 16-byte chunks.
template <int BN, bool ROWS>
__host__ __device__ constexpr int slab_bytes_of(int kch) {
    return ROWS ? kch * 8 * row_stride<BN>() : kch * (BN * 16 + 16);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ s16x4 ds_read_tr16(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// Weight slab staging.  TRANS: B[kk][n] = W[ws][kk][n] (the forward; W rows
// are output channels apart: 16-bit rows are copied as they are (ROWS, see
// row_stride), fp32 ones in E x E blocks transposed in registers).
// !TRANS: B[kk][n] = W[ws][n][kk] (dinput; already contraction-contiguous).
// Chunks beyond CK are zero.  A thread holds up to WREG 16-byte registers of
// the slab so the next offset's slab can be in flight during the MFMAs; any
// rest of a large slab is copied when it is stored.
constexpr int WREG = 8;

template <typename TT, int BN, bool TRANS, bool ROWS>
struct WStage {
    using S = typename TT::storage;
    static constexpr int E = TT::E;
    // one item: an E x E block (fp32 TRANS) or one 16-byte chunk
    static constexpr int ITEM_REGS = (TRANS && !ROWS) ? E : 1;
    static constexpr int PRE = WREG / ITEM_REGS;  // items prefetched per thread
    u32x4 r[WREG];
    // the thread's first item (idx = threadIdx.x) as chunk row kb0 and channel
    // (or channel block) q0; item p is idx + p * CT, stepped from the first
    // without a division: (kb, q) advances by (dr, dq) = (CT % kch, CT / kch)
    // with a carry.  Nothing per item stays in registers across the offsets.
    int32_t kb0, q0, dq, dr, col0;

    __device__ static int items(const ConvArgs& a) { return (TRANS && !ROWS) ? a.kch * (BN / E) : a.kch * BN; }

    // element offset inside a weight slab (-1: zero padding) and LDS byte
    // offset of item (kb, q), or of item idx in the row layout
    __device__ static void place(const ConvArgs& a, int col0, int idx, int kb, int q, int32_t& g, int32_t& l) {
        if (ROWS) {  // consecutive items along a row of W: coalesced reads, consecutive LDS writes
            constexpr int CPR = BN / 8;  // 16-byte chunks per row
            const int kk = idx / CPR, c = idx - kk * CPR;
            g = kk < a.CK ? kk * a.cout + col0 + c * 8 : -1;
            l = kk * row_stride<BN>() + c * 16;
            return;
        }
        const bool real = kb < a.CK / E;  // q: channel block (TRANS) or channel
        if (TRANS) {
            g = real ? kb * E * a.cout + col0 + q * E : -1;
            l = slab_off<BN>(kb, q * E);
        } else {
            g = real ? (col0 + q) * a.cout + kb * E : -1;
            l = slab_off<BN>(kb, q);
        }
    }

    __device__ void init(const ConvArgs& a, int c0) {
        col0 = c0;
        dq = CT / a.kch;
        dr = CT - dq * a.kch;
        kb0 = int(threadIdx.x) % a.kch;
        q0 = int(threadIdx.x) / a.kch;
    }

    // f(p, g, l) for each prefetched item p of this thread (l = -1: no item)
    template <typename F>
    __device__ void each(const ConvArgs& a, F&& f) const {
        const int n = items(a);
        int kb = kb0, q = q0;
#pragma unroll
        for (int p = 0; p < PRE; ++p) {
            const int idx = int(threadIdx.x) + p * CT;
            int32_t g, l;
            place(a, col0, idx, kb, q, g, l);
            if (idx >= n) g = l = -1;
            f(p, g, l);
            kb += dr;
            q += dq;
            if (kb >= a.kch) kb -= a.kch, ++q;
        }
    }

    __device__ static void load_at(u32x4* dst, const S* w, int32_t g, int cout) {
        if (TRANS && !ROWS) {
#pragma unroll
            for (int e = 0; e < E; ++e) dst[e] = g >= 0 ? ld16(w + g + int64_t(e) * cout) : zero4();
        } else {
            dst[0] = g >= 0 ? ld16(w + g) : zero4();
        }
    }

    __device__ static void store_at(char* lds, const u32x4* in, int32_t l) {
        if (TRANS && !ROWS) {
            if constexpr (E == 8) {
                typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
                u16x8 v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = __builtin_bit_cast(u16x8, in[e]);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    u16x8 o = {v[0][j], v[1][j], v[2][j], v[3][j], v[4][j], v[5][j], v[6][j], v[7][j]};
                    st16(lds + l + j * 16, __builtin_bit_cast(u32x4, o));
                }
            } else {
                const uint32_t m[4][4] = {{in[0].x, in[0].y, in[0].z, in[0].w},
                                          {in[1].x, in[1].y, in[1].z, in[1].w},
                                          {in[2].x, in[2].y, in[2].z, in[2].w},
                                          {in[3].x, in[3].y, in[3].z, in[3].w}};
#pragma unroll
                for (int j = 0; j < 4; ++j) st16(lds + l + j * 16, u32x4{m[0][j], m[1][j], m[2][j], m[3][j]});
            }
        } else {
            st16(lds + l, in[0]);
        }
    }

    __device__ void load(const ConvArgs& a, int ws) {
        const S* w = static_cast<const S*>(a.w) + int64_t(ws) * a.cin * a.cout;
        each(a, [&](int p, int32_t g, int32_t l) {
            if (l >= 0) load_at(r + p * ITEM_REGS, w, g, a.cout);
        });
    }

    // The same through the weights' buffer resource, without branches:
    // padding and absent items, and every item when !live, take an
    // out-of-range offset and load zeros without a memory access.
    __device__ void load_buf(const ConvArgs& a, __amdgpu_buffer_rsrc_t wr, int ws, bool live) {
        const uint32_t base = uint32_t(ws) * uint32_t(a.cin) * uint32_t(a.cout);
        each(a, [&](int p, int32_t g, int32_t) {
#pragma unroll
            for (int e = 0; e < ITEM_REGS; ++e) {
                const uint32_t off =
                    live && g >= 0 ? (base + uint32_t(g + e * a.cout)) * uint32_t(sizeof(S)) : BUF_OOB;
                r[p * ITEM_REGS + e] = buf_ld16(wr, off);
            }
        });
    }

    // load_buf for a variant whose contraction is exactly KCH chunks (a.kch
    // == KCH) and whose items are single chunks: item p of this thread is idx
    // = threadIdx.x + p * CT, as in each(), but its place comes from
    // compile-time divisors, so the loads carry no branches and can share a
    // scheduling region with the MFMAs
    template <int KCH, int NP>
    __device__ void load_exact(const ConvArgs& a, __amdgpu_buffer_rsrc_t wr, int ws, bool live) {
        static_assert(ITEM_REGS == 1, "chunk items only");
        constexpr int N = KCH * BN;
        const uint32_t base = uint32_t(ws) * uint32_t(a.cin) * uint32_t(a.cout);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int idx = int(threadIdx.x) + p * CT;
            int32_t g;
            if constexpr (ROWS) {
                constexpr int CPR = BN / 8;
                const int kk = idx / CPR, c = idx - kk * CPR;
                g = kk < a.CK ? kk * a.cout + col0 + c * 8 : -1;
            } else {
                const int kb = idx % KCH, q = idx / KCH;
                g = kb < a.CK / E ? (col0 + q) * a.cout + kb * E : -1;
            }
            const bool ok = live && idx < N && g >= 0;
            r[p] = buf_ld16(wr, ok ? (base + uint32_t(g)) * uint32_t(sizeof(S)) : BUF_OOB);
        }
    }

    __device__ void store(char* lds, const ConvArgs& a, int ws) const {
        each(a, [&](int p, int32_t, int32_t l) {
            if (l >= 0) store_at(lds, r + p * ITEM_REGS, l);
        });
        const int n = items(a);
        if (threadIdx.x + PRE * CT >= n) return;
        const S* w = static_cast<const S*>(a.w) + int64_t(ws) * a.cin * a.cout;
        for (int idx = threadIdx.x + PRE * CT; idx < n; idx += CT) {  // rest of a large slab
            int32_t g, l;
            place(a, col0, idx, idx % a.kch, idx / a.kch, g, l);
            u32x4 t[ITEM_REGS];
            load_at(t, w, g, a.cout);
            store_at(lds, t, l);
        }
    }
};

template <typename TT, int RB, int KCMAX>
__device__ __forceinline__ bool gather_rows(u32x4 (&af)[RB][KCMAX], const ConvArgs& a, const int32_t* tile_k,
                                            int wave, int lr, int lg) {
    using S = typename TT::storage;
    constexpr int E = TT::E;
    const S* x = static_cast<const S*>(a.x);
    const int KC = a.kch / 4;
    bool any = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int32_t src = tile_k[(wave * RB + rb) * 16 + lr];
        any |= src >= 0;
        const S* p = x + int64_t(src) * a.CK + lg * E;
#pragma unroll
        for (int kc = 0; kc < KCMAX; ++kc) {
            af[rb][kc] = zero4();
            if (kc < KC && src >= 0 && (kc * 4 + lg) * E < a.CK) af[rb][kc] = ld16(p + kc * 4 * E);
        }
    }
    return __any(any);
}

// gather_rows through x's buffer resource, without branches: a missing row
// or a chunk past the contraction (every row when !live) takes an
// out-of-range offset and loads zeros without a memory access.
template <typename TT, int RB, int KCMAX>
__device__ __forceinline__ bool gather_buf(u32x4 (&af)[RB][KCMAX], const ConvArgs& a, __amdgpu_buffer_rsrc_t xr,
                                           const int32_t* tile_k, bool live, int wave, int lr, int lg) {
    using S = typename TT::storage;
    constexpr int E = TT::E;
    const uint32_t row_bytes = uint32_t(a.CK) * uint32_t(sizeof(S));
    bool any = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int32_t v = tile_k[(wave * RB + rb) * 16 + lr];  // a valid LDS address either way
        const int32_t src = live ? v : -1;
        any |= src >= 0;
#pragma unroll
        for (int kc = 0; kc < KCMAX; ++kc) {
            const int col = (kc * 4 + lg) * E;
            const bool ok = src >= 0 && col < a.CK;
            af[rb][kc] = buf_ld16(xr, ok ? uint32_t(src) * row_bytes + uint32_t(col) * uint32_t(sizeof(S)) : BUF_OOB);
        }
    }
    return __any(any);
}

// gather_buf with this lane's source rows in registers (src[rb] for its MFMA
// row rb, or -1), as the persistent identity-map walk keeps them.
template <typename TT, int RB, int KCMAX>
__device__ __forceinline__ void gather_src(u32x4 (&af)[RB][KCMAX], const ConvArgs& a, __amdgpu_buffer_rsrc_t xr,
                                           const int32_t (&src)[RB], int lg) {
    using S = typename TT::storage;
    constexpr int E = TT::E;
    const uint32_t row_bytes = uint32_t(a.CK) * uint32_t(sizeof(S));
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int kc = 0; kc < KCMAX; ++kc) {
            const int col = (kc * 4 + lg) * E;
            const bool ok = src[rb] >= 0 && col < a.CK;
            af[rb][kc] = buf_ld16(xr, ok ? uint32_t(src[rb]) * row_bytes + uint32_t(col) * uint32_t(sizeof(S)) : BUF_OOB);
        }
}

// PERSIST (the identity map of a k = 1 layer only, launched by launch_conv_nb
// with a grid of at most two workgroups per CU): the weight slab is staged
// once per workgroup, which then walks tiles blockIdx.x, + gridDim.x, ...
// with the next tile's source rows and gathers in flight behind the current
// tile's MFMAs and epilogue.  Every tile of an identity map costs the same,
// so the fixed stride stays balanced.
template <typename TT, int RB, int NB, bool TRANS, int KCMAX, bool PIPE, bool PERSIST = false>
__global__ __launch_bounds__(CT) void k_conv(ConvArgs a) {
    using S = typename TT::storage;
    constexpr int BN = NB * 16;
    constexpr int BM = NW * RB * 16;
    // row stride of the LDS map tile: an odd stride spreads the writes of
    // consecutive offsets of one row over consecutive banks
    constexpr int BMP = BM + 1;
    static_assert(KTILE % 4 == 0, "the tile keeps the following arrays 16-byte aligned");
    extern __shared__ __attribute__((aligned(16))) char lds[];
    // the two slab buffers are addressed arithmetically from the __shared__
    // base (a pointer table would hide the address space and turn the LDS
    // reads into flat loads that wait on the global prefetches)
    constexpr bool ROWS = rows_layout<TT, TRANS, KCMAX>();
    const int slab_bytes = slab_bytes_of<BN, ROWS>(a.kch);
    int32_t* tile = reinterpret_cast<int32_t*>(lds + 2 * slab_bytes);  // [KTILE][BMP]
    int32_t* flags = tile + KTILE * BMP;                               // [KTILE]
    int32_t* list = flags + KTILE;                                     // [KTILE + 4] (count at KTILE; keeps 16-B alignment)
    // the epilogue stages the tile's outputs over the slabs and the map tile
    constexpr int SROW = BN * int(sizeof(S)) + 16;  // staged output row (16 bytes of padding)
    const int main_bytes = 2 * slab_bytes + (KTILE * BMP + 2 * KTILE + 4) * 4;
    const int rsrc_off = PERSIST ? slab_bytes + BM * SROW : (main_bytes > BM * SROW ? main_bytes : BM * SROW);
    int32_t* rsrc = reinterpret_cast<int32_t*>(lds + rsrc_off);  // [BM]
    float* sbias = reinterpret_cast<float*>(rsrc + BM);                // [BN] bias of this column block, or 0

    const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
    const int lr = lane & 15, lg = lane >> 4;
    // tiles run last-first: in a processing order sorted by neighbour mask
    // the tiles with the most offsets come last, and starting them first
    // keeps them off the end of the launch
    const int col0 = blockIdx.y * BN;
    // rows whose count is in device memory (a strided map built without a
    // host wait): the grid covers the capacity a.n_rows; the first blocks
    // take the live tiles (last-first, as below) and the rest leave at once,
    // after them; a count above the capacity (a map that overflowed and holds
    // no rows) reads as 0
    int n_rows = a.n_rows, tiles = int(gridDim.x);
    if (a.n_rows_dev) {
        const int m = *a.n_rows_dev;
        n_rows = m >= 0 && m <= a.n_rows ? m : 0;
        tiles = (n_rows + BM - 1) / BM;
        if (int(blockIdx.x) >= tiles) return;  // uniform per workgroup, before any barrier
    }
    const int row0 = (tiles - 1 - int(blockIdx.x)) * BM;
    // MFMA steps along CK: the exact variants (KCMAX <= 4) are launched for
    // KC == KCMAX only, so their step loops carry no run-time bound (a branch
    // there would split the loop into one scheduling region per step)
    const int KC = KCMAX <= 4 ? KCMAX : a.kch / 4;

    // the bias (or zeros) into LDS now, so the epilogue reads no global memory
    if (threadIdx.x < BN) sbias[threadIdx.x] = a.bias ? a.bias[col0 + threadIdx.x] : 0.f;

    // the processing order of this tile's rows into LDS: rsrc[r] is the
    // source row of tile row r, or -1
    if (!PERSIST && threadIdx.x < BM) {
        const int row = row0 + threadIdx.x;
        const int rc = row < n_rows ? row : n_rows - 1;
        const int32_t s0 = a.order ? a.order[rc] : rc;
        rsrc[threadIdx.x] = row < n_rows && (unsigned)s0 < (unsigned)n_rows ? s0 : -1;
    }

    f32x4_t acc[RB][NB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[rb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // epilogue: D[channel][row] per 16x16 tile; this lane holds channels
    // lg*4 .. lg*4+3 of row lr.  Bias, then the residual and the ReLU of a
    // fused layer, go on the fp32 value before its one rounding (a residual
    // aliasing y is read here, before any write of this tile).  The rounded
    // values are staged in LDS at `stage` (over the slabs and the map tile,
    // free after the last offset's barrier; after the slab in the persistent
    // walk, which keeps it) and written out as whole 16-byte chunks of each
    // row, consecutive threads on consecutive chunks: a quarter of the write
    // requests of per-lane 8-byte stores.
    S* y = static_cast<S*>(a.y);
    const S* res = static_cast<const S*>(a.res);
    auto epilogue = [&](char* stage) {
        f32x4_t bv[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) bv[nb] = *reinterpret_cast<const f32x4_t*>(sbias + nb * 16 + lg * 4);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int r = (wave * RB + rb) * 16 + lr;
            const int row = rsrc[r];
            f32x4_t v[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) v[nb] = acc[rb][nb] + bv[nb];
            if (res && row >= 0) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) v[nb] += load4<TT>(res + int64_t(row) * a.CN + col0 + nb * 16 + lg * 4);
            }
            if (a.relu) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[nb][e] = v[nb][e] < 0.f ? 0.f : v[nb][e];  // NaN stays NaN
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                store4<TT>(stage + r * SROW + (nb * 16 + lg * 4) * int(sizeof(S)), v[nb]);
        }
        if constexpr (PERSIST)
            lds_barrier();  // the next tile's gathers stay in flight
        else
            __syncthreads();
        constexpr int CPR = BN * int(sizeof(S)) / 16;  // 16-byte chunks per staged row
        static_assert((BM * CPR) % CT == 0, "whole passes over the staged tile");
#pragma unroll
        for (int q = 0; q < BM * CPR / CT; ++q) {
            const int idx = q * CT + int(threadIdx.x);
            const int r = idx / CPR, c = idx - r * CPR;
            const int row = rsrc[r];
            if (row >= 0) st16(y + int64_t(row) * a.CN + col0 + c * (16 / int(sizeof(S))), ld16(stage + r * SROW + c * 16));
        }
    };

    WStage<TT, BN, TRANS, ROWS> wst;
    wst.init(a, col0);
    // slab items a thread loads per offset through load_exact: fewer than the
    // register budget PRE when an exact variant's slab is small (chunk items)
    using WS = WStage<TT, BN, TRANS, ROWS>;
    constexpr int NPRE = WS::ITEM_REGS == 1 && KCMAX <= 4
                             ? (KCMAX * 4 * BN + CT - 1) / CT < WS::PRE ? (KCMAX * 4 * BN + CT - 1) / CT : WS::PRE
                             : WS::PRE;
    u32x4 acur[RB][KCMAX], anext[RB][KCMAX];
    // the identity map (K = 1) has one offset, whose entries are the rows
    // themselves: its column is rsrc, and nothing is staged
    int32_t* const cols = a.map ? tile : rsrc;
    // one offset's MFMAs: gathered rows `cur` against slab buffer j & 1
    // nv: the number of global loads issued just before this call in the
    // same scheduling region, which the 16-bit pattern below spreads among
    // the MFMAs (0: none)
    auto mma = [&](const u32x4 (&cur)[RB][KCMAX], int j, auto nv) {
        constexpr int NV = decltype(nv)::value;
        const char* sl = lds + (j & 1) * slab_bytes;
        if constexpr (!ROWS && TT::E == 8 && KCMAX <= 4) {
            // B fragments in (kc, nb) order, each read BLOOK fragments
            // ahead of its MFMAs, so that several LDS reads are in flight
            // behind the MFMAs instead of one pair at a time.  Reads past
            // the contraction re-read its last chunk row (valid data; the
            // loop ends before those fragments are used).
            constexpr int NI = KCMAX * NB;
            constexpr int LA = (KCMAX <= 2 ? 3 : BLOOK) < NI ? (KCMAX <= 2 ? 3 : BLOOK) : NI;
            auto rd = [&](int i) {
                const int kc = min(i / NB, KC - 1), nb = i % NB;
                return ld16(sl + slab_off<BN>(kc * 4 + lg, nb * 16 + lr));
            };
            u32x4 bq[LA];
#pragma unroll
            for (int i = 0; i < LA; ++i) bq[i] = rd(i);
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int kc = i / NB, nb = i % NB;
                if (kc >= KC) break;
                const u32x4 b = bq[i % LA];
                if (i + LA < NI) bq[i % LA] = rd(i + LA);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) acc[rb][nb] = mfma16<TT>(b, cur[rb][kc], acc[rb][nb]);
            }
            {
                // keep that order through the scheduler, which otherwise
                // pairs each two reads with their MFMAs to save registers:
                // LA reads, then (RB MFMAs, one read) per fragment.  With
                // NV loads in the region (the next offsets' slab and
                // gathers), one load follows every SP-th fragment's MFMAs:
                // a wave then issues its loads between its MFMAs instead
                // of stalling on the load path before the first of them
                // (the gathers' RB source-row reads go first)
                constexpr int SP = NV > 0 && NI / NV > 1 ? NI / NV : 1;
                __builtin_amdgcn_sched_group_barrier(0x100, NV > 0 ? LA + RB : LA, 0);
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, RB, 0);
                    if (i + LA < NI) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    if (NV > 0 && i % SP == 0 && i / SP < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
            }
            return;
        }
#pragma unroll
        for (int kc = 0; kc < KCMAX; ++kc) {
            if (kc >= KC) break;
            u32x4 bf[NB];
            if constexpr (ROWS) {  // transposing reads of the row layout
                const char* p0 = sl + ((kc * 4 + lg) * 8 + (lr >> 2)) * row_stride<BN>() + 4 * (lr & 3) * 2;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const s16x4 lo = ds_read_tr16(p0 + nb * 32), hi = ds_read_tr16(p0 + nb * 32 + 4 * row_stride<BN>());
                    const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
                    bf[nb] = u32x4{l2.x, l2.y, h2.x, h2.y};
                }
            } else {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) bf[nb] = ld16(sl + slab_off<BN>(kc * 4 + lg, nb * 16 + lr));
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) acc[rb][nb] = mfma16<TT>(bf[nb], cur[rb][kc], acc[rb][nb]);
        }
    };
    if constexpr (PERSIST) {
        // the identity map's walk: tile t holds rows t*BM .. t*BM + BM-1 of the
        // processing order, each its own source; this workgroup takes tiles
        // blockIdx.x + i*G
        const int tiles_all = int((int64_t(a.n_rows) + BM - 1) / BM);
        const int G = int(gridDim.x);
        const __amdgpu_buffer_rsrc_t xr = buf_rsrc(a.x, uint32_t(a.n_src) * uint32_t(a.CK) * uint32_t(sizeof(S)));
        // this lane's source row for its MFMA row rb of tile t, or -1 (rows
        // past the end and tiles past the last read a clamped, valid row)
        auto src_of = [&](int t, int32_t (&src)[RB]) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int64_t row = int64_t(t) * BM + (wave * RB + rb) * 16 + lr;
                const int rc = row < a.n_rows ? int(row) : a.n_rows - 1;
                const int32_t s0 = a.order ? a.order[rc] : rc;
                src[rb] = row < a.n_rows && (unsigned)s0 < (unsigned)a.n_rows ? s0 : -1;
            }
        };
        wst.load(a, 0);
        wst.store(lds, a, 0);
        u32x4 ga[RB][KCMAX], gb[RB][KCMAX];
        int32_t sa[RB], sb[RB];
        int t = int(blockIdx.x);
        src_of(t, sa);
        gather_src<TT, RB, KCMAX>(ga, a, xr, sa, lg);
        src_of(t + G, sb);
        lds_barrier();  // the slab and the bias are in place
        constexpr int NVP = !ROWS && TT::E == 8 && KCMAX <= 4 ? RB * KCMAX : 0;
        // one tile: the gathers of tile tt + G (their sources were read a tile
        // ago) and the sources of tile tt + 2G go out first, then tile tt's
        // MFMAs and epilogue; the buffers keep fixed roles in a loop unrolled
        // by two (a copy would wait for its loads)
        auto tile_step = [&](int tt, const u32x4 (&cur)[RB][KCMAX], int32_t (&scur)[RB], u32x4 (&nxt)[RB][KCMAX],
                             const int32_t (&snxt)[RB]) {
            gather_src<TT, RB, KCMAX>(nxt, a, xr, snxt, lg);
            if (lg == 0) {  // the epilogue's row list; every wave writes its own rows
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) rsrc[(wave * RB + rb) * 16 + lr] = scur[rb];
            }
            src_of(tt + 2 * G, scur);
            mma(cur, 0, std::integral_constant<int, NVP>{});
            epilogue(lds + slab_bytes);
            lds_barrier();  // every wave is done with the staged tile and the row list
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) acc[rb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        };
        for (; t < tiles_all; t += 2 * G) {
            tile_step(t, ga, sa, gb, sb);
            if (t + G >= tiles_all) break;
            tile_step(t + G, gb, sb, ga, sa);
        }
        return;
    }
    for (int kt0 = 0; kt0 < a.K; kt0 += KTILE) {
        const int kt = min(KTILE, a.K - kt0);
        if (!a.map) {
            if (threadIdx.x == 0) list[0] = 0, list[KTILE] = 1;
            __syncthreads();  // rsrc, the bias and the list are in place
        } else {
        __syncthreads();  // earlier readers of tile / list / slabs are done
        if (threadIdx.x < KTILE) flags[threadIdx.x] = 0;
        __syncthreads();
        {
            // the chunk's BM x kt map entries, read row by row: entry e of the
            // chunk is (row e / kt, offset e % kt) and thread t takes e = t,
            // t + CT, ..., so a load instruction covers a few whole rows (a few
            // cache lines) rather than one row per lane.  All loads are in
            // flight at once: unguarded, from clamped addresses (an invalid row
            // reads row 0, entries past the chunk re-read its last entry), with
            // the results dropped when they are written to LDS.
            constexpr int MPT = (BM * KTILE + CT - 1) / CT;
            const int dq = CT / kt, dr = CT - dq * kt;
            const int r0 = int(threadIdx.x) / kt, j0 = int(threadIdx.x) - r0 * kt;
            int32_t v[MPT];
            {
                int r = r0, j = j0;
#pragma unroll
                for (int u = 0; u < MPT; ++u) {
                    const bool in = r < BM;
                    const int32_t src = rsrc[in ? r : BM - 1];
                    v[u] = a.map[int64_t(src < 0 ? 0 : src) * a.K + kt0 + (in ? j : kt - 1)];
                    r += dq;
                    j += dr;
                    if (j >= kt) j -= kt, ++r;
                }
            }
            int r = r0, j = j0;
#pragma unroll
            for (int u = 0; u < MPT; ++u) {
                if (r < BM) {
                    const int32_t src = rsrc[r];
                    int32_t val = src < 0 ? -1 : v[u];
                    if ((unsigned)val >= (unsigned)a.n_src) val = -1;
                    tile[j * BMP + r] = val;
                    if (val >= 0) flags[j] = 1;
                }
                r += dq;
                j += dr;
                if (j >= kt) j -= kt, ++r;
            }
        }
        __syncthreads();
        if (wave == 0) {  // compact list of the offsets that hit this tile
            const bool f = lane < kt && flags[lane];
            const uint64_t b = __ballot(f);
            if (f) list[__popcll(b & ((1ull << lane) - 1))] = lane;
            if (lane == 0) list[KTILE] = __popcll(b);
        }
        __syncthreads();
        }
        const int nk = list[KTILE];
        if (nk == 0) continue;

        auto slab_of = [&](int j) { const int kg = kt0 + list[j]; return a.w_rev ? a.K - 1 - kg : kg; };
        if constexpr (PIPE) {
            // Short contractions: two offsets of gathered rows in flight.  Three
            // register buffers take fixed roles in a loop unrolled by three (a
            // buffer copy would wait for its loads), the barriers wait for LDS
            // operations only, so the gathers stay in flight across them, and
            // every load is branch-free (masked lanes, and prefetches past the
            // last offset, take out-of-range buffer offsets and load zeros
            // without a memory access; the slab staged after the last offset
            // goes to the buffer no longer read), so the compiler's wait
            // counts stay exact.  Since the step's loads share its MFMAs'
            // scheduling region it pays on every map with more than one
            // offset (strided and inverse maps too); the identity map of a
            // k = 1 layer runs the plain loop below, which stages nothing
            // past its one offset.
            // The next offset's weight slab is staged one step ahead as before
            // (its loads hit L2).
            u32x4 ga[RB][KCMAX], gb[RB][KCMAX], gc[RB][KCMAX];
            bool fa = false, fb = false, fc = false;
            const __amdgpu_buffer_rsrc_t xr = buf_rsrc(a.x, uint32_t(a.n_src) * uint32_t(a.CK) * uint32_t(sizeof(S)));
            const __amdgpu_buffer_rsrc_t wr =
                buf_rsrc(a.w, uint32_t(a.K) * uint32_t(a.cin) * uint32_t(a.cout) * uint32_t(sizeof(S)));
            // The step's loads (the next slab, the gathers two offsets ahead)
            // share one scheduling region with its MFMAs, which spread them
            // among the MFMAs (mma); a wave without hits at this offset
            // issues the loads alone.
            // With chunk items (every variant except the per-tile transposing
            // forward) the loads are branch-free.  Where the MFMA loop has the
            // interleaving pattern (16-bit, plain slab layout) the MFMAs run
            // for every wave, hits or not (a wave without hits multiplies
            // zero fragments, which leaves its sums as they are), so that
            // loads and MFMAs form one region; elsewhere a wave without hits
            // skips its MFMAs.
            constexpr bool MERGED = WS::ITEM_REGS == 1 && !ROWS && TT::E == 8;
            auto loads = [&](int j, u32x4 (&pre)[RB][KCMAX], bool& any_pre) {
                const int jn = min(j + 1, nk - 1);
                if constexpr (WS::ITEM_REGS == 1)
                    wst.template load_exact<KCMAX * 4, NPRE>(a, wr, slab_of(jn), j + 1 < nk);
                else
                    wst.load_buf(a, wr, slab_of(jn), j + 1 < nk);
                any_pre = gather_buf<TT, RB, KCMAX>(pre, a, xr, cols + list[min(j + 2, nk - 1)] * BMP, j + 2 < nk,
                                                    wave, lr, lg);
            };
            auto step = [&](int j, const u32x4 (&cur)[RB][KCMAX], bool any, u32x4 (&pre)[RB][KCMAX], bool& any_pre) {
                const int jn = min(j + 1, nk - 1);
                loads(j, pre, any_pre);
                if constexpr (MERGED)
                    mma(cur, j, std::integral_constant<int, NPRE + RB * KCMAX>{});
                else if (any)
                    mma(cur, j, std::integral_constant<int, 0>{});
                wst.store(lds + ((j + 1) & 1) * slab_bytes, a, slab_of(jn));
                lds_barrier();
            };
            wst.load_buf(a, wr, slab_of(0), true);
            fa = gather_buf<TT, RB, KCMAX>(ga, a, xr, cols + list[0] * BMP, true, wave, lr, lg);
            fb = gather_buf<TT, RB, KCMAX>(gb, a, xr, cols + list[min(1, nk - 1)] * BMP, nk > 1, wave, lr, lg);
            wst.store(lds, a, slab_of(0));
            lds_barrier();
            for (int j = 0; j < nk; j += 3) {
                step(j, ga, fa, gc, fc);
                if (j + 1 < nk) step(j + 1, gb, fb, ga, fa);
                if (j + 2 < nk) step(j + 2, gc, fc, gb, fb);
            }
            continue;
        }
        wst.load(a, slab_of(0));
        bool any_cur = gather_rows<TT, RB, KCMAX>(acur, a, cols + list[0] * BMP, wave, lr, lg);
        wst.store(lds, a, slab_of(0));
        // drain the prologue's gathers here, so that inside the loop the only
        // loads in flight are the next offset's prefetches and the MFMAs need
        // not wait for them
        __builtin_amdgcn_s_waitcnt(WAIT_VMCNT0);
        __syncthreads();
        for (int j = 0; j < nk; ++j) {
            const bool has_next = j + 1 < nk;
            bool any_next = false;
            if (has_next) {
                wst.load(a, slab_of(j + 1));
                any_next = gather_rows<TT, RB, KCMAX>(anext, a, cols + list[j + 1] * BMP, wave, lr, lg);
            }
            if (any_cur) mma(acur, j, std::integral_constant<int, 0>{});
            if (has_next) wst.store(lds + ((j + 1) & 1) * slab_bytes, a, slab_of(j + 1));
            __syncthreads();
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int kc = 0; kc < KCMAX; ++kc) acur[rb][kc] = anext[rb][kc];
            any_cur = any_next;
        }
    }

    epilogue(lds);

}

constexpr int RB_DEFAULT = 2;

template <typename TT, int NB, bool TRANS, int KCMAX, bool PIPE, bool PERSIST = false>
spc_status launch_conv_nb(const ConvArgs& a, hipStream_t stream) {
    constexpr int BN = NB * 16;
    constexpr int BM = NW * RB_DEFAULT * 16;
    auto kern = k_conv<TT, RB_DEFAULT, NB, TRANS, KCMAX, PIPE, PERSIST>;
    static_assert((2 * KTILE + 4) % 4 == 0, "flags + list keep the following arrays 16-byte aligned");
    using S = typename TT::storage;
    const size_t main_bytes = 2 * size_t(slab_bytes_of<BN, rows_layout<TT, TRANS, KCMAX>()>(a.kch)) +
                              (size_t(KTILE) * (BM + 1) + 2 * KTILE + 4) * 4;
    const size_t stage_bytes = size_t(BM) * (BN * sizeof(S) + 16);  // the epilogue's staged outputs
    // the persistent walk keeps one slab and stages its outputs after it
    const size_t slab1 = size_t(slab_bytes_of<BN, rows_layout<TT, TRANS, KCMAX>()>(a.kch));
    const size_t lds = (PERSIST ? slab1 + stage_bytes : std::max(main_bytes, stage_bytes)) + BM * 4 + BN * 4;
    if (lds > 160 * 1024) return fail(SPC_ERR_UNSUPPORTED, "LDS tile of %zu bytes exceeds 160 KiB", lds);
    if (lds > 64 * 1024) SPC_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)));
    dim3 grid(unsigned(ceil_div(a.n_rows, BM)), unsigned(a.CN / BN));
    if (PERSIST) {
        // at most two workgroups per CU and column block, each with an equal
        // share (to one tile) of the tiles
        const int64_t tiles = ceil_div(a.n_rows, BM);
        const int64_t slots = std::max<int64_t>(1, 2 * int64_t(device_cus()) / int64_t(grid.y));
        const int64_t per = ceil_div(tiles, std::min(tiles, slots));
        grid.x = unsigned(ceil_div(tiles, per));
    }
    hipLaunchKernelGGL(kern, grid, dim3(CT), lds, stream, a);
    SPC_LAUNCHED("k_conv");
    return SPC_OK;
}

template <typename TT, bool TRANS, int KCMAX, bool PIPE = false, bool PERSIST = false>
spc_status launch_conv_k(const ConvArgs& a, hipStream_t stream) {
    const int blocks = a.CN / 16;
    if (blocks % 8 == 0) return launch_conv_nb<TT, 8, TRANS, KCMAX, PIPE, PERSIST>(a, stream);
    if (blocks % 6 == 0) return launch_conv_nb<TT, 6, TRANS, KCMAX, PIPE, PERSIST>(a, stream);
    if (blocks % 4 == 0) return launch_conv_nb<TT, 4, TRANS, KCMAX, PIPE, PERSIST>(a, stream);
    if (blocks % 3 == 0) return launch_conv_nb<TT, 3, TRANS, KCMAX, PIPE, PERSIST>(a, stream);
    if (blocks % 2 == 0) return launch_conv_nb<TT, 2, TRANS, KCMAX, PIPE, PERSIST>(a, stream);
    return launch_conv_nb<TT, 1, TRANS, KCMAX, PIPE, PERSIST>(a, stream);
}

template <typename TT, bool TRANS>
spc_status launch_conv_t(ConvArgs& a, hipStream_t stream) {
    constexpr int E = TT::E;
    a.kch = int(ceil_div(a.CK / E, 4) * 4);
    const int KC = a.kch / 4;
    // gathered-row registers sized to the contraction: a 2-step variant frees
    // 32 registers per lane for contractions of up to 64 (16-bit) channels.
    // Over any map with more than one offset the 1- to 4-step variants keep a
    // second offset of gathers in flight (addressing x and the weights through
    // buffer resources, so both must lie within 2 GiB); the identity map of a
    // k = 1 layer (one offset) keeps the plain loop.
    // Up to 4 steps the variant matches KC exactly (its loops have no run-time
    // bound); 5 to 8 steps share one bounded variant.
    const bool pipe = a.xbuf && a.K > 1;
    // the identity map of a k = 1 layer (rows counted on the host) walks its
    // tiles persistently, with the slab staged once per workgroup
    const bool persist = a.xbuf && !a.map && a.K == 1 && !a.n_rows_dev;
    switch (KC) {
#define SPC_CONV_CASE(N)                                                  \
    case N:                                                               \
        if (pipe) return launch_conv_k<TT, TRANS, N, true>(a, stream);     \
        if (persist) return launch_conv_k<TT, TRANS, N, false, true>(a, stream); \
        return launch_conv_k<TT, TRANS, N>(a, stream);
        SPC_CONV_CASE(1)
        SPC_CONV_CASE(2)
        SPC_CONV_CASE(3)
        SPC_CONV_CASE(4)
#undef SPC_CONV_CASE
        default: break;
    }
    if (KC <= 8) return launch_conv_k<TT, TRANS, 8>(a, stream);
    return fail(SPC_ERR_UNSUPPORTED, "contraction of %d channels exceeds %d for this dtype", a.CK, 8 * 4 * E);
}

}  // namespace
#endif  // SPC_CONV_KERNELS

}  // namespace spc
