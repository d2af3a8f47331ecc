// Weight and bias gradients of the sparse convolution.
//
//   dW[k] = sum over the pairs (i, o) of offset k of x[i]^T dy[o]   [cin, cout]
//   dbias = sum over rows o of dy[o]                                 [cout]
//
// (the Hygon spconv-das README's dfilter, "Public Interface Support").  The
// contraction runs over pairs, so each workgroup takes one offset, one
// channel tile and one fixed-size chunk of that offset's CSR pair list; it
// gathers 64 pairs at a time, transposes them in registers into
// channel-major LDS tiles (the MFMA fragments need 16 bytes of consecutive
// pairs per channel) and accumulates fp32 on MFMA.  Each chunk writes a
// partial tile; a second kernel sums the partials in chunk order, so the
// result does not depend on scheduling.
#include <algorithm>

#include "common.h"

namespace spc {
namespace {

constexpr int DT = 256;          // threads per workgroup (2 x 2 waves)
constexpr int PS = 64;           // pairs staged per step
constexpr int TMAX = 128;        // channel tile edge
constexpr int TARGET_WG = 512;   // workgroups the split count aims for
constexpr int MIN_PAIRS_PER_SPLIT = 1024;

struct DfArgs {
    const void* x;        // [n_in, cin]
    const void* dy;       // [n_out, cout]
    const int32_t* ptr;   // [K+1] or NULL (identity pairs, K == 1)
    const int32_t* pin;
    const int32_t* pout;
    float* part;          // [K, S, cin, cout]
    int32_t n_in, n_out, cin, cout, K, S;
};

// Row stride (bytes) of a channel-major LDS tile: PS pairs plus 16 bytes of
// padding so that consecutive channels fall in different banks.
template <typename TT>
constexpr int lds_row() { return PS * int(sizeof(typename TT::storage)) + 16; }

// Gathers E pairs x (E channels) of one operand and stores them transposed:
// lds[ch][pair] with 16 consecutive bytes of pairs per channel.
template <typename TT>
__device__ __forceinline__ void stage_transposed(char* lds, const typename TT::storage* src, const int32_t* rows,
                                                 int C, int c0, int chunk, int pg) {
    constexpr int E = TT::E;
    u32x4 in[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        in[e] = zero4();
        if (rows[e] >= 0) in[e] = ld16(src + int64_t(rows[e]) * C + c0 + chunk * E);
    }
    char* dst = lds + (chunk * E) * lds_row<TT>() + pg * 16;
    if constexpr (E == 8) {
        typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
        u16x8 v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = __builtin_bit_cast(u16x8, in[e]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            u16x8 o = {v[0][j], v[1][j], v[2][j], v[3][j], v[4][j], v[5][j], v[6][j], v[7][j]};
            st16(dst + j * lds_row<TT>(), __builtin_bit_cast(u32x4, o));
        }
    } else {
        const uint32_t m[4][4] = {{in[0].x, in[0].y, in[0].z, in[0].w},
                                  {in[1].x, in[1].y, in[1].z, in[1].w},
                                  {in[2].x, in[2].y, in[2].z, in[2].w},
                                  {in[3].x, in[3].y, in[3].z, in[3].w}};
#pragma unroll
        for (int j = 0; j < 4; ++j) st16(dst + j * lds_row<TT>(), u32x4{m[0][j], m[1][j], m[2][j], m[3][j]});
    }
}

template <typename TT>
__global__ __launch_bounds__(DT) void k_dfilter(DfArgs a) {
    using S = typename TT::storage;
    constexpr int E = TT::E;
    constexpr int ROW = lds_row<TT>();
    __shared__ __attribute__((aligned(16))) char xt[TMAX * ROW];  // [ci][pairs]
    __shared__ __attribute__((aligned(16))) char gt[TMAX * ROW];  // [co][pairs]

    const int k = blockIdx.y, s = blockIdx.x;
    const int tiles_o = (a.cout + TMAX - 1) / TMAX;
    const int ci0 = (blockIdx.z / tiles_o) * TMAX, co0 = (blockIdx.z % tiles_o) * TMAX;
    const int TI = min(TMAX, a.cin - ci0), TO = min(TMAX, a.cout - co0);
    const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
    const int lr = lane & 15, lg = lane >> 4;
    const int wi = wave >> 1, wo = wave & 1;
    const int MI = (TI / 16 + 1) / 2, NO = (TO / 16 + 1) / 2;  // 16x16 blocks per wave (<= 4)

    int64_t pbeg, pend;
    if (a.ptr) {
        pbeg = a.ptr[k];
        pend = a.ptr[k + 1];
    } else {
        pbeg = 0;
        pend = a.n_in;
    }
    const int64_t total = pend - pbeg;
    const int64_t chunk = ((total + a.S - 1) / a.S + PS - 1) / PS * PS;
    const int64_t c_beg = min(pend, pbeg + s * chunk), c_end = min(pend, c_beg + chunk);

    f32x4_t acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int no = 0; no < 4; ++no) acc[mi][no] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const S* x = static_cast<const S*>(a.x);
    const S* dy = static_cast<const S*>(a.dy);
    constexpr int PG = PS / E;  // pair groups per step
    const int xi_items = PG * (TI / E), go_items = PG * (TO / E);

    for (int64_t p0 = c_beg; p0 < c_end; p0 += PS) {
        __syncthreads();  // the previous step's tiles are consumed
        for (int it = threadIdx.x; it < xi_items + go_items; it += DT) {
            const bool is_x = it < xi_items;
            const int j = is_x ? it : it - xi_items;
            const int pg = j % PG, ch = j / PG;
            int32_t rows[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int64_t p = p0 + pg * E + e;
                int32_t r = -1;
                if (p < c_end) r = a.ptr ? (is_x ? a.pin[p] : a.pout[p]) : int32_t(p);
                if (is_x ? (unsigned)r >= (unsigned)a.n_in : (unsigned)r >= (unsigned)a.n_out) r = -1;
                rows[e] = r;
            }
            if (is_x)
                stage_transposed<TT>(xt, x, rows, a.cin, ci0, ch, pg);
            else
                stage_transposed<TT>(gt, dy, rows, a.cout, co0, ch, pg);
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < PS / (4 * E); ++ks) {
            const int poff = (ks * 4 + lg) * 16;
            u32x4 gf[4], xf[4];
#pragma unroll
            for (int no = 0; no < 4; ++no)
                if (no < NO && (wo * NO + no) * 16 < TO) gf[no] = ld16(gt + ((wo * NO + no) * 16 + lr) * ROW + poff);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
                if (mi < MI && (wi * MI + mi) * 16 < TI) xf[mi] = ld16(xt + ((wi * MI + mi) * 16 + lr) * ROW + poff);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int no = 0; no < 4; ++no)
                    if (mi < MI && no < NO && (wi * MI + mi) * 16 < TI && (wo * NO + no) * 16 < TO)
                        acc[mi][no] = mfma16<TT>(gf[no], xf[mi], acc[mi][no]);
        }
    }

    // D[co][ci] per 16x16 tile: this lane holds co = lg*4 .. +3 of ci = lr
    float* part = a.part + (int64_t(k) * a.S + s) * a.cin * a.cout;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int no = 0; no < 4; ++no) {
            if (!(mi < MI && no < NO && (wi * MI + mi) * 16 < TI && (wo * NO + no) * 16 < TO)) continue;
            const int ci = ci0 + (wi * MI + mi) * 16 + lr;
            const int co = co0 + (wo * NO + no) * 16 + lg * 4;
            *reinterpret_cast<f32x4_t*>(part + int64_t(ci) * a.cout + co) = acc[mi][no];
        }
}

// out[g][j] = sum over s < S (in order) of part[(g*S + s)*L + j], 4 floats per thread.
__global__ __launch_bounds__(256) void k_reduce_splits(const float* __restrict__ part, int S, int64_t L,
                                                       int64_t groups, float* __restrict__ out) {
    const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (t * 4 >= L * groups) return;
    const int64_t g = (t * 4) / L, j = (t * 4) % L;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < S; ++s) acc += *reinterpret_cast<const f32x4_t*>(part + (g * S + s) * L + j);
    *reinterpret_cast<f32x4_t*>(out + g * L + j) = acc;
}

constexpr int COLSUM_ROWS = 1024;  // rows per dbias partial

// part[r][c] = sum of dy rows [r*COLSUM_ROWS, ...) in column c (fp32).
template <typename TT>
__global__ __launch_bounds__(256) void k_colsum(const typename TT::storage* __restrict__ dy, int32_t n, int32_t C,
                                                float* __restrict__ part) {
    const int r = blockIdx.x;
    const int64_t lo = int64_t(r) * COLSUM_ROWS, hi = min<int64_t>(n, lo + COLSUM_ROWS);
    for (int c = threadIdx.x; c < C; c += 256) {
        float s = 0.f;
        for (int64_t i = lo; i < hi; ++i) {
            if constexpr (TT::id == SPC_F32) {
                s += dy[i * C + c];
            } else if constexpr (TT::id == SPC_BF16) {
                s += __uint_as_float(uint32_t(dy[i * C + c]) << 16);
            } else {
                s += float(__builtin_bit_cast(_Float16, dy[i * C + c]));
            }
        }
        part[int64_t(r) * C + c] = s;
    }
}

int split_count(int64_t n_in, int64_t n_out, int32_t cin, int32_t cout, int32_t K) {
    const int64_t pmax = std::min(n_in, n_out);
    const int64_t tiles = ceil_div(cin, TMAX) * ceil_div(cout, TMAX);
    int64_t s = ceil_div(TARGET_WG, int64_t(K) * tiles);
    s = std::min<int64_t>(s, std::max<int64_t>(1, pmax / MIN_PAIRS_PER_SPLIT));
    return int(std::max<int64_t>(1, std::min<int64_t>(s, 256)));
}

struct DfLayout {
    int S;
    int64_t rparts;  // dbias partial rows
    size_t off_dbias, total;
};

DfLayout df_layout(int64_t n_in, int64_t n_out, int32_t cin, int32_t cout, int32_t K, bool dbias) {
    DfLayout l;
    l.S = split_count(n_in, n_out, cin, cout, K);
    l.rparts = dbias ? std::max<int64_t>(1, ceil_div(n_out, COLSUM_ROWS)) : 0;
    l.off_dbias = align_up(size_t(K) * l.S * cin * cout * 4, 256);
    l.total = align_up(l.off_dbias + size_t(l.rparts) * cout * 4, 256);
    return l;
}

template <typename TT>
spc_status launch_dfilter(const DfArgs& a, float* dw, float* dbias, float* bias_part, int64_t rparts,
                          hipStream_t stream) {
    const unsigned tiles = unsigned(ceil_div(a.cin, TMAX) * ceil_div(a.cout, TMAX));
    hipLaunchKernelGGL(k_dfilter<TT>, dim3(unsigned(a.S), unsigned(a.K), tiles), dim3(DT), 0, stream, a);
    SPC_LAUNCHED("k_dfilter");
    const int64_t L = int64_t(a.cin) * a.cout;
    hipLaunchKernelGGL(k_reduce_splits, dim3(unsigned(ceil_div(L * a.K / 4, 256))), dim3(256), 0, stream, a.part, a.S,
                       L, int64_t(a.K), dw);
    SPC_LAUNCHED("k_reduce_splits");
    if (dbias) {
        if (a.n_out > 0) {
            hipLaunchKernelGGL(k_colsum<TT>, dim3(unsigned(rparts)), dim3(256), 0, stream,
                               static_cast<const typename TT::storage*>(a.dy), a.n_out, a.cout, bias_part);
            SPC_LAUNCHED("k_colsum");
        } else {
            hipLaunchKernelGGL(k_colsum<TT>, dim3(1), dim3(256), 0, stream,
                               static_cast<const typename TT::storage*>(a.dy), 0, a.cout, bias_part);
            SPC_LAUNCHED("k_colsum");
        }
        hipLaunchKernelGGL(k_reduce_splits, dim3(unsigned(ceil_div(a.cout / 4, 256))), dim3(256), 0, stream, bias_part,
                           int(std::max<int64_t>(rparts, 1)), int64_t(a.cout), int64_t(1), dbias);
        SPC_LAUNCHED("k_reduce_splits");
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

extern "C" spc_status spc_conv_bwd_filter(spc_dtype dtype, const void* feats, int64_t n_in, int32_t cin,
                                          const void* dout, int64_t n_out, int32_t cout, int32_t K,
                                          const int32_t* pair_ptr, const int32_t* pair_in, const int32_t* pair_out,
                                          float* dw, float* dbias, void* ws, size_t ws_bytes, hipStream_t stream) {
    clear_error();
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
    const void* ptrs[] = {feats, dout, pair_ptr, pair_in, pair_out, dw, dbias, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(SPC_ERR_ARG, "device pointers must be 16-byte aligned");
    const DfLayout l = df_layout(n_in, n_out, cin, cout, K, dbias != nullptr);
    if (!ws) return fail(SPC_ERR_ARG, "workspace is NULL");
    if (ws_bytes < l.total) return fail(SPC_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, l.total);
    DfArgs a{feats, dout, pair_ptr, pair_in, pair_out, static_cast<float*>(ws), int32_t(n_in), int32_t(n_out),
             cin, cout, K, l.S};
    float* bias_part = reinterpret_cast<float*>(static_cast<char*>(ws) + l.off_dbias);
    switch (dtype) {
        case SPC_F32: return launch_dfilter<F32>(a, dw, dbias, bias_part, l.rparts, stream);
        case SPC_F16: return launch_dfilter<F16>(a, dw, dbias, bias_part, l.rparts, stream);
        case SPC_BF16: return launch_dfilter<BF16>(a, dw, dbias, bias_part, l.rparts, stream);
    }
    return SPC_ERR_ARG;
}
