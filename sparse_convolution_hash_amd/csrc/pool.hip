// Sparse max pooling over a strided kernel map (SparseMaxPool3d, spconv
// USAGE.md layer table: downsampling whose dense version is nn.MaxPool3d).
//
//   forward   out[o][c]  = max over k with nbr_out[o][k] >= 0 of x[nbr_out[o][k]][c]
//             argk[o][c] = the first k (offset order) that reaches it
//   backward  din[i][c]  = sum over k with o = nbr_in[i][k] >= 0 and argk[o][c] == k
//                          of dout[o][c]
//
// Both are gathers with no arithmetic to speak of, so they are HBM/L2 bound:
// one thread owns one row and one 16-byte chunk of its channels (consecutive
// threads take consecutive chunks of a row, so every gather and store is a
// contiguous run of the row), reads the row's map entries in batches of KB,
// and keeps KB gathers in flight at once from clamped addresses whose results
// are dropped when the entry is absent.  The backward is input-stationary: it
// reads the transposed map, so every input row is written once, in a fixed
// offset order (no atomics, run-to-run identical).
#include "common.h"

namespace spc {
namespace {

constexpr int PT = 256;  // threads per workgroup
constexpr int KB = 8;    // map entries (and gathers) in flight per thread
constexpr int NO_ARG = 255;

// 16 bytes of the element type as E floats (exact), and back (exact for
// values of the element type).
template <typename TT>
__device__ __forceinline__ void unpack(const u32x4& v, float (&f)[TT::E]);
template <>
__device__ __forceinline__ void unpack<F32>(const u32x4& v, float (&f)[4]) {
    f[0] = __uint_as_float(v.x), f[1] = __uint_as_float(v.y), f[2] = __uint_as_float(v.z), f[3] = __uint_as_float(v.w);
}
template <>
__device__ __forceinline__ void unpack<BF16>(const u32x4& v, float (&f)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) f[2 * i] = __uint_as_float(w[i] << 16), f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
}
template <>
__device__ __forceinline__ void unpack<F16>(const u32x4& v, float (&f)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = float(__builtin_bit_cast(_Float16, uint16_t(w[i] & 0xffffu)));
        f[2 * i + 1] = float(__builtin_bit_cast(_Float16, uint16_t(w[i] >> 16)));
    }
}

template <typename TT>
__device__ __forceinline__ u32x4 pack(const float (&f)[TT::E]);
template <>
__device__ __forceinline__ u32x4 pack<F32>(const float (&f)[4]) {
    return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
}
template <>
__device__ __forceinline__ u32x4 pack<BF16>(const float (&f)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = uint32_t(f32_to_bf16_rne(f[2 * i])) | (uint32_t(f32_to_bf16_rne(f[2 * i + 1])) << 16);
    return u32x4{w[0], w[1], w[2], w[3]};
}
template <>
__device__ __forceinline__ u32x4 pack<F16>(const float (&f)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = uint32_t(f32_to_f16_rne(f[2 * i])) | (uint32_t(f32_to_f16_rne(f[2 * i + 1])) << 16);
    return u32x4{w[0], w[1], w[2], w[3]};
}

// E winner bytes (one per channel) as one 4- or 8-byte word.
template <int E>
struct ArgWord;
template <>
struct ArgWord<4> {
    using T = uint32_t;
    __device__ static T pack(const int (&a)[4]) {
        return uint32_t(a[0]) | (uint32_t(a[1]) << 8) | (uint32_t(a[2]) << 16) | (uint32_t(a[3]) << 24);
    }
    __device__ static int get(T w, int e) { return int((w >> (8 * e)) & 0xffu); }
};
template <>
struct ArgWord<8> {
    using T = uint2;
    __device__ static T pack(const int (&a)[8]) {
        return uint2{uint32_t(a[0]) | (uint32_t(a[1]) << 8) | (uint32_t(a[2]) << 16) | (uint32_t(a[3]) << 24),
                     uint32_t(a[4]) | (uint32_t(a[5]) << 8) | (uint32_t(a[6]) << 16) | (uint32_t(a[7]) << 24)};
    }
    __device__ static int get(T w, int e) { return int(((e < 4 ? w.x : w.y) >> (8 * (e & 3))) & 0xffu); }
};

// Lane layout of both kernels: a row's cpr = C / E 16-byte chunks go to cpr
// consecutive lanes of one wave (rpw = 64 / cpr rows per wave, the last
// 64 - rpw * cpr lanes idle).  The row's map entries are read once, four
// consecutive ones per lane, and handed to the row's lanes by shuffles; a
// batch of 8 offsets that no row of the wave has is skipped.
struct RowLanes {
    int cpr, rpw, grp, j, row;
    bool ok;  // this lane's row exists
    __device__ RowLanes(int C, int E, int n_rows) {
        cpr = C / E;
        rpw = WAVE / cpr;
        const int lane = int(threadIdx.x) & (WAVE - 1);
        const int wave = (int(blockIdx.x) * PT + int(threadIdx.x)) / WAVE;
        grp = lane / cpr;
        j = lane - grp * cpr;
        row = wave * rpw + grp;
        ok = grp < rpw && row < n_rows;
    }
};

// The entries [k0, k0 + 4 cpr) of a row: lane j holds k0 + 4j .. k0 + 4j + 3
// (unguarded loads of a valid row, clamped to the last entry).
__device__ __forceinline__ void load_entries(int32_t (&e)[4], const int32_t* m, int k0, int j, int K) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int k = k0 + 4 * j + q;
        e[q] = m[k < K ? k : K - 1];
    }
}

// Entry k0 + kb + t (t < 8, kb a multiple of 8) of this lane's row.
__device__ __forceinline__ int32_t entry_at(const int32_t (&e)[4], int grp, int cpr, int kb, int t) {
    const int src = grp * cpr + (kb >> 2) + (t >> 2);
    return __shfl(e[t & 3], src);
}

template <typename TT>
__global__ __launch_bounds__(PT) void k_maxpool_fwd(const void* __restrict__ x_, const int32_t* __restrict__ nbr,
                                                    int32_t n_out, int32_t n_in, int32_t C, int32_t K,
                                                    void* __restrict__ y_, uint8_t* __restrict__ argk) {
    constexpr int E = TT::E;
    using S = typename TT::storage;
    using AW = ArgWord<E>;
    const RowLanes L(C, E, n_out);
    if ((int(blockIdx.x) * PT + int(threadIdx.x)) / WAVE * L.rpw >= n_out) return;  // whole wave past the end
    const int ch = L.j * E;
    const S* x = static_cast<const S*>(x_);
    const int32_t* m = nbr + int64_t(L.ok ? L.row : n_out - 1) * K;

    float best[E];
    int arg[E];
#pragma unroll
    for (int e = 0; e < E; ++e) best[e] = -__builtin_inff(), arg[e] = NO_ARG;
    const int kend = n_in > 0 ? K : 0;  // no input rows: nothing to gather (x may be NULL)
    for (int k0 = 0; k0 < kend; k0 += 4 * L.cpr) {
        int32_t e4[4];
        load_entries(e4, m, k0, L.j, K);
        for (int kb = 0; kb < 4 * L.cpr && k0 + kb < K; kb += KB) {
            int32_t idx[KB];
            bool val[KB];
            bool any = false;
#pragma unroll
            for (int t = 0; t < KB; ++t) {
                idx[t] = entry_at(e4, L.grp, L.cpr, kb, t);
                val[t] = L.ok && k0 + kb + t < K && (unsigned)idx[t] < (unsigned)n_in;
                any = any || val[t];
            }
            if (!__any(any)) continue;  // (uniform) no row of this wave has these offsets
            u32x4 v[KB];
#pragma unroll
            for (int t = 0; t < KB; ++t) v[t] = ld16(x + int64_t(val[t] ? idx[t] : 0) * C + ch);
#pragma unroll
            for (int t = 0; t < KB; ++t) {
                if (val[t]) {
                    float f[E];
                    unpack<TT>(v[t], f);
#pragma unroll
                    for (int q = 0; q < E; ++q)
                        if (f[q] > best[q]) best[q] = f[q], arg[q] = k0 + kb + t;  // strictly greater: the first max stays
                }
            }
        }
    }
    if (!L.ok) return;
#pragma unroll
    for (int e = 0; e < E; ++e)
        if (arg[e] == NO_ARG) best[e] = 0.f;
    st16(static_cast<S*>(y_) + int64_t(L.row) * C + ch, pack<TT>(best));
    if (argk) *reinterpret_cast<typename AW::T*>(argk + int64_t(L.row) * C + ch) = AW::pack(arg);
}

template <typename TT>
__global__ __launch_bounds__(PT) void k_maxpool_bwd(const void* __restrict__ dy_, const uint8_t* __restrict__ argk,
                                                    const int32_t* __restrict__ nbr_in, int32_t n_in, int32_t n_out,
                                                    int32_t C, int32_t K, void* __restrict__ dx_) {
    constexpr int E = TT::E;
    using S = typename TT::storage;
    using AW = ArgWord<E>;
    const RowLanes L(C, E, n_in);
    if ((int(blockIdx.x) * PT + int(threadIdx.x)) / WAVE * L.rpw >= n_in) return;  // whole wave past the end
    const int ch = L.j * E;
    const S* dy = static_cast<const S*>(dy_);
    const int32_t* m = nbr_in + int64_t(L.ok ? L.row : n_in - 1) * K;

    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    const int kend = n_out > 0 ? K : 0;  // no output rows: nothing to gather (dout, argk may be NULL)
    for (int k0 = 0; k0 < kend; k0 += 4 * L.cpr) {
        int32_t e4[4];
        load_entries(e4, m, k0, L.j, K);
        for (int kb = 0; kb < 4 * L.cpr && k0 + kb < K; kb += KB) {
            int32_t idx[KB];
            bool val[KB];
            bool any = false;
#pragma unroll
            for (int t = 0; t < KB; ++t) {
                idx[t] = entry_at(e4, L.grp, L.cpr, kb, t);
                val[t] = L.ok && k0 + kb + t < K && (unsigned)idx[t] < (unsigned)n_out;
                any = any || val[t];
            }
            if (!__any(any)) continue;  // (uniform) no row of this wave has these offsets
            u32x4 v[KB];
            typename AW::T w[KB];
#pragma unroll
            for (int t = 0; t < KB; ++t) {
                const int64_t off = int64_t(val[t] ? idx[t] : 0) * C + ch;
                v[t] = ld16(dy + off);
                w[t] = *reinterpret_cast<const typename AW::T*>(argk + off);
            }
#pragma unroll
            for (int t = 0; t < KB; ++t) {
                if (val[t]) {
                    float f[E];
                    unpack<TT>(v[t], f);
#pragma unroll
                    for (int q = 0; q < E; ++q)
                        if (AW::get(w[t], q) == k0 + kb + t) acc[q] += f[q];
                }
            }
        }
    }
    if (!L.ok) return;
    st16(static_cast<S*>(dx_) + int64_t(L.row) * C + ch, pack<TT>(acc));
}

// Threads of a launch over `rows` rows: whole waves of 64 / cpr rows.
inline int64_t pool_threads(int64_t rows, int32_t C, int E) {
    const int rpw = WAVE / (C / E);
    return ceil_div(rows, rpw) * WAVE;
}

template <typename TT>
spc_status launch_fwd(const void* x, const int32_t* nbr, int64_t n_out, int64_t n_in, int32_t C, int32_t K, void* y,
                      uint8_t* argk, hipStream_t stream) {
    const int64_t threads = pool_threads(n_out, C, TT::E);
    hipLaunchKernelGGL(k_maxpool_fwd<TT>, dim3(unsigned(ceil_div(threads, PT))), dim3(PT), 0, stream, x, nbr,
                       int32_t(n_out), int32_t(n_in), C, K, y, argk);
    SPC_LAUNCHED("k_maxpool_fwd");
    return SPC_OK;
}

template <typename TT>
spc_status launch_bwd(const void* dy, const uint8_t* argk, const int32_t* nbr_in, int64_t n_in, int64_t n_out,
                      int32_t C, int32_t K, void* dx, hipStream_t stream) {
    const int64_t threads = pool_threads(n_in, C, TT::E);
    hipLaunchKernelGGL(k_maxpool_bwd<TT>, dim3(unsigned(ceil_div(threads, PT))), dim3(PT), 0, stream, dy, argk,
                       nbr_in, int32_t(n_in), int32_t(n_out), C, K, dx);
    SPC_LAUNCHED("k_maxpool_bwd");
    return SPC_OK;
}

spc_status check_pool(spc_dtype dt, int64_t n_rows, int64_t n_src, int32_t C, int32_t K) {
    if (dt != SPC_F32 && dt != SPC_F16 && dt != SPC_BF16) return fail(SPC_ERR_ARG, "unknown dtype %d", int(dt));
    if (C <= 0 || C % 16) return fail(SPC_ERR_UNSUPPORTED, "C=%d: channels must be a positive multiple of 16", C);
    const int E = dt == SPC_F32 ? 4 : 8;
    if (C / E > WAVE)  // a row's 16-byte chunks share one wave
        return fail(SPC_ERR_UNSUPPORTED, "C=%d: pooling takes at most %d channels of this dtype", C, WAVE * E);
    if (K < 1 || K >= NO_ARG) return fail(SPC_ERR_UNSUPPORTED, "K=%d: pooling takes 1..%d offsets", K, NO_ARG - 1);
    if (n_rows < 0 || n_src < 0 || n_src >= (int64_t(1) << 31)) return fail(SPC_ERR_ARG, "row counts out of range");
    // whole waves of rows, thread indices in 32 bits
    if (pool_threads(n_rows, C, E) >= (int64_t(1) << 31))
        return fail(SPC_ERR_UNSUPPORTED, "%lld rows of %d channels exceed one launch", (long long)n_rows, C);
    return SPC_OK;
}

}  // namespace
}  // namespace spc

using namespace spc;

extern "C" spc_status spc_sparse_maxpool_fwd(spc_dtype dtype, const void* feats, int64_t n_in, int32_t C,
                                             const int32_t* nbr_out, int32_t K, int64_t n_out, void* out,
                                             uint8_t* argk, hipStream_t stream) {
    clear_error();
    spc_status st = check_pool(dtype, n_out, n_in, C, K);
    if (st != SPC_OK) return st;
    if (n_out == 0) return SPC_OK;
    if (!nbr_out || !out || (n_in > 0 && !feats)) return fail(SPC_ERR_ARG, "feats, nbr_out or out is NULL");
    for (const void* p : {feats, (const void*)nbr_out, (const void*)out, (const void*)argk})
        if (p && !aligned16(p)) return fail(SPC_ERR_ARG, "device pointers must be 16-byte aligned");
    switch (dtype) {
        case SPC_F32: return launch_fwd<F32>(feats, nbr_out, n_out, n_in, C, K, out, argk, stream);
        case SPC_F16: return launch_fwd<F16>(feats, nbr_out, n_out, n_in, C, K, out, argk, stream);
        case SPC_BF16: return launch_fwd<BF16>(feats, nbr_out, n_out, n_in, C, K, out, argk, stream);
    }
    return fail(SPC_ERR_ARG, "unknown dtype %d", int(dtype));
}

extern "C" spc_status spc_sparse_maxpool_bwd(spc_dtype dtype, const void* dout, int64_t n_out, int32_t C,
                                             const uint8_t* argk, const int32_t* nbr_in, int32_t K, int64_t n_in,
                                             void* din, hipStream_t stream) {
    clear_error();
    spc_status st = check_pool(dtype, n_in, n_out, C, K);
    if (st != SPC_OK) return st;
    if (n_in == 0) return SPC_OK;
    if (!nbr_in || !din || (n_out > 0 && (!dout || !argk)))
        return fail(SPC_ERR_ARG, "dout, argk, nbr_in or din is NULL");
    for (const void* p : {dout, (const void*)argk, (const void*)nbr_in, (const void*)din})
        if (p && !aligned16(p)) return fail(SPC_ERR_ARG, "device pointers must be 16-byte aligned");
    switch (dtype) {
        case SPC_F32: return launch_bwd<F32>(dout, argk, nbr_in, n_in, n_out, C, K, din, stream);
        case SPC_F16: return launch_bwd<F16>(dout, argk, nbr_in, n_in, n_out, C, K, din, stream);
        case SPC_BF16: return launch_bwd<BF16>(dout, argk, nbr_in, n_in, n_out, C, K, din, stream);
    }
    return fail(SPC_ERR_ARG, "unknown dtype %d", int(dtype));
}
