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

template <typename TT>
__global__ __launch_bounds__(PT) void k_maxpool_fwd(const void* __restrict__ x_, const int32_t* __restrict__ nbr,
                                                    int32_t n_out, int32_t n_in, int32_t C, int32_t K,
                                                    void* __restrict__ y_, uint8_t* __restrict__ argk) {
    constexpr int E = TT::E;
    using S = typename TT::storage;
    using AW = ArgWord<E>;
    const int cpr = C / E;  // 16-byte chunks per row
    const int g = int(blockIdx.x) * PT + int(threadIdx.x);
    if (g >= n_out * cpr) return;
    const int row = g / cpr, ch = (g - row * cpr) * E;
    const S* x = static_cast<const S*>(x_);
    const int32_t* m = nbr + int64_t(row) * K;

    float best[E];
    int arg[E];
#pragma unroll
    for (int e = 0; e < E; ++e) best[e] = -__builtin_inff(), arg[e] = NO_ARG;
    const int kend = n_in > 0 ? K : 0;  // no input rows: nothing to gather (x may be NULL)
    for (int k0 = 0; k0 < kend; k0 += KB) {
        int32_t idx[KB];
#pragma unroll
        for (int j = 0; j < KB; ++j) idx[j] = m[k0 + j < K ? k0 + j : K - 1];
        u32x4 v[KB];
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            const int32_t s = (unsigned)idx[j] < (unsigned)n_in ? idx[j] : 0;
            v[j] = ld16(x + int64_t(s) * C + ch);
        }
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            if (k0 + j < K && (unsigned)idx[j] < (unsigned)n_in) {
                float f[E];
                unpack<TT>(v[j], f);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (f[e] > best[e]) best[e] = f[e], arg[e] = k0 + j;  // strictly greater: the first max stays
            }
        }
    }
#pragma unroll
    for (int e = 0; e < E; ++e)
        if (arg[e] == NO_ARG) best[e] = 0.f;
    st16(static_cast<S*>(y_) + int64_t(row) * C + ch, pack<TT>(best));
    if (argk) *reinterpret_cast<typename AW::T*>(argk + int64_t(row) * C + ch) = AW::pack(arg);
}

template <typename TT>
__global__ __launch_bounds__(PT) void k_maxpool_bwd(const void* __restrict__ dy_, const uint8_t* __restrict__ argk,
                                                    const int32_t* __restrict__ nbr_in, int32_t n_in, int32_t n_out,
                                                    int32_t C, int32_t K, void* __restrict__ dx_) {
    constexpr int E = TT::E;
    using S = typename TT::storage;
    using AW = ArgWord<E>;
    const int cpr = C / E;
    const int g = int(blockIdx.x) * PT + int(threadIdx.x);
    if (g >= n_in * cpr) return;
    const int row = g / cpr, ch = (g - row * cpr) * E;
    const S* dy = static_cast<const S*>(dy_);
    const int32_t* m = nbr_in + int64_t(row) * K;

    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    const int kend = n_out > 0 ? K : 0;  // no output rows: nothing to gather (dout, argk may be NULL)
    for (int k0 = 0; k0 < kend; k0 += KB) {
        int32_t idx[KB];
#pragma unroll
        for (int j = 0; j < KB; ++j) idx[j] = m[k0 + j < K ? k0 + j : K - 1];
        u32x4 v[KB];
        typename AW::T w[KB];
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            const int32_t s = (unsigned)idx[j] < (unsigned)n_out ? idx[j] : 0;
            v[j] = ld16(dy + int64_t(s) * C + ch);
            w[j] = *reinterpret_cast<const typename AW::T*>(argk + int64_t(s) * C + ch);
        }
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            if (k0 + j < K && (unsigned)idx[j] < (unsigned)n_out) {
                float f[E];
                unpack<TT>(v[j], f);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (AW::get(w[j], e) == k0 + j) acc[e] += f[e];
            }
        }
    }
    st16(static_cast<S*>(dx_) + int64_t(row) * C + ch, pack<TT>(acc));
}

template <typename TT>
spc_status launch_fwd(const void* x, const int32_t* nbr, int64_t n_out, int64_t n_in, int32_t C, int32_t K, void* y,
                      uint8_t* argk, hipStream_t stream) {
    const int64_t threads = n_out * (C / TT::E);
    hipLaunchKernelGGL(k_maxpool_fwd<TT>, dim3(unsigned(ceil_div(threads, PT))), dim3(PT), 0, stream, x, nbr,
                       int32_t(n_out), int32_t(n_in), C, K, y, argk);
    SPC_LAUNCHED("k_maxpool_fwd");
    return SPC_OK;
}

template <typename TT>
spc_status launch_bwd(const void* dy, const uint8_t* argk, const int32_t* nbr_in, int64_t n_in, int64_t n_out,
                      int32_t C, int32_t K, void* dx, hipStream_t stream) {
    const int64_t threads = n_in * (C / TT::E);
    hipLaunchKernelGGL(k_maxpool_bwd<TT>, dim3(unsigned(ceil_div(threads, PT))), dim3(PT), 0, stream, dy, argk,
                       nbr_in, int32_t(n_in), int32_t(n_out), C, K, dx);
    SPC_LAUNCHED("k_maxpool_bwd");
    return SPC_OK;
}

spc_status check_pool(spc_dtype dt, int64_t n_rows, int64_t n_src, int32_t C, int32_t K) {
    if (dt != SPC_F32 && dt != SPC_F16 && dt != SPC_BF16) return fail(SPC_ERR_ARG, "unknown dtype %d", int(dt));
    if (C <= 0 || C % 16) return fail(SPC_ERR_UNSUPPORTED, "C=%d: channels must be a positive multiple of 16", C);
    if (K < 1 || K >= NO_ARG) return fail(SPC_ERR_UNSUPPORTED, "K=%d: pooling takes 1..%d offsets", K, NO_ARG - 1);
    if (n_rows < 0 || n_src < 0 || n_src >= (int64_t(1) << 31)) return fail(SPC_ERR_ARG, "row counts out of range");
    // one thread per (row, 16-byte chunk), indexed in 32 bits
    if (n_rows * (C / (dt == SPC_F32 ? 4 : 8)) >= (int64_t(1) << 31))
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
