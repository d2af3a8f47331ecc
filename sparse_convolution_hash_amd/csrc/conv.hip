// C entry points of the convolutions (the kernels live in conv_kernel.h and
// are compiled per storage type in conv_f32.hip, conv_f16.hip, conv_bf16.hip),
// and the weight transpose that feeds spc_conv_fwd_wt.
#include "conv_kernel.h"

namespace spc {
namespace {

spc_status run_conv(spc_dtype dt, ConvArgs& a, bool trans, hipStream_t stream) {
    if (a.n_rows == 0) return SPC_OK;
    const int64_t es = dt == SPC_F32 ? 4 : 2;
    a.xbuf = int64_t(a.n_src) * a.CK * es < (int64_t(1) << 31) && int64_t(a.K) * a.cin * a.cout * es < (int64_t(1) << 31);
    switch (dt) {
        case SPC_F32: return run_conv_f32(a, trans, stream);
        case SPC_F16: return run_conv_f16(a, trans, stream);
        case SPC_BF16: return run_conv_bf16(a, trans, stream);
    }
    return fail(SPC_ERR_ARG, "unknown dtype %d", int(dt));
}

// weight_t[k][n][c] = w[k][c][n]: one 32 x 32 block of one offset's matrix
// per workgroup, through an LDS tile padded against bank conflicts, so that
// both the reads and the writes run along rows
template <typename T>
__global__ __launch_bounds__(256) void k_transpose_w(const T* __restrict__ w, T* __restrict__ wt, int cin,
                                                     int cout) {
    __shared__ T t[32][33];
    const int64_t base = int64_t(blockIdx.z) * cin * cout;
    const int c0 = blockIdx.y * 32, n0 = blockIdx.x * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
#pragma unroll
    for (int i = ty; i < 32; i += 8)
        if (c0 + i < cin && n0 + tx < cout) t[i][tx] = w[base + int64_t(c0 + i) * cout + n0 + tx];
    __syncthreads();
#pragma unroll
    for (int i = ty; i < 32; i += 8)
        if (n0 + i < cout && c0 + tx < cin) wt[base + int64_t(n0 + i) * cin + c0 + tx] = t[tx][i];
}

spc_status check_common(spc_dtype dt, int64_t n_rows, int64_t n_src, int32_t cin, int32_t cout, int32_t K,
                        const void* x, const void* w, const float* bias, const void* y, const int32_t* map,
                        const int32_t* order, bool map_required) {
    if (dt != SPC_F32 && dt != SPC_F16 && dt != SPC_BF16) return fail(SPC_ERR_ARG, "unknown dtype %d", int(dt));
    if (n_rows < 0 || n_rows >= (int64_t(1) << 31) || n_src < 0 || n_src >= (int64_t(1) << 31))
        return fail(SPC_ERR_ARG, "row counts out of range");
    if (cin <= 0 || cout <= 0 || cin % 16 || cout % 16)
        return fail(SPC_ERR_UNSUPPORTED, "cin=%d cout=%d: channel counts must be positive multiples of 16", cin, cout);
    if (K <= 0 || K > 343) return fail(SPC_ERR_ARG, "K=%d must be in 1..343", K);
    if (n_rows > 0) {
        if (!w || !y) return fail(SPC_ERR_ARG, "weight or output pointer is NULL");
        if (n_src > 0 && !x) return fail(SPC_ERR_ARG, "input pointer is NULL");
        if (map_required && !map) return fail(SPC_ERR_ARG, "map is NULL");
    }
    const void* ptrs[] = {x, w, bias, y, map, order};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(SPC_ERR_ARG, "device pointers must be 16-byte aligned");
    return SPC_OK;
}

}  // namespace
}  // namespace spc

using namespace spc;

extern "C" spc_status spc_subm_conv_fwd(spc_dtype dtype, const void* feats, int64_t n, int32_t cin,
                                        const void* weight, int32_t K, int32_t cout, const float* bias,
                                        const int32_t* nbr, const int32_t* order, void* out, hipStream_t stream) {
    clear_error();
    spc_status st = check_common(dtype, n, n, cin, cout, K, feats, weight, bias, out, nbr, order, K != 1);
    if (st != SPC_OK) return st;
    // a 1x1x1 map is the identity: skip reading it
    ConvArgs a{feats, weight, bias, K == 1 ? nullptr : nbr, K == 1 ? nullptr : order, out, int32_t(n), int32_t(n),
               K, cin, cout, cin, cout, 0, 0};
    return run_conv(dtype, a, true, stream);
}

extern "C" spc_status spc_sparse_conv_fwd(spc_dtype dtype, const void* feats, int64_t n_in, int32_t cin,
                                          const void* weight, int32_t K, int32_t cout, const float* bias,
                                          const int32_t* nbr_out, const int32_t* order, int64_t n_out, void* out,
                                          hipStream_t stream) {
    clear_error();
    spc_status st = check_common(dtype, n_out, n_in, cin, cout, K, feats, weight, bias, out, nbr_out, order, true);
    if (st != SPC_OK) return st;
    ConvArgs a{feats, weight, bias, nbr_out, order, out, int32_t(n_out), int32_t(n_in), K, cin, cout, cin, cout, 0, 0};
    return run_conv(dtype, a, true, stream);
}

extern "C" spc_status spc_sparse_inverse_conv_fwd(spc_dtype dtype, const void* feats, int64_t n_coarse,
                                                  int32_t cin, const void* weight, int32_t K, int32_t cout,
                                                  const float* bias, const int32_t* nbr_in, const int32_t* order_in,
                                                  int64_t n_fine, void* out, hipStream_t stream) {
    clear_error();
    spc_status st = check_common(dtype, n_fine, n_coarse, cin, cout, K, feats, weight, bias, out, nbr_in, order_in,
                                 true);
    if (st != SPC_OK) return st;
    // the fine rows gather the coarse rows through the transposed map: the
    // same output-stationary kernel as the strided forward
    ConvArgs a{feats, weight, bias, nbr_in, order_in, out, int32_t(n_fine), int32_t(n_coarse), K, cin, cout, cin,
               cout, 0, 0};
    return run_conv(dtype, a, true, stream);
}

extern "C" spc_status spc_conv_fwd_fused(spc_dtype dtype, const void* feats, int64_t n_src, int32_t cin,
                                         const void* weight, int32_t K, int32_t cout, const float* bias,
                                         const int32_t* map, const int32_t* order, int64_t n_rows,
                                         const void* residual, int32_t relu, void* out, hipStream_t stream) {
    clear_error();
    const bool identity = K == 1 && map == nullptr;
    if (identity && n_src != n_rows)
        return fail(SPC_ERR_ARG, "an identity map needs n_src == n_rows (%lld vs %lld)", (long long)n_src,
                    (long long)n_rows);
    spc_status st = check_common(dtype, n_rows, n_src, cin, cout, K, feats, weight, bias, out, map, order, !identity);
    if (st != SPC_OK) return st;
    if (residual && !aligned16(residual)) return fail(SPC_ERR_ARG, "device pointers must be 16-byte aligned");
    ConvArgs a{feats, weight, bias, identity ? nullptr : map, identity ? nullptr : order, out, int32_t(n_rows),
               int32_t(n_src), K, cin, cout, cin, cout, 0, 0, residual, relu ? 1 : 0};
    return run_conv(dtype, a, true, stream);
}

extern "C" spc_status spc_transpose_weight(spc_dtype dtype, const void* weight, int32_t K, int32_t cin, int32_t cout,
                                           void* weight_t, hipStream_t stream) {
    clear_error();
    if (dtype != SPC_F32 && dtype != SPC_F16 && dtype != SPC_BF16) return fail(SPC_ERR_ARG, "unknown dtype %d", int(dtype));
    if (K <= 0 || K > 343 || cin <= 0 || cout <= 0 || cin > 65535 * 32 || cout > 2147483647 / 32)
        return fail(SPC_ERR_ARG, "K=%d cin=%d cout=%d out of range", K, cin, cout);
    if (!weight || !weight_t) return fail(SPC_ERR_ARG, "weight pointer is NULL");
    const size_t es = dtype == SPC_F32 ? 4 : 2;
    const size_t bytes = size_t(K) * size_t(cin) * size_t(cout) * es;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(weight), b0 = reinterpret_cast<uintptr_t>(weight_t);
    if (a0 < b0 + bytes && b0 < a0 + bytes) return fail(SPC_ERR_ARG, "weight and weight_t overlap");
    const dim3 grid(unsigned(ceil_div(cout, 32)), unsigned(ceil_div(cin, 32)), unsigned(K));
    if (es == 4)
        hipLaunchKernelGGL(k_transpose_w<uint32_t>, grid, dim3(256), 0, stream, static_cast<const uint32_t*>(weight),
                           static_cast<uint32_t*>(weight_t), cin, cout);
    else
        hipLaunchKernelGGL(k_transpose_w<uint16_t>, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(weight),
                           static_cast<uint16_t*>(weight_t), cin, cout);
    SPC_LAUNCHED("k_transpose_w");
    return SPC_OK;
}

extern "C" spc_status spc_conv_fwd_wt(spc_dtype dtype, const void* feats, int64_t n_src, int32_t cin,
                                      const void* weight_t, int32_t K, int32_t cout, const float* bias,
                                      const int32_t* map, int32_t map_is_subm, const int32_t* order, int64_t n_rows,
                                      const void* residual, int32_t relu, void* out, hipStream_t stream) {
    clear_error();
    const bool identity = K == 1 && map == nullptr;
    if (identity && n_src != n_rows)
        return fail(SPC_ERR_ARG, "an identity map needs n_src == n_rows (%lld vs %lld)", (long long)n_src,
                    (long long)n_rows);
    spc_status st =
        check_common(dtype, n_rows, n_src, cin, cout, K, feats, weight_t, bias, out, map, order, !identity);
    if (st != SPC_OK) return st;
    if (residual && !aligned16(residual)) return fail(SPC_ERR_ARG, "device pointers must be 16-byte aligned");
    // the dinput staging with the roles of the weight's dims exchanged:
    // slab entry B[kk][n] = weight_t[k][n][kk], a row of weight_t per output
    // channel, contraction-contiguous (weight dims: cout rows of cin)
    ConvArgs a{feats, weight_t, bias, identity ? nullptr : map, identity ? nullptr : order, out, int32_t(n_rows),
               int32_t(n_src), K, cin, cout, cout, cin, 0, 0, residual, relu ? 1 : 0};
    return run_conv(dtype, a, false, stream);
}

extern "C" spc_status spc_conv_bwd_input(spc_dtype dtype, const void* dout, int64_t n_out, int32_t cout,
                                         const void* weight, int32_t K, int32_t cin, const int32_t* map,
                                         int32_t map_is_subm, const int32_t* order, int64_t n_in, void* din,
                                         hipStream_t stream) {
    clear_error();
    const bool identity = (K == 1 && map == nullptr);
    spc_status st = check_common(dtype, n_in, n_out, cin, cout, K, dout, weight, nullptr, din, map, order, !identity);
    if (st != SPC_OK) return st;
    if ((map_is_subm || identity) && n_out != n_in)
        return fail(SPC_ERR_ARG, "submanifold dinput needs n_out == n_in (%lld vs %lld)", (long long)n_out, (long long)n_in);
    // din rows gather dout rows: contraction over cout, output channels cin
    ConvArgs a{dout, weight, nullptr, map, identity ? nullptr : order, din, int32_t(n_in), int32_t(n_out), K, cout,
               cin, cin, cout, map_is_subm ? 1 : 0, 0};
    return run_conv(dtype, a, false, stream);
}

extern "C" spc_status spc_conv_fwd_dev_rows(spc_dtype dtype, const void* feats, int64_t n_src, int32_t cin,
                                            const void* weight, int32_t weight_t, int32_t K, int32_t cout,
                                            const float* bias, const int32_t* map, const int32_t* order,
                                            int64_t row_cap, const int32_t* n_rows_dev, const void* residual,
                                            int32_t relu, void* out, hipStream_t stream) {
    clear_error();
    if (!n_rows_dev) return fail(SPC_ERR_ARG, "n_rows_dev is NULL");
    spc_status st = check_common(dtype, row_cap, n_src, cin, cout, K, feats, weight, bias, out, map, order, true);
    if (st != SPC_OK) return st;
    if (!aligned16(n_rows_dev) || (residual && !aligned16(residual)))
        return fail(SPC_ERR_ARG, "device pointers must be 16-byte aligned");
    // the forward over a strided map's output rows, whose count the map wrote
    // to n_rows_dev: W as it is (the spc_sparse_conv_fwd staging) or
    // pre-transposed by spc_transpose_weight (the spc_conv_fwd_wt staging)
    ConvArgs a = weight_t ? ConvArgs{feats, weight, bias, map, order, out, int32_t(row_cap), int32_t(n_src), K, cin,
                                     cout, cout, cin, 0, 0, residual, relu ? 1 : 0}
                          : ConvArgs{feats, weight, bias, map, order, out, int32_t(row_cap), int32_t(n_src), K, cin,
                                     cout, cin, cout, 0, 0, residual, relu ? 1 : 0};
    a.n_rows_dev = n_rows_dev;
    return run_conv(dtype, a, !weight_t, stream);
}
