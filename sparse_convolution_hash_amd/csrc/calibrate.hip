// Measurement support: the dense MFMA issue rate of this part, for the
// roofline the convolutions are reported against.  Each wave runs
// independent accumulator chains of one MFMA shape on register operands (no
// memory traffic inside the loop); the caller times the launch.  This file is
// built with the accumulators in VGPRs (build.py): in AGPRs the compiler
// shuffles the chains between registers every round.
#include "common.h"

namespace spc {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// CH independent chains of v_mfma_f32_16x16x32_bf16 (shape 0) or
// v_mfma_f32_32x32x16_bf16 (shape 1); one float per thread to `sink` keeps
// the work alive.
template <int SHAPE, int CH>
__global__ __launch_bounds__(256) void k_mfma_rate(float* __restrict__ sink, int iters) {
    bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = __bf16(float(threadIdx.x & 7) * 0.125f + float(i));
        b[i] = __bf16(float(i) * 0.5f);
    }
    float s = 0.f;
    if constexpr (SHAPE == 0) {
        f32x4_t acc[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int c = 0; c < CH; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
#pragma unroll
        for (int c = 0; c < CH; ++c) s += acc[c][0] + acc[c][3];
    } else {
        f32x16_t acc[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int c = 0; c < CH; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
#pragma unroll
        for (int c = 0; c < CH; ++c) s += acc[c][0] + acc[c][15];
    }
    sink[int64_t(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

}  // namespace
}  // namespace spc

using namespace spc;

extern "C" spc_status spc_calibrate_mfma(int32_t shape, int32_t blocks, int32_t iters, float* sink,
                                         double* flop, hipStream_t stream) {
    clear_error();
    if (shape != 0 && shape != 1) return fail(SPC_ERR_ARG, "shape=%d must be 0 (16x16x32) or 1 (32x32x16)", shape);
    if (blocks <= 0 || blocks > 65536 || iters <= 0) return fail(SPC_ERR_ARG, "blocks=%d iters=%d", blocks, iters);
    if (!sink || !aligned16(sink)) return fail(SPC_ERR_ARG, "sink must be a 16-byte aligned device pointer");
    if (shape == 0)
        hipLaunchKernelGGL((k_mfma_rate<0, 8>), dim3(unsigned(blocks)), dim3(256), 0, stream, sink, iters);
    else
        hipLaunchKernelGGL((k_mfma_rate<1, 4>), dim3(unsigned(blocks)), dim3(256), 0, stream, sink, iters);
    SPC_LAUNCHED("k_mfma_rate");
    // per wave: CH chains x iters MFMAs of 2*M*N*K FLOP (8 x 16x16x32 or 4 x 32x32x16)
    const double per_wave = shape == 0 ? 8.0 * 2 * 16 * 16 * 32 : 4.0 * 2 * 32 * 32 * 16;
    if (flop) *flop = per_wave * double(iters) * double(blocks) * 4.0;
    return SPC_OK;
}
