// The F32 variants of the fused convolution kernel (conv_kernel.h).
#define SPC_CONV_KERNELS
#include "conv_kernel.h"

namespace spc {

spc_status run_conv_f32(ConvArgs& a, bool trans, hipStream_t stream) {
    return trans ? launch_conv_t<F32, true>(a, stream) : launch_conv_t<F32, false>(a, stream);
}

}  // namespace spc
