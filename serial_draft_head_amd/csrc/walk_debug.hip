// walk_debug.hip -- diagnostics kernels: the Gumbel-max variate of every noise
// word the walk kernels can draw, for a test of its error against binary64.
#include "walk_device.h"

namespace dsw {

// out[i] = gumbel_of_word(i << 9) for i < 2^23: word i << 9 maps to
// U = (2 i + 1) 2^-24, so the table covers every U the noise can take.
__global__ void __launch_bounds__(256) gumbel_table_kernel(float* out) {
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    out[i] = gumbel_of_word(i << 9);
}

}  // namespace dsw

extern "C" int dsw_internal_gumbel_table(float* out, void* stream) {
    hipLaunchKernelGGL(dsw::gumbel_table_kernel, dim3((1u << 23) / 256u), dim3(256), 0,
                       static_cast<hipStream_t>(stream), out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}
