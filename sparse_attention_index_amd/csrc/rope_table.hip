// rope_table.hip -- rotary cos/sin table on the GPU.
//
// Page "DeepSeek-V3.2-Exp . RoPE coefficients" (precompute_freqs_cis
// excerpt): frequencies theta_i = base^(-2i/64) held in float32, the YaRN
// blend freqs/factor*(1-smooth) + freqs*smooth beyond the original length,
// angles as the float32 product position*theta_i, table = (cos, sin).
// The ramp that defines `smooth` is not shown on the page; it is the linear
// ramp of the YaRN paper (Peng et al. 2023) between the correction dims
// low/high, which the host computes and passes in.
// Every transcendental is evaluated in double and rounded once to float32.
#include "dsa_common.h"

namespace dsa {

__global__ __launch_bounds__(256) void rope_table_kernel(int P, int npairs, double base,
                                                         int yarn, double low, double high,
                                                         double factor, float* __restrict__ cos_out,
                                                         float* __restrict__ sin_out) {
#pragma clang fp contract(off)
    const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= static_cast<int64_t>(P) * npairs) return;
    const int i = static_cast<int>(t % npairs);
    const int p = static_cast<int>(t / npairs);
    float f = static_cast<float>(pow(base, -(2.0 * i) / (2.0 * npairs)));
    if (yarn) {
        double ramp = (static_cast<double>(i) - low) / (high - low);
        ramp = ramp < 0.0 ? 0.0 : (ramp > 1.0 ? 1.0 : ramp);
        const double smooth = 1.0 - ramp;
        const double fd = static_cast<double>(f);
        const double a = fd / factor * (1.0 - smooth);
        const double b = fd * smooth;
        f = static_cast<float>(a + b);
    }
    const float ang = static_cast<float>(p) * f;
    cos_out[t] = static_cast<float>(cos(static_cast<double>(ang)));
    sin_out[t] = static_cast<float>(sin(static_cast<double>(ang)));
}

hipError_t launch_rope_table(int P, int npairs, double base, int yarn, double low, double high,
                             double factor, float* cos_out, float* sin_out, hipStream_t stream) {
    const int64_t n = static_cast<int64_t>(P) * npairs;
    const int threads = 256;
    const int64_t blocks = (n + threads - 1) / threads;
    hipLaunchKernelGGL(rope_table_kernel, dim3(static_cast<unsigned>(blocks)), dim3(threads), 0,
                       stream, P, npairs, base, yarn, low, high, factor, cos_out, sin_out);
    return hipGetLastError();
}

}  // namespace dsa
