// Standalone causal-conv1d decode step over a given fp32 input (the step
// itself is in conv1d.hpp, shared with the fused GEMV epilogue): one thread
// per channel.
#include "conv1d.hpp"

namespace wsg {
namespace {

__global__ __launch_bounds__(kBlock) void conv1d_step_kernel(const float *__restrict__ x, ConvOut cv, int64_t C) {
    const int64_t c = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (c < C)
        conv_step(cv, c, x[c]);
}

}  // namespace

hipError_t launch_conv1d_step(const float *x, const ConvOut &cv, int64_t C, hipStream_t s) {
    if (C <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(conv1d_step_kernel, dim3((unsigned)((C + kBlock - 1) / kBlock)), dim3(kBlock), 0, s, x, cv,
                       C);
    return hipGetLastError();
}

}  // namespace wsg
