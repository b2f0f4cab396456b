// One decode step of a causal depthwise 1-D convolution for one channel
// (MiniCPM-V 4.6 on Orange Pi AIPro post, third change: the causal-conv1d
// step of each decode iteration, there a vectorised step kernel).  Here it
// is also fused into the epilogue of the linear whose output it convolves,
// so the step costs no launch and no re-read of that output.
//
//   window = (state[c][0..W-2], x)  (oldest first)
//   pre    = bias[c] + sum_j w[c][j] * window[j]   (fp32, w fp16)
//   out[c] = silu ? pre / (1 + exp(-pre)) : pre
//   state[c] <- (window[1..W-1])
#pragma once

#include "wsg_common.hpp"

namespace wsg {

constexpr int kMaxConvWidth = 8;

__device__ __forceinline__ void conv_step(const ConvOut &cv, int64_t c, float x) {
    const int W = cv.W;
    auto *st = glob(cv.state + c * (W - 1));
    const auto *w = glob(cv.w + c * W);
    float win[kMaxConvWidth];
#pragma unroll
    for (int j = 0; j < kMaxConvWidth - 1; ++j)
        if (j < W - 1)
            win[j] = st[j];
    float pre = cv.bias ? *glob(cv.bias + c) : 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxConvWidth; ++j) {
        if (j < W) {
            const float v = j < W - 1 ? win[j] : x;
            pre = __builtin_fmaf((float)__builtin_bit_cast(_Float16, w[j]), v, pre);
        }
    }
#pragma unroll
    for (int j = 0; j < kMaxConvWidth - 1; ++j)
        if (j < W - 1)
            st[j] = j + 1 < W - 1 ? win[j + 1] : x;
    *glob(cv.out + c) = cv.silu ? pre / (1.0f + __expf(-pre)) : pre;
}

}  // namespace wsg
