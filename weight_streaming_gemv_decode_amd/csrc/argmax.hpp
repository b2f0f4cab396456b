// Greedy token choice fused into a producer kernel: every workgroup that
// writes some logits folds them into one 64-bit key and stores it in its own
// slot of a key array; a one-workgroup finish kernel, next on the stream,
// reduces the keys and writes the token.  No atomics: every launch rewrites
// all of its slots, and the result does not depend on workgroup order.
//
// This is the reduce of the lm_head's sliced results that picks the next
// token in the MiniCPM-V 4.6 on Orange Pi AIPro post (second change), kept
// on the device.  Order: logits compare as IEEE numbers (-0 equals +0), a
// NaN is below every number, and among equal values the lowest index wins.
//
// Key = (order-preserving 32-bit image of the value) << 32 | (~index), so
// the unsigned maximum of the keys is the largest value at its lowest index.
#pragma once

#include "wsg_common.hpp"

namespace wsg {

__device__ __forceinline__ unsigned long long arg_key(float v, int64_t index) {
    if (v == 0.0f)
        v = 0.0f;  // -0 and +0 are one value
    const uint32_t b = __builtin_bit_cast(uint32_t, v);
    uint32_t u = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    if (__builtin_isnan(v))
        u = 0u;
    return ((unsigned long long)u << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)index);
}

__device__ __forceinline__ unsigned long long max_u64(unsigned long long a, unsigned long long b) {
    return a > b ? a : b;
}

// The key of lane l ^ o (every lane of the wave active; o a power of two).
__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int o) {
    const uint32_t lo = xor_lane((uint32_t)v, o);
    const uint32_t hi = xor_lane((uint32_t)(v >> 32), o);
    return ((unsigned long long)hi << 32) | lo;
}

// Maximum key over a workgroup of WAVES waves (contains a barrier).
template <int WAVES = kWavesPerBlock>
__device__ __forceinline__ unsigned long long block_max_key(unsigned long long best) {
    __shared__ unsigned long long red[WAVES];
#pragma unroll
    for (int i = 0; i < 6; ++i)
        best = max_u64(best, shfl_xor_u64(best, (kWave / 2) >> i));
    const int tid = threadIdx.x;
    if ((tid & (kWave - 1)) == 0)
        red[tid / kWave] = best;
    __syncthreads();
    best = red[0];
#pragma unroll
    for (int w = 1; w < WAVES; ++w)
        best = max_u64(best, red[w]);
    __syncthreads();  // red[] may be rewritten by the next call
    return best;
}

// Called by every thread of the workgroup (it contains barriers), with the
// thread's best key for position m (0 when it holds no logit of that
// position); slot k of position m's key row receives the workgroup's best.
__device__ __forceinline__ void arg_publish(const ArgOut &a, unsigned long long best, int64_t k, int m = 0) {
    best = block_max_key(best);
    if (threadIdx.x == 0)
        *glob(a.keys + (int64_t)m * a.stride + k) = best;
}

// After a work unit has written rows [r0, r0 + nrows) of output row y (one
// position), the whole workgroup re-reads them and publishes their best key
// in slot k of position m.  Keeping no key in registers during the weight
// stream costs one barrier and a few L2 reads per unit.
__device__ __forceinline__ void publish_rows(const ArgOut &a, const float *y, int64_t r0, int64_t nrows,
                                             int64_t k, int m = 0) {
    __syncthreads();  // the unit's stores of y are visible to the whole workgroup
    unsigned long long best = 0;
    for (int64_t i = threadIdx.x; i < nrows; i += kBlock)
        best = max_u64(best, arg_key(*glob(y + r0 + i), r0 + i));
    arg_publish(a, best, k, m);
}

// The token of position m from its best key (written by the finish kernel).
__device__ __forceinline__ void arg_write(const ArgOut &a, unsigned long long key, int m) {
    const uint32_t u = (uint32_t)(key >> 32);
    const uint32_t bits = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
    a.idx[m] = (int32_t)(0xFFFFFFFFu - (uint32_t)key);
    if (a.val)
        a.val[m] = __builtin_bit_cast(float, bits);
}

}  // namespace wsg
