// Top-k of an fp32 vector in the greedy token's order (argmax.hpp): the k
// largest values, larger first, NaN below every number, -0 equal to +0,
// lower index first among equals.  This widens the reduce of the sliced
// lm_head results that picks the next token (MiniCPM-V 4.6 on Orange Pi
// AIPro post, second change) to the k best candidates.
//
// Keys are unique (the index is part of the key), so "the next best" is the
// largest key below the last one taken.  Each wave picks the k best of its
// candidates (held in registers) by k rounds of a wavefront maximum under a
// moving threshold, with no barrier between rounds; after one barrier, the
// first wave picks the k best of the waves' results the same way.  A
// selection pass gives every workgroup 2048 candidates and writes its k best
// keys; passes repeat until one workgroup of 1024 threads (16 candidates per
// thread) picks the final k in order.  No atomics; the result does not
// depend on workgroup order.
#include <algorithm>

#include "argmax.hpp"

// Wavefront maximum from the ROCm device library (a DPP reduction over the
// active lanes; the result is returned to every lane).
extern "C" __device__ __attribute__((const)) unsigned long long __ockl_wfred_max_u64(unsigned long long);

namespace wsg {
namespace {

constexpr int kPerThread = 8;
constexpr int kChunk = kBlock * kPerThread;  // candidates per workgroup of a pass
constexpr int kFinalThreads = 1024;
constexpr int kFinalPerThread = 16;          // the final workgroup takes up to 16384 candidates
constexpr int kMaxK = 64;

// The k best of this wave's candidates c[0..E) per lane, in order, into
// res[0..k) (lane 0 writes).  All 64 lanes must be active.
template <int E>
__device__ __forceinline__ void wave_topk(const unsigned long long (&c)[E], int k, unsigned long long *res) {
    const int lane = threadIdx.x & (kWave - 1);
    unsigned long long thr = ~0ull;
    for (int r = 0; r < k; ++r) {
        unsigned long long best = 0ull;
#pragma unroll
        for (int j = 0; j < E; ++j)
            if (c[j] < thr)
                best = max_u64(best, c[j]);
        best = __ockl_wfred_max_u64(best);  // the wave's maximum, in every lane
        if (lane == 0)
            res[r] = best;
        thr = best;  // 0 once exhausted: every later key is 0 too
    }
}

// Per workgroup of WAVES waves: every wave picks its k best of E candidates
// per lane, then wave 0 picks the k best of the WAVES * k results (held as
// WAVES * k / 64 per lane, at most 16) into res[0..k).
template <int WAVES, int E>
__device__ __forceinline__ bool block_topk(const unsigned long long (&c)[E], int k, unsigned long long *res) {
    __shared__ unsigned long long wres[WAVES * kMaxK];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    wave_topk(c, k, wres + wave * kMaxK);
    __syncthreads();
    if (wave != 0)
        return false;
    constexpr int E2 = WAVES * kMaxK / kWave;
    unsigned long long c2[E2];
#pragma unroll
    for (int j = 0; j < E2; ++j) {
        const int i = lane + j * kWave;                // candidate i: wave i / k, rank i % k
        c2[j] = i < WAVES * k ? wres[(i / k) * kMaxK + i % k] : 0ull;
    }
    wave_topk(c2, k, res);
    return true;
}

// FROM_Y: candidates are y[0..count) (keys formed here); otherwise keys.
template <bool FROM_Y>
__global__ __launch_bounds__(kBlock) void topk_pass_kernel(const float *__restrict__ y,
                                                          const unsigned long long *__restrict__ in, int64_t count,
                                                          int k, unsigned long long *__restrict__ out) {
    const int64_t base = (int64_t)blockIdx.x * kChunk;
    unsigned long long c[kPerThread];
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
        const int64_t i = base + threadIdx.x + (int64_t)j * kBlock;
        c[j] = 0ull;
        if (i < count)
            c[j] = FROM_Y ? arg_key(y[i], i) : in[i];
    }
    __shared__ unsigned long long res[kMaxK];
    if (block_topk<kWavesPerBlock>(c, k, res)) {
        // wave 0 only: its lane-0 writes of res are visible to its own lanes
        if ((int)threadIdx.x < k)
            out[(int64_t)blockIdx.x * k + threadIdx.x] = res[threadIdx.x];
    }
}

__global__ __launch_bounds__(kFinalThreads) void topk_final_kernel(const unsigned long long *__restrict__ in,
                                                                  int64_t count, int k, int32_t *idx, float *val) {
    unsigned long long c[kFinalPerThread];
#pragma unroll
    for (int j = 0; j < kFinalPerThread; ++j) {
        const int64_t i = threadIdx.x + (int64_t)j * kFinalThreads;
        c[j] = i < count ? in[i] : 0ull;
    }
    __shared__ unsigned long long res[kMaxK];
    if (block_topk<kFinalThreads / kWave>(c, k, res)) {
        if ((int)threadIdx.x < k) {
            ArgOut a{};
            a.idx = idx;
            a.val = val;
            arg_write(a, res[threadIdx.x], threadIdx.x);
        }
    }
}

}  // namespace

// Candidate counts of the passes for (N, k): N, then ceil(count / 2048) * k
// until at most 16384 remain for the final workgroup.  Returns the number of
// keys the workspace must hold for the two ping-pong buffers.
int64_t topk_plan(int64_t N, int k, int64_t *max_keys, int *passes) {
    int64_t count = N, biggest = 0;
    int p = 0;
    while (count > (int64_t)kFinalThreads * kFinalPerThread || p == 0) {
        const int64_t next = (count + kChunk - 1) / kChunk * k;
        biggest = std::max(biggest, next);
        count = next;
        ++p;
        if (p > 8)
            break;
    }
    if (max_keys)
        *max_keys = biggest;
    if (passes)
        *passes = p;
    return count;
}

hipError_t launch_topk(const float *y, int64_t N, int k, int32_t *idx, float *val, unsigned long long *ws_a,
                       unsigned long long *ws_b, hipStream_t s) {
    int64_t count = N;
    const unsigned long long *in = nullptr;
    unsigned long long *out = ws_a;
    bool first = true;
    do {
        const int64_t blocks = (count + kChunk - 1) / kChunk;
        if (first)
            hipLaunchKernelGGL(topk_pass_kernel<true>, dim3((unsigned)blocks), dim3(kBlock), 0, s, y, nullptr, count, k,
                               out);
        else
            hipLaunchKernelGGL(topk_pass_kernel<false>, dim3((unsigned)blocks), dim3(kBlock), 0, s, nullptr, in, count,
                               k, out);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        count = blocks * k;
        in = out;
        out = (out == ws_a) ? ws_b : ws_a;
        first = false;
    } while (count > (int64_t)kFinalThreads * kFinalPerThread);
    hipLaunchKernelGGL(topk_final_kernel, dim3(1), dim3(kFinalThreads), 0, s, in, count, k, idx, val);
    return hipGetLastError();
}

}  // namespace wsg
