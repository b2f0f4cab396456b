// Top-k of an fp32 vector in the greedy token's order (argmax.hpp): the k
// largest values, larger first, NaN below every number, -0 equal to +0,
// lower index first among equals.  This widens the reduce of the sliced
// lm_head results that picks the next token (MiniCPM-V 4.6 on Orange Pi
// AIPro post, second change) to the k best candidates.
//
// Keys are unique (the index is part of the key), so the top k are exactly
// the keys at or above the k-th largest.  A workgroup finds that key by a
// radix select on its 64-bit keys, one byte at a time from the top: a
// histogram of the current byte over the keys that share the bytes already
// fixed (shared-memory atomic adds), then the bin that holds the k-th
// largest; it stops early once that bin holds exactly the keys still
// needed.  The keys at or above it are gathered and one wave sorts them
// (bitonic, through lane exchanges).  A selection pass gives every
// workgroup 2048 candidates and writes its k best keys; passes repeat until
// one workgroup of 1024 threads (16 candidates per thread) picks the final
// k in order.  No global atomics; the result does not depend on workgroup
// order.
#include <algorithm>

#include "argmax.hpp"

namespace wsg {
namespace {

constexpr int kPerThread = 8;
constexpr int kChunk = kBlock * kPerThread;  // candidates per workgroup of a pass
constexpr int kFinalThreads = 1024;
constexpr int kFinalPerThread = 16;          // the final workgroup takes up to 16384 candidates
constexpr int kMaxK = 64;

// The k largest of the workgroup's candidates (E per thread, 0 = none), in
// descending order, into res[0..k) (shared memory; zeros when fewer than k
// candidates are nonzero).  Every thread must call it.  Zero keys never
// enter a histogram, so padding costs nothing.
template <int THREADS, int E>
__device__ __forceinline__ void block_select(const unsigned long long (&c)[E], int k, unsigned long long *res) {
    __shared__ uint32_t hist[2][256];  // this round's histogram and the next one's, zeroed ahead
    __shared__ unsigned long long s_prefix;
    __shared__ int s_need, s_done, s_count;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    if (tid == 0) {
        s_prefix = 0ull;
        s_need = k;
        s_done = 0;
        s_count = 0;
    }
    for (int i = tid; i < 2 * 256; i += THREADS)
        hist[i >> 8][i & 255] = 0u;
    __syncthreads();
    for (int d = 7; d >= 0 && !s_done; --d) {
        uint32_t *h_cur = hist[d & 1], *h_next = hist[(d + 1) & 1];
        const unsigned long long prefix = s_prefix;
        const int hi_shift = 8 * (d + 1);
#pragma unroll
        for (int j = 0; j < E; ++j) {
            // zero keys are padding (no candidate): they stay out of the histograms
            const bool match = c[j] != 0ull && (d == 7 || (c[j] >> hi_shift) == (prefix >> hi_shift));
            if (match)
                atomicAdd(&h_cur[(c[j] >> (8 * d)) & 255u], 1u);
        }
        __syncthreads();
        if (tid < kWave) {
            // lane l owns bins 255 - 4l .. 252 - 4l; find the bin holding the need-th largest
            uint32_t h[4], t = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                h[q] = h_cur[255 - 4 * lane - q];
                t += h[q];
            }
            uint32_t above = t;  // inclusive scan over lanes (higher bins first)
            for (int o = 1; o < kWave; o <<= 1) {
                const uint32_t v = __shfl_up(above, o);
                if (lane >= o)
                    above += v;
            }
            above -= t;  // keys in bins above this lane's
            const uint32_t need = (uint32_t)s_need;
            if (d == 7 && lane == kWave - 1 && above + t < need) {
                // fewer than k candidates in all: every one of them is taken
                s_prefix = 0ull;
                s_done = 1;
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (above < need && need <= above + h[q]) {
                    const uint32_t bin = 255u - 4u * lane - q;
                    s_prefix = prefix | ((unsigned long long)bin << (8 * d));
                    s_need = (int)(need - above);
                    s_done = h[q] == need - above;  // every key of the bin is needed
                }
                above += h[q];
            }
        } else {
            for (int i = tid - kWave; i < 256; i += THREADS - kWave)
                h_next[i] = 0u;
        }
        __syncthreads();
    }
    // the threshold: s_prefix with the bytes below the last fixed one at zero
    // (when the search ended early) is at or below exactly the k largest
    const unsigned long long thr = s_prefix;
    __shared__ unsigned long long sel[kMaxK];
    if (tid < kMaxK)
        sel[tid] = 0ull;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < E; ++j) {
        if (c[j] != 0ull && c[j] >= thr) {
            const int pos = atomicAdd(&s_count, 1);
            if (pos < kMaxK)
                sel[pos] = c[j];
        }
    }
    __syncthreads();
    if (tid < kWave) {
        // bitonic sort of the 64 gathered keys, descending, one per lane
        unsigned long long v = sel[lane];
        for (int size = 2; size <= kWave; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                const unsigned long long o = shfl_xor_u64(v, stride);
                const bool lower = (lane & stride) == 0;
                const bool desc = (lane & size) == 0;   // direction of this lane's sequence
                const bool take_max = lower == desc;
                v = take_max ? max_u64(v, o) : (v < o ? v : o);
            }
        }
        if (lane < k)
            res[lane] = v;
    }
    __syncthreads();
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
    block_select<kBlock>(c, k, res);
    if ((int)threadIdx.x < k)
        out[(int64_t)blockIdx.x * k + threadIdx.x] = res[threadIdx.x];
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
    block_select<kFinalThreads>(c, k, res);
    if ((int)threadIdx.x < k) {
        ArgOut a{};
        a.idx = idx;
        a.val = val;
        arg_write(a, res[threadIdx.x], threadIdx.x);
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
