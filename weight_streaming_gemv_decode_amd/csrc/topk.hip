// Top-k of an fp32 vector in the greedy token's order (argmax.hpp): the k
// largest values, larger first, NaN below every number, -0 equal to +0,
// lower index first among equals.  This widens the reduce of the sliced
// lm_head results that picks the next token (MiniCPM-V 4.6 on Orange Pi
// AIPro post, second change) to the k best candidates.
//
// Keys are unique (the index is part of the key), so the top k are exactly
// the keys at or above the k-th largest.  A selection pass gives every
// workgroup 1024 candidates; the workgroup finds the k-th largest by a radix
// select on the 64-bit keys, one byte at a time from the top (a histogram of
// the current byte over the keys that share the bytes already fixed, in
// shared memory, then the bin that holds the k-th largest; it stops early
// once that bin holds exactly the keys still needed), gathers the keys at or
// above it, and one wave sorts them (bitonic, through lane exchanges).  Each
// workgroup writes its k best keys as a sorted list.  Passes repeat until at
// most 256 lists remain.  The merge then runs in two launches when more than
// 16 lists remain: workgroups of 16 waves merge 32 lists each (two per wave)
// on their own compute units, and one workgroup merges their results.  Two sorted lists
// of 64 merge in one wave as the lane-wise maximum of one list and the other
// reversed (the 64 largest of both, in bitonic order) followed by six
// exchange stages.  No global atomics; the result does not depend on
// workgroup order.
#include <algorithm>

#include "argmax.hpp"

namespace wsg {
namespace {

constexpr int kPerThread = 4;
constexpr int kChunk = kBlock * kPerThread;  // candidates per workgroup of a pass
constexpr int kMergeWaves = 16;              // waves of the merging workgroup
constexpr int kMergeLists = 256;             // most sorted lists the merge takes
constexpr int kListsPerWave = kMergeLists / kMergeWaves;
constexpr int kGroupLists = 2 * kMergeWaves;    // lists per workgroup of a first merge launch
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
#pragma unroll
        for (int ls = 1; ls <= 6; ++ls) {  // sequences of size 2^ls
            const int size = 1 << ls;
#pragma unroll
            for (int j = 1; j <= ls; ++j) {
                const int stride = size >> j;
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

// The key of lane 63 - l: reversed within each 16-lane row, then rows
// swapped across (xor 48).
__device__ __forceinline__ unsigned long long mirror_u64(unsigned long long v) {
    uint32_t lo = __builtin_amdgcn_mov_dpp((uint32_t)v, 0x140, 0xF, 0xF, false);  // row_mirror
    uint32_t hi = __builtin_amdgcn_mov_dpp((uint32_t)(v >> 32), 0x140, 0xF, 0xF, false);
    lo = xor_lane(xor_lane(lo, 32), 16);
    hi = xor_lane(xor_lane(hi, 32), 16);
    return ((unsigned long long)hi << 32) | lo;
}

// Lane l's key of the 64 largest of two descending lists held one key per
// lane (v, b), in descending order.  b reversed is ascending, so the
// lane-wise maximum holds the 64 largest of both in bitonic order; a bitonic
// merge (lower lane takes the larger) sorts it.
__device__ __forceinline__ unsigned long long merge64(unsigned long long v, unsigned long long b, int lane) {
    v = max_u64(v, mirror_u64(b));
#pragma unroll
    for (int i = 0; i < 6; ++i) {
        const int stride = (kWave / 2) >> i;
        const unsigned long long o = shfl_xor_u64(v, stride);
        v = (lane & stride) ? (v < o ? v : o) : max_u64(v, o);
    }
    return v;
}

// The k largest keys of sorted lists (list l = in[l k .. l k + k),
// descending, zero-padded), in descending order.  Workgroup g takes lists
// [g per_wg, min(lists, (g + 1) per_wg)): every wave merges its share of them
// (all loaded first), then the waves' results are merged pairwise through
// shared memory.  The result goes to out[g k .. g k + k) as a sorted list
// when out is given, else (one workgroup) as the token rule's indices and
// values.
__global__ __launch_bounds__(kMergeWaves * kWave) void topk_merge_kernel(const unsigned long long *__restrict__ in,
                                                                        int lists, int per_wg, int k,
                                                                        unsigned long long *out, int32_t *idx,
                                                                        float *val) {
    __shared__ unsigned long long part[kMergeWaves][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int first = blockIdx.x * per_wg;
    const int last = min(lists, first + per_wg);
    unsigned long long b[kListsPerWave];
#pragma unroll
    for (int j = 0; j < kListsPerWave; ++j) {
        const int l = first + wave + j * kMergeWaves;
        b[j] = (l < last && lane < k) ? *glob(in + (int64_t)l * k + lane) : 0ull;
    }
    unsigned long long v = b[0];  // one list is sorted already
#pragma unroll
    for (int j = 1; j < kListsPerWave; ++j)
        if (first + wave + j * kMergeWaves < last)  // wave-uniform
            v = merge64(v, b[j], lane);
    // waves at or above `have` hold no list: the pairwise rounds start at the
    // smallest power of two that covers the ones that do
    const int have = min(last - first, kMergeWaves);
    int top = 1;
    while (top < have)
        top <<= 1;
    part[wave][lane] = v;
    for (int half = top / 2; half > 0; half >>= 1) {
        __syncthreads();
        if (wave < half)
            v = merge64(part[wave][lane], part[wave + half][lane], lane);
        __syncthreads();
        if (wave < half)
            part[wave][lane] = v;
    }
    if (wave == 0 && lane < k) {
        if (out != nullptr) {
            *glob(out + (int64_t)blockIdx.x * k + lane) = v;
        } else {
            ArgOut a{};
            a.idx = idx;
            a.val = val;
            arg_write(a, v, lane);
        }
    }
}

}  // namespace

// The selection passes for (N, k): each turns `count` candidates into one
// sorted list of k per 1024, until at most 256 lists remain for the merge.
// Returns the number of lists left; *max_keys is the most keys one pass
// writes (each of the two ping-pong buffers must hold that many).
int64_t topk_plan(int64_t N, int k, int64_t *max_keys, int *passes) {
    int64_t count = N, biggest = 0, lists = 0;
    int p = 0;
    do {
        lists = (count + kChunk - 1) / kChunk;
        count = lists * k;
        biggest = std::max(biggest, count);
        ++p;
    } while (lists > kMergeLists && p < 8);
    if (max_keys)
        *max_keys = biggest;
    if (passes)
        *passes = p;
    return lists;
}

hipError_t launch_topk(const float *y, int64_t N, int k, int32_t *idx, float *val, unsigned long long *ws_a,
                       unsigned long long *ws_b, hipStream_t s) {
    int passes = 0;
    topk_plan(N, k, nullptr, &passes);
    int64_t count = N, lists = 0;
    const unsigned long long *in = nullptr;
    unsigned long long *out = ws_a;
    for (int p = 0; p < passes; ++p) {
        lists = (count + kChunk - 1) / kChunk;
        if (p == 0)
            hipLaunchKernelGGL(topk_pass_kernel<true>, dim3((unsigned)lists), dim3(kBlock), 0, s, y, nullptr, count,
                               k, out);
        else
            hipLaunchKernelGGL(topk_pass_kernel<false>, dim3((unsigned)lists), dim3(kBlock), 0, s, nullptr, in,
                               count, k, out);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        count = lists * k;
        in = out;
        out = (out == ws_a) ? ws_b : ws_a;
    }
    if (lists > kMergeWaves) {
        // two lists per wave on several compute units; the other ping-pong
        // buffer (room for at least lists * k keys) takes the groups' lists
        const int groups = (int)((lists + kGroupLists - 1) / kGroupLists);
        hipLaunchKernelGGL(topk_merge_kernel, dim3(groups), dim3(kMergeWaves * kWave), 0, s, in, (int)lists,
                           kGroupLists, k, out, nullptr, nullptr);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        in = out;
        lists = groups;
    }
    hipLaunchKernelGGL(topk_merge_kernel, dim3(1), dim3(kMergeWaves * kWave), 0, s, in, (int)lists, kMergeLists, k,
                       nullptr, idx, val);
    return hipGetLastError();
}

}  // namespace wsg
