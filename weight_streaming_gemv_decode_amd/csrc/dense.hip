// Row-major weight streaming for M = 1: fp16 weights (fp32 accumulate via
// v_dot2_f32_f16), int8 weights x int8 activations (exact int32 via
// v_dot4_i32_i8), the same with fp16 activations quantised per token in the
// kernel, the on-device split-K reduce, and the HBM read probe.
//
// The product is the decode-step vector-matrix product of the MiniCPM-V 4.6
// on Orange Pi AIPro (Ascend 310B) post (baseline paragraph: M = 1; closing
// paragraph: the step is bound by streaming the weights from memory).  The
// int8 form is the W8A8 product of the vLLM Arm CPU optimisation post (INT8
// W8A8 section).  The split-K partials and their reduce follow the same
// MiniCPM-V post, second change (the lm_head cut into slices whose results
// are reduced; here on the device, in fixed slice order).
//
// Mapping onto gfx950.  A workgroup is 4 waves and owns one work unit: a
// tile of rows and one k-slice.  Each lane streams 16-byte vectors, lane l
// taking vectors l, l+64, ... of a row, so every wave-wide load instruction
// reads 1 KiB of contiguous weights.  A wave step covers R rows x CH vectors
// per lane; the next step's loads are issued before the current step is
// consumed (two register buffers), so each lane keeps up to 2*R*CH 16-byte
// loads in flight.  The activation slice is staged once per unit in LDS
// (read with ds_read_b128, shared by the R rows of a step).  Row sums are
// reduced across the wave with a halving exchange (R values per lane become
// one row per 64/R lanes in log2(64) lane-exchange stages), then written as
// y (and its fp16 copy), or as a partial that a second small kernel adds in
// slice order.
#include "argmax.hpp"
#include "conv1d.hpp"

#include <algorithm>

namespace wsg {
namespace {

template <bool NT>
__device__ __forceinline__ u32x4 load_w(const u32x4 *p) {
    if constexpr (NT)
        return __builtin_nontemporal_load(glob(p));
    else
        return *glob(p);
}

template <int KIND>
struct DenseOps;

template <>
struct DenseOps<kF16> {
    using Acc = float;
    __device__ static __forceinline__ float dot(u32x4 w, u32x4 x, float a) {
        a = __builtin_amdgcn_fdot2(as_h2(w.x), as_h2(x.x), a, false);
        a = __builtin_amdgcn_fdot2(as_h2(w.y), as_h2(x.y), a, false);
        a = __builtin_amdgcn_fdot2(as_h2(w.z), as_h2(x.z), a, false);
        a = __builtin_amdgcn_fdot2(as_h2(w.w), as_h2(x.w), a, false);
        return a;
    }
};

template <>
struct DenseOps<kW8A8> {
    using Acc = int32_t;
    __device__ static __forceinline__ int32_t dot(u32x4 w, u32x4 x, int32_t a) {
        a = __builtin_amdgcn_sdot4((int)w.x, (int)x.x, a, false);
        a = __builtin_amdgcn_sdot4((int)w.y, (int)x.y, a, false);
        a = __builtin_amdgcn_sdot4((int)w.z, (int)x.z, a, false);
        a = __builtin_amdgcn_sdot4((int)w.w, (int)x.w, a, false);
        return a;
    }
};

template <>
struct DenseOps<kW8A8D> : DenseOps<kW8A8> {};

// Per-token activation scale of fp16 x [nvec8 16-byte vectors]: s_x =
// max|x| / 127 in fp32, over the whole vector, by the whole workgroup (the
// same reading as the int4 W4A8 kernel: vLLM Arm CPU optimisation post,
// INT8 sections).  A maximum is order-free, so every workgroup that
// computes it gets the same bits.  Contains barriers.
// The largest |value| of 8 fp16 values.
__device__ __forceinline__ float absmax8(u32x4 h, float amax) {
    const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const f16x2 p = as_h2(hw[j]);
        amax = fmaxf(amax, fmaxf(fabsf((float)p[0]), fabsf((float)p[1])));
    }
    return amax;
}

// Maximum over the workgroup (contains barriers).
__device__ __forceinline__ float block_max_f32(float amax) {
    __shared__ float red[kWavesPerBlock];
#pragma unroll
    for (int i = 0; i < 6; ++i)
        amax = fmaxf(amax, xor_lane(amax, 32 >> i));
    if ((threadIdx.x & (kWave - 1)) == 0)
        red[threadIdx.x / kWave] = amax;
    __syncthreads();
    amax = red[0];
#pragma unroll
    for (int w = 1; w < kWavesPerBlock; ++w)
        amax = fmaxf(amax, red[w]);
    __syncthreads();  // red[] may be rewritten by the next call
    return amax;
}

__device__ __forceinline__ float dyn_scale(const u32x4 *x, int64_t nvec8) {
    float amax = 0.0f;
    constexpr int U = 4;  // loads in flight per thread
    for (int64_t v0 = threadIdx.x; v0 < nvec8; v0 += (int64_t)kBlock * U) {
        u32x4 h[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t v = v0 + (int64_t)u * kBlock;
            h[u] = v < nvec8 ? *glob(x + v) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            amax = absmax8(h[u], amax);
    }
    return block_max_f32(amax) / 127.0f;
}

// The 16 int8 codes of 16 fp16 values (lo: the first 8, hi: the next 8):
// clamp(rint(x / s_x), -127, 127) with IEEE fp32 division, ties to even
// (int8_codes; rsx = fp32(1 / s_x)); all zero when s_x = 0.  Byte b of the
// result is the code of element 16 v + b.
__device__ __forceinline__ u32x4 quantize16(u32x4 lo, u32x4 hi, float sx, float rsx) {
    const uint32_t hw[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    uint32_t out[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {  // four codes per output word keep few registers live
        const f16x2 p0 = as_h2(hw[2 * w]), p1 = as_h2(hw[2 * w + 1]);
        const float v[4] = {(float)p0[0], (float)p0[1], (float)p1[0], (float)p1[1]};
        int c[4] = {0, 0, 0, 0};
        if (sx != 0.0f)
            int8_codes(v, sx, rsx, c);
        out[w] = ((uint32_t)c[0] & 255u) | ((uint32_t)c[1] & 255u) << 8 | ((uint32_t)c[2] & 255u) << 16 |
                 ((uint32_t)c[3] & 255u) << 24;
    }
    return u32x4{out[0], out[1], out[2], out[3]};
}

// Sum R per-lane values over the 64 lanes of a wave.  Stage o (o = 32, 16,
// ...) pairs lane l with l^o: the lane with bit o set keeps the upper half
// of its remaining values and receives its partner's upper half, the other
// keeps the lower half; after log2(R) stages each lane carries one value of
// row lane / (64/R), and plain xor-butterflies finish the sum.  Lane
// r * (64/R) ends with the total of row r.
template <int R, typename T>
__device__ __forceinline__ T reduce_rows(T (&v)[R], int lane) {
    if constexpr (R >= 8) {
        const bool up = lane & 32;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            T keep = up ? v[i + 4] : v[i];
            T send = up ? v[i] : v[i + 4];
            v[i] = keep + xor_lane(send, 32);
        }
    }
    if constexpr (R >= 4) {
        constexpr int o = R >= 8 ? 16 : 32;
        const bool up = lane & o;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            T keep = up ? v[i + 2] : v[i];
            T send = up ? v[i] : v[i + 2];
            v[i] = keep + xor_lane(send, o);
        }
    }
    if constexpr (R >= 2) {
        constexpr int o = R >= 8 ? 8 : (R >= 4 ? 16 : 32);
        const bool up = lane & o;
        T keep = up ? v[1] : v[0];
        T send = up ? v[0] : v[1];
        v[0] = keep + xor_lane(send, o);
    }
    T s = v[0];
    // strides 32/R .. 1, counted by an affine index so the loop unrolls and
    // every exchange gets a constant stride
    constexpr int kSteps = R == 1 ? 6 : R == 2 ? 5 : R == 4 ? 4 : 3;
#pragma unroll
    for (int i = 0; i < kSteps; ++i)
        s += xor_lane(s, (32 / R) >> i);
    return s;
}

// Row `row` of y from its whole sum v (and acc_out, y16); sx is the
// activation scale of the dynamically quantised kind.  Returns y[row].
template <int KIND, typename Acc>
__device__ __forceinline__ float finish_row(const DenseLin &L, int64_t row, Acc v, float sx) {
    float yv;
    if constexpr (KIND == kF16) {
        yv = v;
    } else {
        if (L.acc_out)
            *glob(L.acc_out + row) = v;
        yv = ((float)v * *glob(L.w_scale + row)) * (KIND == kW8A8D ? sx : *glob(L.x_scale));
    }
    *glob(L.y + row) = yv;
    if (L.y16)
        *glob(L.y16 + row) = f16_bits(yv);
    return yv;
}

// Writes row `row`: y (S = 1) or its partial of slice s (S > 1; written
// through to the device's coherence point when the last unit of the row
// tile sums them, FUSED).
template <int KIND, bool FUSED, typename Acc>
__device__ __forceinline__ void store_row(const DenseLin &L, int s, int64_t row, Acc v, float sx) {
    if (L.S > 1) {
        auto *p = glob(static_cast<Acc *>(L.part) + (int64_t)s * L.N + row);
        if constexpr (FUSED)
            __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
            *p = v;
    } else {
        finish_row<KIND>(L, row, v, sx);
    }
}

// One work unit: rows of row tile `tile` over k slice s.  Returns the
// activation scale of the dynamically quantised kind (0 for the others).
template <int KIND, int R, int CH, bool NT, bool TAIL, bool FUSED = false, bool DYNEARLY = false>
__device__ __forceinline__ float dense_unit(const DenseLin &L, int tile, int s, u32x4 *xs) {
    using Ops = DenseOps<KIND>;
    using Acc = typename Ops::Acc;
    constexpr int CHUNK = kWave * CH;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);

    const int kv0 = s * L.kvs;
    const int nv = min(L.kvs, L.kvec - kv0);
    const int nchunk = (nv + CHUNK - 1) / CHUNK;
    const int64_t row0 = (int64_t)tile * L.tile_rows;
    const int rows = (int)min((int64_t)L.tile_rows, L.N - row0);
    const int64_t last_row = row0 + rows - 1;
    const int ngroups = (rows + R - 1) / R;
    const int mygroups = wave < ngroups ? (ngroups - 1 - wave) / kWavesPerBlock + 1 : 0;
    const int nsteps = mygroups * nchunk;

    auto load_step = [&](u32x4(&buf)[R][CH], int gi, int c) {
        // Row pointers are wave-uniform (scalar base); only the lane offset
        // lives in a vector register.
        const int64_t rbase = row0 + (int64_t)(wave + gi * kWavesPerBlock) * R;
        const int v0 = c * CHUNK;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const u32x4 *p = L.W + (min(rbase + r, last_row) * L.kvec + kv0 + v0);
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                if constexpr (TAIL) {
                    buf[r][j] = u32x4{0u, 0u, 0u, 0u};
                    if (v0 + j * kWave + lane < nv)
                        buf[r][j] = load_w<NT>(p + j * kWave + lane);
                } else {
                    buf[r][j] = load_w<NT>(p + j * kWave + lane);
                }
            }
        }
    };

    Acc acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        acc[r] = 0;
    float sx = 0.0f;  // kW8A8D: the activation scale

    auto consume = [&](const u32x4(&buf)[R][CH], int gi, int c) {
        u32x4 xv[CH];
#pragma unroll
        for (int j = 0; j < CH; ++j)
            xv[j] = xs[c * CHUNK + j * kWave + lane];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int j = 0; j < CH; ++j)
                acc[r] = Ops::dot(buf[r][j], xv[j], acc[r]);
        if (c == nchunk - 1) {
            Acc v = reduce_rows<R>(acc, lane);
            constexpr int span = kWave / R;
            if ((lane & (span - 1)) == 0) {
                const int64_t row = row0 + (int64_t)(wave + gi * kWavesPerBlock) * R + lane / span;
                if (row <= last_row) {
                    store_row<KIND, FUSED>(L, s, row, v, sx);
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r)
                acc[r] = 0;
        }
    };

    // Two orders of the unit's start, chosen by the size of a wave's step.
    // Late (the default): the first weight step goes out, then the
    // activation slice is staged in LDS; vector-memory loads retire in issue
    // order, so the staging waits for that step too, and the second step
    // goes out behind the barrier.  Early (steps of at most 4 KiB per wave,
    // the plain kinds): the slice's first vectors are loaded into registers
    // ahead of both weight steps, so the staging waits for them alone and
    // both steps are in flight across the barrier.  Measured on MI355X, early
    // makes the 2-row shapes faster when a row takes two or more steps (int8
    // 4096x14336: 10.8 vs 11.4 us; 2048x2048: 3.6-3.9 vs 3.9 us), and
    // slower where it does not (the dependent decode chain, whose linears
    // mostly take one step per row: 484 vs 469 us) and for the 8-row shapes
    // of the decode step and the lm_head (about 2%).
    constexpr bool kEarly = KIND != kW8A8D && R * CH <= 4;
    // Steps are (row group gi, chunk c) in order; a is the step in bufA.
    int ga = 0, ca = 0;
    auto next = [&](int &g, int &c) {
        if (++c == nchunk) {
            c = 0;
            ++g;
        }
    };
    u32x4 bufA[R][CH], bufB[R][CH];

    // The early order for fp16 activations quantised in the kernel
    // (DYNEARLY: a kernel of its own, for rows of 513..1024 code vectors,
    // which every thread holds 3 or 4 of): the row goes out first (every
    // thread loads a clamped, in-bounds index, so the loads carry no branch
    // and the wait for them does not include the weight loads behind them),
    // then four weight steps (a ring of four buffers, refilled four steps
    // ahead); the maximum, the scale and the codes are computed while the
    // weights are in flight.  Four steps measured faster than two (4096 x
    // 14336: 12.5-12.7 against 13.4 us) and than eight (14.6 us, 183
    // VGPRs).  Holding the row and the steps costs registers (119 against
    // 70), so shorter rows keep the late order, in the other kernel: there
    // it measured faster (int8 14336 x 4096: 11.8 against 12.8 us).
    constexpr int kDynHold = 4;
    constexpr int kDynDepth = 4;  // weight steps in flight
    if (DYNEARLY) {
        u32x4 h[kDynHold][2];
#pragma unroll
        for (int j = 0; j < kDynHold; ++j) {
            const int i = min(tid + j * kBlock, L.kvec - 1);  // a repeat does not change the maximum
            h[j][0] = *glob(L.x + 2 * i);
            h[j][1] = *glob(L.x + 2 * i + 1);
        }
        // four steps go out (a wave with fewer steps loads its first step
        // again): with no branch around them the waits for x below count
        // exactly the weight loads behind it
        auto step_gc = [&](int st, int &g, int &c) {
            const int q = st < nsteps ? st : 0;
            g = q / nchunk;
            c = q - g * nchunk;
        };
        u32x4 bufs[kDynDepth][R][CH];
#pragma unroll
        for (int j = 0; j < kDynDepth; ++j) {
            int g, c;
            step_gc(j, g, c);
            load_step(bufs[j], g, c);
        }
        __builtin_amdgcn_sched_barrier(0);  // every load is out before the maximum waits for x
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < kDynHold; ++j)
            amax = absmax8(h[j][1], absmax8(h[j][0], amax));
        sx = block_max_f32(amax) / 127.0f;
        const float rsx = 1.0f / sx;
        const bool write_codes = L.xq_out != nullptr && tile == 0;
        for (int i = nv + tid; i < nchunk * CHUNK; i += kBlock)
            xs[i] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < kDynHold; ++j) {
            const int i = tid + j * kBlock;
            if (i >= kv0 && i < kv0 + nv) {
                const u32x4 q = quantize16(h[j][0], h[j][1], sx, rsx);
                xs[i - kv0] = q;
                if (write_codes)
                    *glob(reinterpret_cast<u32x4 *>(L.xq_out) + i) = q;
            }
        }
        if (tile == 0 && s == 0 && tid == 0) {
            if (L.sx_out != nullptr)
                *glob(L.sx_out) = sx;
            if (L.sx_part != nullptr)
                *glob(L.sx_part) = sx;
        }
        __syncthreads();
        // a buffer is refilled with the step kDynDepth ahead once it is consumed
        for (int st = 0; st < nsteps; st += kDynDepth) {
#pragma unroll
            for (int j = 0; j < kDynDepth; ++j) {
                if (st + j >= nsteps)
                    break;
                int g, c;
                step_gc(st + j, g, c);
                consume(bufs[j], g, c);
                if (st + j + kDynDepth < nsteps) {
                    step_gc(st + j + kDynDepth, g, c);
                    load_step(bufs[j], g, c);
                }
            }
        }
        return sx;
    }

    if (kEarly && nchunk >= 2) {
        constexpr int kXHold = 4;  // activation vectors per thread loaded ahead
        const u32x4 *xg = L.x + kv0;
        const int nx = nchunk * CHUNK;
        u32x4 xh[kXHold];
#pragma unroll
        for (int j = 0; j < kXHold; ++j) {
            const int i = tid + j * kBlock;
            xh[j] = u32x4{0u, 0u, 0u, 0u};
            if (i < nv)
                xh[j] = *glob(xg + i);
        }
        int gb = 0, cb = 0;
        next(gb, cb);
        if (nsteps > 0)
            load_step(bufA, 0, 0);
        if (nsteps > 1)
            load_step(bufB, gb, cb);
#pragma unroll
        for (int j = 0; j < kXHold; ++j) {
            const int i = tid + j * kBlock;
            if (i < nx)
                xs[i] = xh[j];
        }
        for (int i = tid + kXHold * kBlock; i < nx; i += kBlock)
            xs[i] = i < nv ? *glob(xg + i) : u32x4{0u, 0u, 0u, 0u};
        __syncthreads();
        // a buffer is refilled with the step after next once it is consumed
        for (int st = 0; st < nsteps; st += 2) {
            consume(bufA, ga, ca);
            if (st + 2 < nsteps) {
                next(ga, ca);
                next(ga, ca);
                load_step(bufA, ga, ca);
            }
            if (st + 1 >= nsteps)
                break;
            consume(bufB, gb, cb);
            if (st + 3 < nsteps) {
                next(gb, cb);
                next(gb, cb);
                load_step(bufB, gb, cb);
            }
        }
        return sx;
    }

    if (nsteps > 0)
        load_step(bufA, 0, 0);
    if constexpr (KIND == kW8A8D) {
        // fp16 x quantised per token: the scale over the whole row, then the
        // codes of this slice into LDS (and to xq_out from the first row tile)
        const bool write_codes = L.xq_out != nullptr && tile == 0;
        auto put = [&](int i, u32x4 q) {  // code vector i of the row
            xs[i - kv0] = q;
            if (write_codes)
                *glob(reinterpret_cast<u32x4 *>(L.xq_out) + i) = q;
        };
        for (int i = nv + tid; i < nchunk * CHUNK; i += kBlock)
            xs[i] = u32x4{0u, 0u, 0u, 0u};
        constexpr int kHold = 4;  // code vectors per thread kept in registers
        if (L.kvec <= kHold * kBlock) {
            // one pass over x: each thread keeps its fp16 values for the codes
            u32x4 h[kHold][2];
            float amax = 0.0f;
#pragma unroll
            for (int j = 0; j < kHold; ++j) {
                const int i = tid + j * kBlock;
                h[j][0] = h[j][1] = u32x4{0u, 0u, 0u, 0u};
                if (i < L.kvec) {
                    h[j][0] = *glob(L.x + 2 * i);
                    h[j][1] = *glob(L.x + 2 * i + 1);
                }
            }
#pragma unroll
            for (int j = 0; j < kHold; ++j)
                amax = absmax8(h[j][1], absmax8(h[j][0], amax));
            sx = block_max_f32(amax) / 127.0f;
            const float rsx = 1.0f / sx;
#pragma unroll
            for (int j = 0; j < kHold; ++j) {
                const int i = tid + j * kBlock;
                if (i >= kv0 && i < kv0 + nv)
                    put(i, quantize16(h[j][0], h[j][1], sx, rsx));
            }
        } else {
            // a longer row: the scale from one pass over x, then the codes of
            // this slice from a second
            sx = dyn_scale(L.x, (int64_t)L.kvec * 2);
            const float rsx = 1.0f / sx;
            for (int i = kv0 + tid; i < kv0 + nv; i += kBlock)
                put(i, quantize16(*glob(L.x + 2 * i), *glob(L.x + 2 * i + 1), sx, rsx));
        }
        if (tile == 0 && s == 0 && tid == 0) {
            if (L.sx_out != nullptr)
                *glob(L.sx_out) = sx;
            if (L.sx_part != nullptr)
                *glob(L.sx_part) = sx;
        }
    } else {
        const u32x4 *xg = L.x + kv0;
        for (int i = tid; i < nchunk * CHUNK; i += kBlock)
            xs[i] = i < nv ? *glob(xg + i) : u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();

    if (nsteps == 0)
        return sx;
    int st = 0;
    while (st + 2 < nsteps) {
        int gb = ga, cb = ca;
        next(gb, cb);
        load_step(bufB, gb, cb);
        consume(bufA, ga, ca);
        int gn = gb, cn = cb;
        next(gn, cn);
        load_step(bufA, gn, cn);
        consume(bufB, gb, cb);
        ga = gn;
        ca = cn;
        st += 2;
    }
    if (st + 1 < nsteps) {
        int gb = ga, cb = ca;
        next(gb, cb);
        load_step(bufB, gb, cb);
        consume(bufA, ga, ca);
        consume(bufB, gb, cb);
    } else {
        consume(bufA, ga, ca);
    }
    return sx;
}

// The epilogues of a finished unit (S = 1) that read its rows of y back:
// the causal-conv1d step of each row, then the greedy-token key.  Nothing
// of them stays live in registers during the weight stream.
__device__ __forceinline__ void dense_after_unit(const DenseLin &L, int tile) {
    const int64_t r0 = (int64_t)tile * L.tile_rows;
    const int64_t nrows = min((int64_t)L.tile_rows, L.N - r0);
    if (L.conv.out != nullptr) {
        __syncthreads();  // the unit's stores of y are visible to the whole workgroup
        for (int64_t i = threadIdx.x; i < nrows; i += kBlock)
            conv_step(L.conv, r0 + i, *glob(L.y + r0 + i));
    }
    if (L.arg.keys != nullptr)
        publish_rows(L.arg, L.y, r0, nrows, tile);
}

// Split k summed by the last unit of each row tile to finish: every unit
// writes its partials with agent-scope stores (written through to the
// device's coherence point, where the other compute dies' L2 caches read
// them), waits until they are complete, then counts itself in on the
// tile's counter; the unit that counts last reads the S partials back with
// agent-scope loads and sums them in slice order (the reduce kernel's
// order, so the result is the same bits), then runs the epilogues.  The
// counter wraps to zero on the last arrival, ready for the next launch.
// (Ordering plain stores by agent-scope release and acquire fences instead
// writes back and invalidates the whole L2 per wave: 2.4 ms on the
// 248320x1024 lm_head, against 77 us.)
template <int KIND>
__device__ __forceinline__ void dense_last_arriver(const DenseLin &L, int tile, float sx) {
    using Acc = typename DenseOps<KIND>::Acc;
    __shared__ uint32_t s_old;
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const uint32_t last = (uint32_t)L.S - 1u;
    if (threadIdx.x == 0)
        s_old = __builtin_amdgcn_atomic_inc32(glob(L.ctr + tile), last, __ATOMIC_RELAXED, "agent");
    __syncthreads();
    if (s_old != last)
        return;
    const int64_t r0 = (int64_t)tile * L.tile_rows;
    const int nrows = (int)min((int64_t)L.tile_rows, L.N - r0);
    const Acc *p = static_cast<const Acc *>(L.part);
    for (int i = threadIdx.x; i < nrows; i += kBlock) {
        const int64_t n = r0 + i;
        Acc a = 0;
        for (int s = 0; s < L.S; ++s) {
            const auto *q = glob(p + (int64_t)s * L.N + n);
            const Acc v = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            a = s == 0 ? v : a + v;
        }
        finish_row<KIND>(L, n, a, sx);
    }
    if (L.arg.keys != nullptr || L.conv.out != nullptr)
        dense_after_unit(L, tile);
}

// FUSED (split linears whose last unit per row tile sums the partials) is
// a kernel of its own: the arrival code costs registers, and fewer resident
// waves make the plain kernel slower (82 against 71.5 us on the lm_head).
template <int KIND, int R, int CH, bool NT, bool TAIL, bool FUSED, bool DYNEARLY = false>
__global__ __launch_bounds__(kBlock) void dense_gemv_kernel(DenseLin L) {
    extern __shared__ u32x4 xs_dyn[];
    const int u = blockIdx.x;
    const float sx = dense_unit<KIND, R, CH, NT, TAIL, FUSED, DYNEARLY>(L, u / L.S, u % L.S, xs_dyn);
    if constexpr (FUSED) {
        dense_last_arriver<KIND>(L, u / L.S, sx);
    } else if (L.S == 1 && (L.arg.keys != nullptr || L.conv.out != nullptr)) {
        dense_after_unit(L, u);
    }
}

template <int KIND, int R, int CH, bool NT, bool TAIL>
__global__ __launch_bounds__(kBlock) void dense_grouped_kernel(const DenseLin *__restrict__ lins,
                                                               const Unit *__restrict__ units) {
    extern __shared__ u32x4 xs_dyn[];
    const Unit u = units[blockIdx.x];
    const DenseLin L = lins[u.lin];
    dense_unit<KIND, R, CH, NT, TAIL>(L, u.tile, u.s, xs_dyn);
    if (L.S == 1 && (L.arg.keys != nullptr || L.conv.out != nullptr))
        dense_after_unit(L, u.tile);
}

// y[n] = sum over slices s = 0..S-1, in that order, of part[s][n]; and the
// greedy token over y when the linear takes one.
template <int KIND>
__global__ __launch_bounds__(kBlock) void dense_reduce_kernel(DenseLin L) {
    const int64_t n = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    unsigned long long best = 0;
    float sx = 0.0f;
    if constexpr (KIND == kW8A8D)
        sx = *L.sx_part;  // published by the first work unit of the launch
    if (n < L.N) {
        using Acc = typename DenseOps<KIND>::Acc;
        const Acc *p = static_cast<const Acc *>(L.part);
        Acc a = p[n];
        for (int s = 1; s < L.S; ++s)
            a += p[(int64_t)s * L.N + n];
        const float yv = finish_row<KIND>(L, n, a, sx);
        best = arg_key(yv, n);
        if (L.conv.out != nullptr)
            conv_step(L.conv, n, yv);
    }
    if (L.arg.keys != nullptr)
        arg_publish(L.arg, best, blockIdx.x);
}

// ------------------------------------------------- persistent chain step --
//
// One cooperative launch runs a whole list of fp16 linears in which a linear
// may read (part of) an earlier linear's fp16 output.  Workgroup g runs work
// units g, g + G, ... (G = the grid) in list order, so a unit only ever waits
// for units of smaller index, all of which belong to resident workgroups.  A
// unit issues its first two weight steps, then waits for its input, stages it
// in LDS and streams the rest of its rows.  A producer publishes each output
// as the 32-bit word (tag << 16) | fp16 with an agent-scope atomic store; a
// consumer reads its input words with agent-scope atomic loads and takes a
// word only when its tag is the step's, polling again (after a tunable sleep)
// for the ones that are not yet current.  Every wait ends: after spin_limit
// polls, or once another workgroup has given up in this step, the unit goes
// on without its input and the give-up is counted for the host.

constexpr int kMaxChainVec = 512;  // largest input staged per unit, in 16-byte vectors (K <= 4096)

// 8 tagged words -> 8 fp16 (one LDS vector); true when every tag is `want`.
__device__ __forceinline__ bool poll_vec(const uint32_t *p, uint32_t want, u32x4 &out) {
    const auto *q = reinterpret_cast<const uint64_t *>(p);
    uint64_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        w[i] = __hip_atomic_load(glob(q + i), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool ok = true;
    uint32_t v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = (uint32_t)w[i], hi = (uint32_t)(w[i] >> 32);
        ok = ok && (lo >> 16) == want && (hi >> 16) == want;
        v[i] = (lo & 0xFFFFu) | (hi << 16);
    }
    out = u32x4{v[0], v[1], v[2], v[3]};
    return ok;
}

// The unit's input, vectors [0, nv) of L's input, into xs (zero up to nx).
// Contains barriers; on return xs is visible to the whole workgroup.
__device__ __forceinline__ void chain_stage(const ChainLin &L, const ChainArgs &a, int nv, int nx, u32x4 *xs) {
    const int tid = threadIdx.x;
    if (L.x_tag == nullptr) {
        for (int i = tid; i < nx; i += kBlock)
            xs[i] = i < nv ? *glob(L.x + i) : u32x4{0u, 0u, 0u, 0u};
        __syncthreads();
        return;
    }
    constexpr int kPer = kMaxChainVec / kBlock;
    __shared__ uint32_t s_stop[2];
    uint32_t pend = 0;  // bit j: vector tid + j * kBlock is not current yet
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = tid + j * kBlock;
        if (i < nv) {
            u32x4 v;
            if (poll_vec(L.x_tag + 8 * (int64_t)i, a.want, v))
                xs[i] = v;
            else
                pend |= 1u << j;
        } else if (i < nx) {
            xs[i] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    // While inputs are missing, only thread 0 polls: one input vector (a
    // different one per workgroup, so the pollers of one input spread over
    // its cache lines); the workgroup re-reads its missing vectors once that
    // probe is current.  Thread 0 also decides whether to stop waiting; its
    // decisions are read by all after the barrier (two slots, so the next
    // round's write cannot overtake a slow reader of this one).
    const int probe = (int)(((uint32_t)blockIdx.x * 2654435761u) % (uint32_t)nv);
    for (uint32_t it = 0;; ++it) {
        if (tid == 0) {
            uint32_t d = 0;
            if (it > 0) {
                u32x4 v;
                if (poll_vec(L.x_tag + 8 * (int64_t)probe, a.want, v))
                    d |= 2u;
                if (it >= a.spin_limit ||
                    __hip_atomic_load(&a.ctl->abort_epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.epoch)
                    d |= 1u;
            }
            s_stop[it & 1] = d;
        }
        if (!__syncthreads_or(pend != 0))
            return;
        const uint32_t d = s_stop[it & 1];
        if (d & 1u) {
            if (tid == 0) {
                __hip_atomic_fetch_add(&a.ctl->give_ups, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&a.ctl->abort_epoch, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            return;
        }
        for (int z = 0; z < a.sleep; ++z)
            __builtin_amdgcn_s_sleep(1);
        if (!(d & 2u))
            continue;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            if (pend & (1u << j)) {
                const int i = tid + j * kBlock;
                u32x4 v;
                if (poll_vec(L.x_tag + 8 * (int64_t)i, a.want, v)) {
                    xs[i] = v;
                    pend &= ~(1u << j);
                }
            }
        }
    }
}

// tr: the unit's trace record (four 64-bit words), or nullptr.
template <int R, int CH, bool TAIL>
__device__ __forceinline__ void chain_unit(const ChainLin &L, int tile, const ChainArgs &a, u32x4 *xs,
                                           uint64_t *tr) {
    using Ops = DenseOps<kF16>;
    constexpr int CHUNK = kWave * CH;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int nv = L.kvec;
    const int nchunk = (nv + CHUNK - 1) / CHUNK;
    const int64_t row0 = (int64_t)tile * L.tile_rows;
    const int rows = (int)min((int64_t)L.tile_rows, L.N - row0);
    const int64_t last_row = row0 + rows - 1;
    const int ngroups = (rows + R - 1) / R;
    const int mygroups = wave < ngroups ? (ngroups - 1 - wave) / kWavesPerBlock + 1 : 0;
    const int nsteps = mygroups * nchunk;

    auto load_step = [&](u32x4(&buf)[R][CH], int gi, int c) {
        const int64_t rbase = row0 + (int64_t)(wave + gi * kWavesPerBlock) * R;
        const int v0 = c * CHUNK;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const u32x4 *p = L.W + (min(rbase + r, last_row) * L.kvec + v0);
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                if constexpr (TAIL) {
                    buf[r][j] = u32x4{0u, 0u, 0u, 0u};
                    if (v0 + j * kWave + lane < nv)
                        buf[r][j] = load_w<true>(p + j * kWave + lane);
                } else {
                    buf[r][j] = load_w<true>(p + j * kWave + lane);
                }
            }
        }
    };

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        acc[r] = 0.0f;

    auto consume = [&](const u32x4(&buf)[R][CH], int gi, int c) {
        u32x4 xv[CH];
#pragma unroll
        for (int j = 0; j < CH; ++j)
            xv[j] = xs[c * CHUNK + j * kWave + lane];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int j = 0; j < CH; ++j)
                acc[r] = Ops::dot(buf[r][j], xv[j], acc[r]);
        if (c == nchunk - 1) {
            const float v = reduce_rows<R>(acc, lane);
            constexpr int span = kWave / R;
            if ((lane & (span - 1)) == 0) {
                const int64_t row = row0 + (int64_t)(wave + gi * kWavesPerBlock) * R + lane / span;
                if (row <= last_row) {
                    const uint16_t h = f16_bits(v);
                    *glob(L.y + row) = v;
                    if (L.y16)
                        *glob(L.y16 + row) = h;
                    if (L.tag_out)
                        __hip_atomic_store(glob(L.tag_out + row), (a.tag << 16) | h, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r)
                acc[r] = 0.0f;
        }
    };

    int ga = 0, ca = 0;
    auto next = [&](int &g, int &c) {
        if (++c == nchunk) {
            c = 0;
            ++g;
        }
    };
    u32x4 bufA[R][CH], bufB[R][CH];
    int gb = 0, cb = 0;
    next(gb, cb);
    // the weight loads go out before the wait for the input
    if (nsteps > 0)
        load_step(bufA, 0, 0);
    if (nsteps > 1)
        load_step(bufB, gb, cb);
    chain_stage(L, a, nv, nchunk * CHUNK, xs);
    if (tr != nullptr && threadIdx.x == 0)
        *glob(tr + 1) = __builtin_amdgcn_s_memrealtime();
    // a buffer is refilled with the step after next once it is consumed
    for (int st = 0; st < nsteps; st += 2) {
        consume(bufA, ga, ca);
        if (st + 2 < nsteps) {
            next(ga, ca);
            next(ga, ca);
            load_step(bufA, ga, ca);
        }
        if (st + 1 >= nsteps)
            break;
        consume(bufB, gb, cb);
        if (st + 3 < nsteps) {
            next(gb, cb);
            next(gb, cb);
            load_step(bufB, gb, cb);
        }
    }
}

// TRACE (a kernel of its own, so that the untraced kernel carries none of
// it): thread 0 records for unit u in a.trace, from the chip's 100 MHz
// real-time clock (one time base for every compute unit), when the workgroup
// starts the unit, when its input is staged, and when the whole workgroup
// has finished it (after a barrier that only tracing adds), then the unit's
// linear and workgroup.
template <int R, int CH, bool TAIL, bool TRACE>
__global__ __launch_bounds__(kBlock) void chain_kernel(ChainArgs a) {
    extern __shared__ u32x4 xs_dyn[];
    int k = 0;
    for (int u = blockIdx.x; u < a.n_units; u += gridDim.x, ++k) {
        const Unit un = a.units[u];
        const ChainLin L = a.lins[un.lin];
        uint64_t *tr = TRACE ? a.trace + 4 * (int64_t)u : nullptr;
        if (TRACE && threadIdx.x == 0)
            *glob(tr) = __builtin_amdgcn_s_memrealtime();
        chain_unit<R, CH, TAIL>(L, un.tile, a, xs_dyn + (k & 1) * a.xs_vecs, tr);
        if constexpr (TRACE) {
            __syncthreads();
            if (threadIdx.x == 0) {
                *glob(tr + 2) = __builtin_amdgcn_s_memrealtime();
                *glob(tr + 3) = (uint64_t)(uint32_t)un.lin | (uint64_t)blockIdx.x << 32;
            }
        }
    }
}

constexpr int kChainR = 2, kChainCH = 2;

__global__ __launch_bounds__(kBlock) void zero_f32_kernel(float *p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i < n)
        p[i] = 0.0f;
}

__global__ __launch_bounds__(kBlock) void zero_u16_kernel(uint16_t *p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i < n)
        p[i] = 0;
}

// The token from the key array: one workgroup of 1024 threads reduces
// a.keys[0..n_keys), each thread taking 8 consecutive keys (four 16-byte
// loads, all in flight together) per round.
constexpr int kFinishThreads = 1024;

// One workgroup per position m (blockIdx.x).
__global__ __launch_bounds__(kFinishThreads) void argmax_finish_kernel(ArgOut a) {
    const int n = a.n_keys, m = blockIdx.x;
    const unsigned long long *keys = a.keys + (int64_t)m * a.stride;
    unsigned long long best = 0;
    for (int base = threadIdx.x * 8; base < n; base += kFinishThreads * 8) {
        if (base + 8 <= n) {
            const u32x4 *p = reinterpret_cast<const u32x4 *>(keys + base);
            u32x4 v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[j] = p[j];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                best = max_u64(best, ((unsigned long long)v[j].y << 32) | v[j].x);
                best = max_u64(best, ((unsigned long long)v[j].w << 32) | v[j].z);
            }
        } else {
            for (int i = base; i < n; ++i)
                best = max_u64(best, keys[i]);
        }
    }
    best = block_max_key<kFinishThreads / kWave>(best);
    if (threadIdx.x == 0)
        arg_write(a, best, m);
}

// Greedy token over a given fp32 vector: at most kArgBlocks workgroups, each
// striding over the vector in kBlock-wide rows, then the finish kernel.  A
// thread issues the loads of kArgLoads rows before it folds any of them, so
// their latencies overlap.
constexpr int kArgBlocks = 1024;
constexpr int kArgLoads = 8;

__global__ __launch_bounds__(kBlock) void argmax_f32_kernel(const float *__restrict__ y, int64_t N, ArgOut a) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    unsigned long long best = 0;
    for (int64_t n0 = (int64_t)blockIdx.x * kBlock + threadIdx.x; n0 < N; n0 += kArgLoads * stride) {
        float v[kArgLoads];
#pragma unroll
        for (int j = 0; j < kArgLoads; ++j)
            v[j] = n0 + j * stride < N ? *glob(y + n0 + j * stride) : 0.0f;
#pragma unroll
        for (int j = 0; j < kArgLoads; ++j)
            if (n0 + j * stride < N)
                best = max_u64(best, arg_key(v[j], n0 + j * stride));
    }
    arg_publish(a, best, blockIdx.x);
}

// Read-only stream over buf, U 16-byte loads in flight per lane per
// iteration.  CHUNKED = false: grid-stride over the whole buffer; true: each
// workgroup reads one contiguous share.  The xor of everything read is
// folded per workgroup into out[blockIdx.x].
template <int U, bool NT, bool CHUNKED>
__global__ __launch_bounds__(kBlock) void read_probe_kernel(const u32x4 *__restrict__ buf, int64_t nvec,
                                                            float *out) {
    uint32_t acc = 0;
    int64_t begin = 0, end = nvec, first, stride;
    if constexpr (CHUNKED) {
        const int64_t share = (nvec + gridDim.x - 1) / gridDim.x;
        begin = min(nvec, (int64_t)blockIdx.x * share);
        end = min(nvec, begin + share);
        first = begin + threadIdx.x;
        stride = (int64_t)kBlock * U;
    } else {
        first = (int64_t)blockIdx.x * kBlock * U + threadIdx.x;
        stride = (int64_t)gridDim.x * kBlock * U;
    }
    for (int64_t base = first; base < end; base += stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + (int64_t)u * kBlock;
            v[u] = u32x4{0u, 0u, 0u, 0u};
            if (i < end)
                v[u] = load_w<NT>(buf + i);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (int o = 32; o >= 1; o >>= 1)
        acc ^= __shfl_xor(acc, o);
    __shared__ uint32_t red[kWavesPerBlock];
    if ((threadIdx.x & (kWave - 1)) == 0)
        red[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t a = 0;
        for (int w = 0; w < kWavesPerBlock; ++w)
            a ^= red[w];
        out[blockIdx.x] = (float)(a & 0xFFFFu);
    }
}

template <int U, bool NT, bool CHUNKED>
hipError_t launch_probe(const u32x4 *buf, int64_t nvec, float *out, int grid, hipStream_t s) {
    hipLaunchKernelGGL((read_probe_kernel<U, NT, CHUNKED>), dim3(grid), dim3(kBlock), 0, s, buf, nvec, out);
    return hipGetLastError();
}

template <int KIND, int R, int CH, bool NT, bool TAIL>
hipError_t launch_single(const DenseLin &L, hipStream_t s) {
    const int units = L.n_tiles * L.S;
    const int lds = dense_lds_bytes(L, CH);
    const bool fused = L.S > 1 && L.fuse;
    if constexpr (KIND == kW8A8D) {
        if (L.kvec > 2 * kBlock && L.kvec <= 4 * kBlock) {
            if (fused)
                hipLaunchKernelGGL((dense_gemv_kernel<KIND, R, CH, NT, TAIL, true, true>), dim3(units), dim3(kBlock),
                                   lds, s, L);
            else
                hipLaunchKernelGGL((dense_gemv_kernel<KIND, R, CH, NT, TAIL, false, true>), dim3(units),
                                   dim3(kBlock), lds, s, L);
            return hipGetLastError();
        }
    }
    if (fused)
        hipLaunchKernelGGL((dense_gemv_kernel<KIND, R, CH, NT, TAIL, true>), dim3(units), dim3(kBlock), lds, s, L);
    else
        hipLaunchKernelGGL((dense_gemv_kernel<KIND, R, CH, NT, TAIL, false>), dim3(units), dim3(kBlock), lds, s, L);
    return hipGetLastError();
}

template <int KIND, int R, int CH, bool NT, bool TAIL>
hipError_t launch_group(const DenseLin *lins, const Unit *units, int n_units, int lds, hipStream_t s) {
    hipLaunchKernelGGL((dense_grouped_kernel<KIND, R, CH, NT, TAIL>), dim3(n_units), dim3(kBlock), lds, s, lins,
                       units);
    return hipGetLastError();
}

// The instantiated (R, CH) shapes.  The host launch table only asks for
// these; anything else is rejected.
template <int KIND, bool NT, bool TAIL>
hipError_t dispatch_single(const DenseLin &L, const DenseCfg &c, hipStream_t s) {
    if (c.CH == 2) {
        if (c.R == 4) return launch_single<KIND, 4, 2, NT, TAIL>(L, s);
        if (c.R == 2) return launch_single<KIND, 2, 2, NT, TAIL>(L, s);
        if (c.R == 1) return launch_single<KIND, 1, 2, NT, TAIL>(L, s);
    } else if (c.CH == 1) {
        if (c.R == 8) return launch_single<KIND, 8, 1, NT, TAIL>(L, s);
        if (c.R == 4) return launch_single<KIND, 4, 1, NT, TAIL>(L, s);
    }
    return hipErrorInvalidValue;
}

template <int KIND, bool NT, bool TAIL>
hipError_t dispatch_group(const DenseLin *lins, const Unit *units, int n, int lds, const DenseCfg &c,
                          hipStream_t s) {
    if (c.CH == 2) {
        if (c.R == 4) return launch_group<KIND, 4, 2, NT, TAIL>(lins, units, n, lds, s);
        if (c.R == 2) return launch_group<KIND, 2, 2, NT, TAIL>(lins, units, n, lds, s);
    } else if (c.CH == 1) {
        if (c.R == 8) return launch_group<KIND, 8, 1, NT, TAIL>(lins, units, n, lds, s);
    }
    return hipErrorInvalidValue;
}

template <int KIND>
hipError_t single_kind(const DenseLin &L, const DenseCfg &c, hipStream_t s) {
    if (c.nt)
        return c.tail ? dispatch_single<KIND, true, true>(L, c, s) : dispatch_single<KIND, true, false>(L, c, s);
    return c.tail ? dispatch_single<KIND, false, true>(L, c, s) : dispatch_single<KIND, false, false>(L, c, s);
}

template <int KIND>
hipError_t group_kind(const DenseLin *lins, const Unit *units, int n, int lds, const DenseCfg &c, hipStream_t s) {
    if (c.nt)
        return c.tail ? dispatch_group<KIND, true, true>(lins, units, n, lds, c, s)
                      : dispatch_group<KIND, true, false>(lins, units, n, lds, c, s);
    return c.tail ? dispatch_group<KIND, false, true>(lins, units, n, lds, c, s)
                  : dispatch_group<KIND, false, false>(lins, units, n, lds, c, s);
}

}  // namespace

hipError_t launch_dense(int kind, const DenseLin &L, const DenseCfg &c, hipStream_t s) {
    if (kind == kF16)
        return single_kind<kF16>(L, c, s);
    if (kind == kW8A8)
        return single_kind<kW8A8>(L, c, s);
    if (kind == kW8A8D)
        return single_kind<kW8A8D>(L, c, s);
    return hipErrorInvalidValue;
}

hipError_t launch_dense_grouped(int kind, const DenseLin *lins, const Unit *units, int n_units, int lds_bytes,
                                const DenseCfg &c, hipStream_t s) {
    if (kind == kF16)
        return group_kind<kF16>(lins, units, n_units, lds_bytes, c, s);
    if (kind == kW8A8)
        return group_kind<kW8A8>(lins, units, n_units, lds_bytes, c, s);
    if (kind == kW8A8D)
        return group_kind<kW8A8D>(lins, units, n_units, lds_bytes, c, s);
    return hipErrorInvalidValue;
}

static const void *chain_fn(bool tail, bool trace) {
    if (trace)
        return tail ? reinterpret_cast<const void *>(&chain_kernel<kChainR, kChainCH, true, true>)
                    : reinterpret_cast<const void *>(&chain_kernel<kChainR, kChainCH, false, true>);
    return tail ? reinterpret_cast<const void *>(&chain_kernel<kChainR, kChainCH, true, false>)
                : reinterpret_cast<const void *>(&chain_kernel<kChainR, kChainCH, false, false>);
}

hipError_t launch_chain(const ChainArgs &a, int grid, int lds_bytes, bool tail, hipStream_t s) {
    ChainArgs args = a;
    void *kargs[] = {&args};
    return hipLaunchCooperativeKernel(chain_fn(tail, a.trace != nullptr), dim3(grid), dim3(kBlock), kargs,
                                      (unsigned)lds_bytes, s);
}

// The smaller of the plain and the traced kernel's occupancy, so that one
// grid fits either.
hipError_t chain_blocks_per_cu(int lds_bytes, bool tail, int *blocks) {
    int b[2] = {0, 0};
    for (int t = 0; t < 2; ++t) {
        const hipError_t e =
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&b[t], chain_fn(tail, t == 1), kBlock, (size_t)lds_bytes);
        if (e != hipSuccess)
            return e;
    }
    *blocks = std::min(b[0], b[1]);
    return hipSuccess;
}

int dense_reduce_blocks(int64_t N) { return (int)((N + kBlock - 1) / kBlock); }

hipError_t launch_dense_reduce(int kind, const DenseLin &L, hipStream_t s) {
    const int grid = dense_reduce_blocks(L.N);
    if (kind == kF16)
        hipLaunchKernelGGL(dense_reduce_kernel<kF16>, dim3(grid), dim3(kBlock), 0, s, L);
    else if (kind == kW8A8D)
        hipLaunchKernelGGL(dense_reduce_kernel<kW8A8D>, dim3(grid), dim3(kBlock), 0, s, L);
    else
        hipLaunchKernelGGL(dense_reduce_kernel<kW8A8>, dim3(grid), dim3(kBlock), 0, s, L);
    return hipGetLastError();
}

// Workgroups (and keys) of the reduce over a given vector: 16 values per
// thread, at most kArgBlocks.
int argmax_f32_blocks(int64_t N) {
    const int64_t b = (N + 16 * kBlock - 1) / (16 * kBlock);
    return (int)std::min<int64_t>(std::max<int64_t>(b, 1), kArgBlocks);
}

hipError_t launch_argmax_finish(const ArgOut &a, hipStream_t s) {
    hipLaunchKernelGGL(argmax_finish_kernel, dim3(a.M > 1 ? a.M : 1), dim3(kFinishThreads), 0, s, a);
    return hipGetLastError();
}

// The reduce over y then the finish; a.n_keys must equal argmax_f32_blocks(N).
hipError_t launch_argmax_f32(const float *y, int64_t N, ArgOut a, hipStream_t s) {
    hipLaunchKernelGGL(argmax_f32_kernel, dim3(a.n_keys), dim3(kBlock), 0, s, y, N, a);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? launch_argmax_finish(a, s) : e;
}

hipError_t launch_zero_f32(float *p, int64_t n, hipStream_t s) {
    if (n <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)((n + kBlock - 1) / kBlock)), dim3(kBlock), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_zero_u16(uint16_t *p, int64_t n, hipStream_t s) {
    if (n <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(zero_u16_kernel, dim3((unsigned)((n + kBlock - 1) / kBlock)), dim3(kBlock), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_read_probe(const u32x4 *buf, int64_t nvec, float *out, int grid, const ProbeCfg &c,
                             hipStream_t s) {
#define WSG_PROBE(Uv)                                                                              \
    if (c.U == Uv)                                                                                 \
        return c.nt ? (c.chunked ? launch_probe<Uv, true, true>(buf, nvec, out, grid, s)           \
                                 : launch_probe<Uv, true, false>(buf, nvec, out, grid, s))         \
                    : (c.chunked ? launch_probe<Uv, false, true>(buf, nvec, out, grid, s)          \
                                 : launch_probe<Uv, false, false>(buf, nvec, out, grid, s));
    WSG_PROBE(4)
    WSG_PROBE(8)
    WSG_PROBE(16)
#undef WSG_PROBE
    return hipErrorInvalidValue;
}

}  // namespace wsg
