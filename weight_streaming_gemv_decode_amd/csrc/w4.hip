// INT4 weights x fp16 activations with the dequantisation fused into the
// product, for the decode product (M = 1, VALU) and a speculative-verify
// block (M = 2..8, MFMA), plus the load-time packer.
//
// Sources: MiniCPM-V 4.6 on Orange Pi AIPro (Ascend 310B) post, closing
// paragraph (fused INT4 dequantisation is the next lever once the step is
// bound by streaming weights); vLLM Arm CPU optimisation post, INT8 W4A8
// section (4-bit weights cut memory traffic) and dense-weight prepacking
// section (weights packed into the kernel's layout once at warm-up); EdgeFM
// summary, section 2C (a drafted block of tokens verified by the base model
// against the same weights).
//
// Weight value: w[n,k] = (q[n,k] - 8) * s[n, k/128], q in 0..15.
//
// Packed layout (one layout for both kernels).  Rows are cut into 16-row
// tiles and k into 128-wide blocks (one scale group).  Tile (t, b) is 1 KiB:
// lane l = r + 16 g (r = l % 16, g = l / 16) holds four 32-bit words; word i
// carries the 8 weights k = 128 b + 32 i + 8 g + (0..7) of row 16 t + r.
// Inside a word, weight j sits in 4-bit field (j >> 1) + 4 (j & 1), so that
// masking with 0x000F000F (and 0x00F000F0, and the same after >> 8) yields
// the fp16 pairs (j, j+1) = (0,1), (2,3), (4,5), (6,7) directly.  One wave
// therefore reads a tile with one coalesced 16-byte load per lane, and word
// i of lane l is exactly the B-operand fragment lane l supplies to the i-th
// v_mfma_f32_16x16x32_f16 of the block (column n = l % 16, k = 8 g .. 8 g+7).
//
// Dequantisation per word, all exact in fp16: OR-ing a 4-bit field into the
// mantissa of 1024.0 (0x6400) gives 1024 + q, minus 1032 gives q - 8; for
// the fields shifted by 4, 1024 + 16 q times 1/16 minus 72 gives q - 8.  This
// is the known integer-to-float magic-number conversion (the mantissa of a
// float with a fixed exponent holds the integer).  The 32 weights of a lane
// in one block are dotted with x in fp32 (v_dot2_f32_f16), then scaled by
// the group's scale in fp32: the scale is never folded into fp16 weights.
//
// Scales are packed per (tile, 4 consecutive blocks, row): 4 fp16 in 8 bytes,
// so a lane fetches the scales of a 4-block step with one 8-byte load.
//
// int8 activations (vLLM Arm CPU optimisation post, INT8 W4A8 section: 4-bit
// weights times 8-bit activations).  Every workgroup computes the per-token
// scale s_x = max|x| / 127 of the whole fp16 row itself (a max is order-free,
// so all workgroups agree bit for bit), quantises its k-slice to int8 with
// ties-to-even and a +-127 clamp into LDS, and then each packed word costs
// two masks and two v_dot4_i32_i8: the nibbles (e0,e4,e1,e5) and
// (e2,e6,e3,e7) of the word's interleaved order meet activation bytes staged
// in that same order.  The zero-point enters exactly, in integers, as an
// initial accumulator of -8 * (sum of the lane's 32 activation codes).
#include "argmax.hpp"
#include "conv1d.hpp"

namespace wsg {
namespace {

// An LDS pointer for the direct-to-LDS load builtin.
template <typename T>
__device__ __forceinline__ __attribute__((address_space(3))) T *lds(T *p) {
    return (__attribute__((address_space(3))) T *)p;
}

// s_waitcnt immediate that waits for at most n outstanding vector-memory
// operations and nothing else (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt 6:4 and lgkmcnt 11:8 left at their maximum).
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// A split-K partial: written through at agent scope when the last unit of
// the row tile sums the partials (FUSED), else a plain store for the reduce
// kernel.
template <bool FUSED>
__device__ __forceinline__ void store_part(float *p, float v) {
    if constexpr (FUSED)
        __hip_atomic_store(glob(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        *glob(p) = v;
}

template <bool NT>
__device__ __forceinline__ u32x4 load_w(const u32x4 *p) {
    if constexpr (NT)
        return __builtin_nontemporal_load(glob(p));
    else
        return *glob(p);
}

// Constants of the unpack, pinned in registers once per kernel: gfx9 VOP3
// instructions take no 32-bit literal, so with the masks in SGPRs and the
// magic in a VGPR each masked field costs one v_and_or_b32.
struct Unpack {
    uint32_t magic;  // fp16 1024.0 in both halves (VGPR)
    uint32_t lo;     // 0x000F000F (SGPR)
    uint32_t hi;     // 0x00F000F0 (SGPR)
    __device__ __forceinline__ Unpack() : magic(0x64006400u), lo(0x000F000Fu), hi(0x00F000F0u) {
        asm volatile("" : "+v"(magic));
        asm volatile("" : "+s"(lo));
        asm volatile("" : "+s"(hi));
    }
};

// q - 8 for the 8 weights of a packed word, as the fp16 pairs (0,1) .. (6,7).
__device__ __forceinline__ void unpack8(uint32_t w, const Unpack &u, f16x2 (&h)[4]) {
    const uint32_t w8 = w >> 8;
    const f16x2 a = __builtin_bit_cast(f16x2, (w & u.lo) | u.magic);   // 1024 + q0, 1024 + q1
    const f16x2 b = __builtin_bit_cast(f16x2, (w & u.hi) | u.magic);   // 1024 + 16 q2, 1024 + 16 q3
    const f16x2 c = __builtin_bit_cast(f16x2, (w8 & u.lo) | u.magic);  // q4, q5
    const f16x2 d = __builtin_bit_cast(f16x2, (w8 & u.hi) | u.magic);  // 16 q6, 16 q7
    const f16x2 bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const f16x2 bias16 = {(_Float16)-72.0f, (_Float16)-72.0f};
    h[0] = a + bias;
    h[1] = __builtin_elementwise_fma(b, sixteenth, bias16);
    h[2] = c + bias;
    h[3] = __builtin_elementwise_fma(d, sixteenth, bias16);
}

__device__ __forceinline__ float scale_of(u32x2 sc, int b) {
    const uint32_t w = (b < 2) ? sc.x : sc.y;
    const uint16_t h = (b & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xFFFFu);
    return (float)__builtin_bit_cast(_Float16, h);
}

// One work unit: `tile_rtiles` 16-row tiles starting at unit `tile`, k-slice s.
// A wave step covers R tiles x B blocks (B = 4 or 8: 4 or 8 KiB of weights
// per wave in flight per step, two steps in flight).
// MODE kA16: fp16 activations, M = 1 on the VALU.  kMfma: fp16 activations,
// M = 2..8 on the matrix cores.  kA8: int8 activations quantised in the
// prologue, M = 1 on the VALU.
// TAIL = false requires every slice to hold a whole number of steps (the
// blocks of a slice are a multiple of B): then the step loads carry no
// guards, and the compiler can keep the next step's loads in flight while
// the current step is consumed (a guarded load path makes it wait for all).
template <int R, int B, bool NT, int MODE, bool TAIL, bool FUSED = false>
__device__ __forceinline__ void w4_unit(const W4Lin &L, int tile, int s, u32x4 *xs) {
    static_assert(B % 4 == 0, "steps are whole 4-block scale quads");
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int r16 = lane & 15, g = lane >> 4;

    const int kb0 = s * L.kbs;                     // first block of the slice
    const int nkb = min(L.kbs, L.kb - kb0);        // blocks in the slice
    const int nquad = (nkb + B - 1) / B;   // steps per row group
    const int nxv = nkb * 16;                      // 16-byte x vectors per row in the slice
    // LDS row stride of the verify block's activations: a row is padded by
    // 64 bytes, so the A-fragment reads of one instruction (rows 0..M-1, the
    // same k) fall in different LDS banks instead of all in the same ones
    const int xstride = nxv + kW4XRowPad;
    const int64_t n_rtiles = (L.N + 15) / 16;
    const int64_t rt0 = (int64_t)tile * L.tile_rtiles;
    const int nrt = (int)min((int64_t)L.tile_rtiles, n_rtiles - rt0);
    const int64_t last_rt = rt0 + nrt - 1;
    const int ngroups = (nrt + R - 1) / R;
    const int mygroups = wave < ngroups ? (ngroups - 1 - wave) / kWavesPerBlock + 1 : 0;
    const int nsteps = mygroups * nquad;
    constexpr bool MFMA = MODE == kMfma;
    const int M = MFMA ? L.M : 1;
    float sx = 1.0f;  // kA8: activation scale of this row
    const Unpack U;

    struct Buf {
        u32x4 w[R][B];
        u32x2 sc[R][B / 4];
    };

    auto load_step = [&](Buf &Bf, int gi, int c) {
        const int64_t rtb = rt0 + (int64_t)(wave + gi * kWavesPerBlock) * R;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t rt = min(rtb + r, last_rt);
            // wave-uniform tile pointers; the lane offset is the only vector part
            const u32x4 *p = L.Wp + (rt * L.kb + kb0 + B * c) * kWave;
            const u32x2 *q = L.Sp + (rt * L.kq + (kb0 + B * c) / 4) * 16;
            if (!TAIL || B * c + B <= nkb) {
#pragma unroll
                for (int qq = 0; qq < B / 4; ++qq)
                    Bf.sc[r][qq] = *glob(q + qq * 16 + r16);
#pragma unroll
                for (int b = 0; b < B; ++b)
                    Bf.w[r][b] = load_w<NT>(p + b * kWave + lane);
            } else {
#pragma unroll
                for (int qq = 0; qq < B / 4; ++qq) {
                    Bf.sc[r][qq] = u32x2{0u, 0u};
                    if (B * c + 4 * qq < nkb)
                        Bf.sc[r][qq] = *glob(q + qq * 16 + r16);
                }
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    Bf.w[r][b] = u32x4{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
                    if (B * c + b < nkb)
                        Bf.w[r][b] = load_w<NT>(p + b * kWave + lane);
                }
            }
        }
    };

    float acc1[R];
    f32x4 accm[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        acc1[r] = 0.0f;
        accm[r] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    auto finish_group = [&](int gi) {
        const int64_t rtb = rt0 + (int64_t)(wave + gi * kWavesPerBlock) * R;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t rt = rtb + r;
            if constexpr (!MFMA) {
                float v = acc1[r];
                v += xor_lane(v, 16);
                v += xor_lane(v, 32);
                if constexpr (MODE == kA8)
                    v *= sx;
                const int64_t n = rt * 16 + r16;
                if (lane < 16 && rt <= last_rt && n < L.N) {
                    if (L.S > 1) {
                        store_part<FUSED>(L.part + (int64_t)s * L.N + n, v);
                    } else {
                        *glob(L.y + n) = v;
                        if (L.y16)
                            *glob(L.y16 + n) = f16_bits(v);
                    }
                }
                acc1[r] = 0.0f;
            } else {
                // D layout of a 16x16 MFMA: lane l holds column l % 16 (here
                // the output row n) and rows 4 (l / 16) + i (here m).
                const int64_t n = rt * 16 + r16;
                if (rt <= last_rt && n < L.N) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m = 4 * g + i;
                        if (m < M) {
                            if (L.S > 1) {
                                store_part<FUSED>(L.part + ((int64_t)s * M + m) * L.N + n, accm[r][i]);
                            } else {
                                *glob(L.y + (int64_t)m * L.N + n) = accm[r][i];
                                if (L.y16)
                                    *glob(L.y16 + (int64_t)m * L.N + n) = f16_bits(accm[r][i]);
                            }
                        }
                    }
                }
                accm[r] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
    };

    auto consume = [&](const Buf &Bf, int gi, int c) {
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (TAIL && B * c + b >= nkb)
                break;
            const int xv0 = (B * c + b) * 16 + g;  // x vector of word 0 of this lane in the block
            if constexpr (MODE == kA8) {
                // activation codes of this lane's 4 words: 2 x 16 bytes; the
                // lane's zero-point term -8 * sum(codes) starts the chain
                const int pg = (B * c + b) * 4 + g;
                const u32x4 xa = xs[2 * pg], xb = xs[2 * pg + 1];
                const int zs = -8 * reinterpret_cast<const int *>(xs + 8 * nkb)[pg];
                constexpr uint32_t kLo = 0x0F0F0F0Fu;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint32_t w0 = Bf.w[r][b].x, w1 = Bf.w[r][b].y, w2 = Bf.w[r][b].z, w3 = Bf.w[r][b].w;
                    int a = zs;
                    a = __builtin_amdgcn_sdot4((int)(w0 & kLo), (int)xa.x, a, false);
                    a = __builtin_amdgcn_sdot4((int)((w0 >> 4) & kLo), (int)xa.y, a, false);
                    a = __builtin_amdgcn_sdot4((int)(w1 & kLo), (int)xa.z, a, false);
                    a = __builtin_amdgcn_sdot4((int)((w1 >> 4) & kLo), (int)xa.w, a, false);
                    a = __builtin_amdgcn_sdot4((int)(w2 & kLo), (int)xb.x, a, false);
                    a = __builtin_amdgcn_sdot4((int)((w2 >> 4) & kLo), (int)xb.y, a, false);
                    a = __builtin_amdgcn_sdot4((int)(w3 & kLo), (int)xb.z, a, false);
                    a = __builtin_amdgcn_sdot4((int)((w3 >> 4) & kLo), (int)xb.w, a, false);
                    acc1[r] += (float)a * scale_of(Bf.sc[r][b / 4], b % 4);
                }
            } else if constexpr (!MFMA) {
                u32x4 xv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    xv[i] = xs[xv0 + 4 * i];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint32_t words[4] = {Bf.w[r][b].x, Bf.w[r][b].y, Bf.w[r][b].z, Bf.w[r][b].w};
                    float p = 0.0f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        f16x2 h[4];
                        unpack8(words[i], U, h);
                        p = __builtin_amdgcn_fdot2(h[0], as_h2(xv[i].x), p, false);
                        p = __builtin_amdgcn_fdot2(h[1], as_h2(xv[i].y), p, false);
                        p = __builtin_amdgcn_fdot2(h[2], as_h2(xv[i].z), p, false);
                        p = __builtin_amdgcn_fdot2(h[3], as_h2(xv[i].w), p, false);
                    }
                    acc1[r] += p * scale_of(Bf.sc[r][b / 4], b % 4);
                }
            } else {
                // A operand: lane l supplies row m = l % 16 of X, k = 32 i + 8 g
                // .. + 7 of the block.  Result rows m >= M are never stored, so
                // their lanes repeat row M - 1 instead of zeros: every lane reads
                // LDS unconditionally, with no masking and no zero fill.
                const int am = min(r16, M - 1);
                f16x8 a[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    a[i] = __builtin_bit_cast(f16x8, xs[am * xstride + xv0 + 4 * i]);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint32_t words[4] = {Bf.w[r][b].x, Bf.w[r][b].y, Bf.w[r][b].z, Bf.w[r][b].w};
                    f32x4 d = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        f16x2 h[4];
                        unpack8(words[i], U, h);
                        const u32x4 hb = {__builtin_bit_cast(uint32_t, h[0]), __builtin_bit_cast(uint32_t, h[1]),
                                          __builtin_bit_cast(uint32_t, h[2]), __builtin_bit_cast(uint32_t, h[3])};
                        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], __builtin_bit_cast(f16x8, hb), d, 0, 0, 0);
                    }
                    accm[r] += d * scale_of(Bf.sc[r][b / 4], b % 4);
                }
            }
        }
        if (c == nquad - 1)
            finish_group(gi);
    };

    // Steps are (row group gi, step c) in order, c fastest; a is the step
    // in bufA.
    int ga = 0, ca = 0;
    auto next = [&](int &gg, int &cc) {
        if (++cc == nquad) {
            cc = 0;
            ++gg;
        }
    };
    Buf bufA, bufB;

    if constexpr (MFMA) {
        // Verify blocks stage M rows of activations per unit.  Where a row
        // of the slice is whole 64-vector chunks (no tail), each chunk goes
        // straight from memory to LDS (gfx950 direct-to-LDS 16-byte loads,
        // one chunk per wave instruction) ahead of both weight steps: no
        // registers hold it, and since vector-memory loads retire in issue
        // order, a wait for all but the weight loads issued after them
        // leaves both weight steps in flight across the barrier.  Other
        // slices stage through registers behind the weight steps.
        const int64_t xrow = (int64_t)L.K / 8;
        const bool dma = !TAIL && nxv % kWave == 0;
        if (dma) {
            // chunks c = wave, wave + 4, ... of the M rows: row m, vectors v0 .. v0 + 63
            int m = 0, v0 = wave * kWave;
            while (v0 >= nxv) {
                v0 -= nxv;
                ++m;
            }
            for (; m < M;) {
                __builtin_amdgcn_global_load_lds(glob(L.x + m * xrow + (int64_t)kb0 * 16 + v0 + lane),
                                                 lds(xs + m * xstride + v0), 16, 0, 0);
                v0 += kWavesPerBlock * kWave;
                while (v0 >= nxv) {
                    v0 -= nxv;
                    ++m;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        int gb = 0, cb = 0;
        next(gb, cb);
        if (nsteps > 0)
            load_step(bufA, 0, 0);
        if (nsteps > 1)
            load_step(bufB, gb, cb);
        if (dma) {
            __builtin_amdgcn_sched_barrier(0);
            constexpr int kStepLoads = R * (B + B / 4);  // weight and scale loads of one step
            if (nsteps > 1)
                __builtin_amdgcn_s_waitcnt(vmcnt_only(2 * kStepLoads));
            else if (nsteps == 1)
                __builtin_amdgcn_s_waitcnt(vmcnt_only(kStepLoads));
            else
                __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
        } else {
            const int nx = M * nxv;
            for (int i = tid; i < nx; i += kBlock) {
                const int m = i / nxv, v = i - m * nxv;
                xs[i + m * kW4XRowPad] = *glob(L.x + m * xrow + (int64_t)kb0 * 16 + v);
            }
            __syncthreads();
        }
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
        return;
    }

    if constexpr (MODE == kA8) {
        // The per-token scale needs max |x| over the whole fp16 row before
        // any code.  A row of at most kA8HoldVec vectors per thread is loaded
        // into registers ahead of the first weight step and stashed in LDS
        // for the codes, so neither pass waits for weights (loads retire in
        // issue order) and x is read from memory once; longer rows are read
        // twice, behind the first weight step.  The second step goes out
        // behind the barrier, as in the fp16 M = 1 kernel: issuing it earlier
        // made the kernel hold 94 VGPRs instead of 72 (five waves per SIMD
        // instead of seven).
        const bool held = a8_row_held(L.K);
        const int nxall = L.K / 8;
        u32x4 *xraw = xs + 9 * L.kbs + 1;  // after the codes, sums and red[]
        float amax = 0.0f;
        auto absmax_vec = [&](u32x4 h) {
            const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f16x2 p = as_h2(hw[j]);
                amax = fmaxf(amax, fmaxf(fabsf((float)p[0]), fabsf((float)p[1])));
            }
        };
        if (held) {
            u32x4 xh[kA8HoldVec];
#pragma unroll
            for (int j = 0; j < kA8HoldVec; ++j) {
                const int i = tid + j * kBlock;
                xh[j] = u32x4{0u, 0u, 0u, 0u};
                if (i < nxall)
                    xh[j] = *glob(L.x + i);
            }
            if (nsteps > 0)
                load_step(bufA, 0, 0);
#pragma unroll
            for (int j = 0; j < kA8HoldVec; ++j) {
                const int i = tid + j * kBlock;
                if (i < nxall) {
                    xraw[i] = xh[j];
                    absmax_vec(xh[j]);
                }
            }
        } else {
            // the first weight step goes out before the row is read
            if (nsteps > 0)
                load_step(bufA, 0, 0);
            for (int v = tid; v < nxall; v += kBlock)
                absmax_vec(*glob(L.x + v));
        }
        // (1) max |x| over the whole row (the barrier also publishes xraw)
#pragma unroll
        for (int i = 0; i < 6; ++i)
            amax = fmaxf(amax, xor_lane(amax, 32 >> i));
        float *red = reinterpret_cast<float *>(reinterpret_cast<int *>(xs + 8 * nkb) + 4 * nkb);
        if (lane == 0)
            red[wave] = amax;
        __syncthreads();
        amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        sx = amax / 127.0f;
        const float rsx = 1.0f / sx;
        // (2) codes of this slice, one (block, lane group) pair per thread:
        // 8 bytes per packed word in the order (e0,e4,e1,e5 | e2,e6,e3,e7)
        u32x2 *xq8 = reinterpret_cast<u32x2 *>(xs);
        int *sumx = reinterpret_cast<int *>(xs + 8 * nkb);
        const bool write_codes = L.xq_out != nullptr && tile == 0;
        for (int p = tid; p < nkb * 4; p += kBlock) {
            const int b = p >> 2, gg = p & 3;
            int sum = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t v = (int64_t)(kb0 + b) * 16 + 4 * i + gg;   // k = 8 v .. 8 v + 7
                const u32x4 h = held ? xraw[v] : *glob(L.x + v);
                const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
                int e[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
                for (int j = 0; j < 4; j += 2) {  // four codes at a time keep few registers live
                    const f16x2 p0 = as_h2(hw[j]), p1 = as_h2(hw[j + 1]);
                    const float xv[4] = {(float)p0[0], (float)p0[1], (float)p1[0], (float)p1[1]};
                    int c[4] = {0, 0, 0, 0};
                    if (amax != 0.0f)
                        int8_codes(xv, sx, rsx, c);
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        e[2 * j + t] = c[t];
                }
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    sum += e[j];
                const uint32_t d0 = (uint32_t)(e[0] & 255) | (uint32_t)(e[4] & 255) << 8 |
                                    (uint32_t)(e[1] & 255) << 16 | (uint32_t)(e[5] & 255) << 24;
                const uint32_t d1 = (uint32_t)(e[2] & 255) | (uint32_t)(e[6] & 255) << 8 |
                                    (uint32_t)(e[3] & 255) << 16 | (uint32_t)(e[7] & 255) << 24;
                xq8[p * 4 + i] = u32x2{d0, d1};
                if (write_codes) {
                    const uint32_t n0 = (uint32_t)(e[0] & 255) | (uint32_t)(e[1] & 255) << 8 |
                                        (uint32_t)(e[2] & 255) << 16 | (uint32_t)(e[3] & 255) << 24;
                    const uint32_t n1 = (uint32_t)(e[4] & 255) | (uint32_t)(e[5] & 255) << 8 |
                                        (uint32_t)(e[6] & 255) << 16 | (uint32_t)(e[7] & 255) << 24;
                    *glob(reinterpret_cast<u32x2 *>(L.xq_out) + v) = u32x2{n0, n1};
                }
            }
            sumx[p] = sum;
        }
        if (L.sx_out != nullptr && tile == 0 && s == 0 && tid == 0)
            *glob(L.sx_out) = sx;
        __syncthreads();
    } else {
        // M = 1, fp16 activations: the first vectors of the activation slice
        // are loaded ahead of the first weight step, so that staging them
        // waits for them alone; the second step goes out behind the barrier.
        constexpr int kXHold1 = 2;
        u32x4 xh[kXHold1];
#pragma unroll
        for (int j = 0; j < kXHold1; ++j) {
            const int i = tid + j * kBlock;
            if (i < nxv)
                xh[j] = *glob(L.x + (int64_t)kb0 * 16 + i);
        }
        if (nsteps > 0)
            load_step(bufA, 0, 0);
#pragma unroll
        for (int j = 0; j < kXHold1; ++j) {
            const int i = tid + j * kBlock;
            if (i < nxv)
                xs[i] = xh[j];
        }
        for (int i = tid + kXHold1 * kBlock; i < nxv; i += kBlock)
            xs[i] = *glob(L.x + (int64_t)kb0 * 16 + i);
        __syncthreads();
    }

    if (nsteps == 0)
        return;
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
}

// The epilogues of a finished unit (S = 1) that read its rows of y back:
// the causal-conv1d step of each row (M = 1), then the greedy-token key of
// each output row m < M.
__device__ __forceinline__ void w4_after_unit(const W4Lin &L, int tile) {
    const int64_t r0 = (int64_t)tile * L.tile_rtiles * 16;
    const int64_t nrows = min((int64_t)L.tile_rtiles * 16, L.N - r0);
    if (L.conv.out != nullptr) {
        __syncthreads();  // the unit's stores of y are visible to the whole workgroup
        for (int64_t i = threadIdx.x; i < nrows; i += kBlock)
            conv_step(L.conv, r0 + i, *glob(L.y + r0 + i));
    }
    for (int m = 0; L.arg.keys != nullptr && m < L.M; ++m)
        publish_rows(L.arg, L.y + (int64_t)m * L.N, r0, nrows, tile, m);
}

// The matrix-core variant holds the A operands, the MFMA chains and two
// steps of weights; left alone the compiler gives the 2-tile x 4-block shape
// 196 VGPRs + 32 AGPRs, two waves per SIMD.  Capping it at three waves per
// SIMD (168 registers) costs no spills and keeps more weight loads in
// flight.  Steps of 16 blocks would spill under the cap and keep the default.
template <int R, int B, int MODE>
constexpr int w4_min_waves_per_simd() {
    return MODE == kMfma && R * B <= 8 ? 3 : 1;
}

// Split k summed by the last unit of each row tile (the dense kinds' scheme:
// written-through partials, the wave's stores complete before it counts in
// on the tile's counter, which wraps to zero on the last arrival; the last
// unit reads the S partials back with agent-scope loads and adds them in
// slice order, the reduce kernel's order), then the epilogues.
__device__ __forceinline__ void w4_last_arriver(const W4Lin &L, int tile) {
    __shared__ uint32_t s_old;
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const uint32_t last = (uint32_t)L.S - 1u;
    if (threadIdx.x == 0)
        s_old = __builtin_amdgcn_atomic_inc32(glob(L.ctr + tile), last, __ATOMIC_RELAXED, "agent");
    __syncthreads();
    if (s_old != last)
        return;
    const int64_t r0 = (int64_t)tile * L.tile_rtiles * 16;
    const int nrows = (int)min((int64_t)L.tile_rtiles * 16, L.N - r0);
    const int64_t total = (int64_t)L.M * L.N;
    for (int m = 0; m < L.M; ++m) {
        for (int i = threadIdx.x; i < nrows; i += kBlock) {
            const int64_t j = (int64_t)m * L.N + r0 + i;
            float a = 0.0f;
            for (int sl = 0; sl < L.S; ++sl) {
                const float v = __hip_atomic_load(glob(L.part + (int64_t)sl * total + j), __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
                a = sl == 0 ? v : a + v;
            }
            *glob(L.y + j) = a;
            if (L.y16)
                *glob(L.y16 + j) = f16_bits(a);
        }
    }
    if (L.arg.keys != nullptr || L.conv.out != nullptr)
        w4_after_unit(L, tile);
}

// FUSED is a kernel of its own, so that the arrival code leaves the plain
// kernel's registers (and resident waves) as they are.
template <int R, int B, bool NT, int MODE, bool TAIL, bool FUSED>
__global__ __launch_bounds__(kBlock, (w4_min_waves_per_simd<R, B, MODE>())) void w4_gemv_kernel(W4Lin L) {
    extern __shared__ u32x4 xs_dyn[];
    const int u = blockIdx.x;
    w4_unit<R, B, NT, MODE, TAIL, FUSED>(L, u / L.S, u % L.S, xs_dyn);
    if constexpr (FUSED)
        w4_last_arriver(L, u / L.S);
    else if (L.S == 1 && (L.arg.keys != nullptr || L.conv.out != nullptr))
        w4_after_unit(L, u);
}

template <int R, int B, bool NT, int MODE, bool TAIL>
__global__ __launch_bounds__(kBlock, (w4_min_waves_per_simd<R, B, MODE>())) void w4_grouped_kernel(const W4Lin *__restrict__ lins,
                                                            const Unit *__restrict__ units) {
    extern __shared__ u32x4 xs_dyn[];
    const Unit u = units[blockIdx.x];
    const W4Lin L = lins[u.lin];
    w4_unit<R, B, NT, MODE, TAIL>(L, u.tile, u.s, xs_dyn);
    if (L.S == 1 && (L.arg.keys != nullptr || L.conv.out != nullptr))
        w4_after_unit(L, u.tile);
}

// y[m][n] = sum over slices s = 0..S-1, in that order, of part[s][m][n];
// every row m's greedy-token key of this workgroup when taken; and the
// causal-conv1d step over y (M = 1) when taken.
__global__ __launch_bounds__(kBlock) void w4_reduce_kernel(W4Lin L) {
    const int64_t total = (int64_t)L.M * L.N;
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    unsigned long long key = 0;
    int m = -1;
    if (i < total) {
        float a = L.part[i];
        for (int s = 1; s < L.S; ++s)
            a += L.part[(int64_t)s * total + i];
        L.y[i] = a;
        if (L.y16)
            L.y16[i] = f16_bits(a);
        m = (int)(i / L.N);
        key = arg_key(a, i - (int64_t)m * L.N);
        if (L.conv.out != nullptr)  // M = 1
            conv_step(L.conv, i, a);
    }
    if (L.arg.keys != nullptr)
        for (int mm = 0; mm < L.M; ++mm)
            arg_publish(L.arg, mm == m ? key : 0ull, blockIdx.x, mm);
}

// One thread per packed word: tile t, block b, lane l, word i.
__global__ __launch_bounds__(kBlock) void pack_w4_kernel(const uint32_t *__restrict__ Wc,
                                                         uint32_t *__restrict__ Wp, int64_t N, int32_t K) {
    const int32_t kb = K / 128;
    const int64_t n_rtiles = (N + 15) / 16;
    const int64_t total = n_rtiles * kb * 256;  // 64 lanes x 4 words per tile
    const int64_t idx = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (idx >= total)
        return;
    const int i = (int)(idx & 3);
    const int l = (int)((idx >> 2) & 63);
    const int64_t tb = idx >> 8;             // tile index t * kb + b
    const int64_t t = tb / kb;
    const int b = (int)(tb - t * kb);
    const int64_t n = t * 16 + (l & 15);
    const int gq = l >> 4;
    uint32_t out = 0x88888888u;              // padding rows: q = 8, weight 0
    if (n < N) {
        const uint32_t w = Wc[n * (K / 8) + (int64_t)b * 16 + 4 * i + gq];  // k = 128 b + 32 i + 8 g
        out = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t q = (w >> (4 * j)) & 15u;
            out |= q << (4 * ((j >> 1) + 4 * (j & 1)));
        }
    }
    Wp[idx] = out;
}

// Scales: Sp[(t * kq + q) * 16 + r] holds s4[n = 16 t + r][4 q + (0..3)], zero past K or N.
__global__ __launch_bounds__(kBlock) void pack_s4_kernel(const uint16_t *__restrict__ s4,
                                                         uint16_t *__restrict__ Sp, int64_t N, int32_t K) {
    const int32_t kb = K / 128, kq = (kb + 3) / 4;
    const int64_t n_rtiles = (N + 15) / 16;
    const int64_t total = n_rtiles * kq * 64;  // 16 rows x 4 scales per (tile, quad)
    const int64_t idx = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (idx >= total)
        return;
    const int j = (int)(idx & 3);
    const int r = (int)((idx >> 2) & 15);
    const int64_t tq = idx >> 6;
    const int64_t t = tq / kq;
    const int q = (int)(tq - t * kq);
    const int64_t n = t * 16 + r;
    const int b = 4 * q + j;
    Sp[idx] = (n < N && b < kb) ? s4[n * kb + b] : (uint16_t)0;
}

template <int R, int B, bool NT, int MODE, bool TAIL>
hipError_t launch_one(const W4Lin &L, hipStream_t s) {
    const int units = L.n_tiles * L.S;
    if (L.S > 1 && L.fuse)
        hipLaunchKernelGGL((w4_gemv_kernel<R, B, NT, MODE, TAIL, true>), dim3(units), dim3(kBlock),
                           w4_lds_bytes(L, MODE), s, L);
    else
        hipLaunchKernelGGL((w4_gemv_kernel<R, B, NT, MODE, TAIL, false>), dim3(units), dim3(kBlock),
                           w4_lds_bytes(L, MODE), s, L);
    return hipGetLastError();
}

template <int R, int B, bool NT, int MODE, bool TAIL>
hipError_t launch_grp(const W4Lin *lins, const Unit *units, int n, int lds, hipStream_t s) {
    hipLaunchKernelGGL((w4_grouped_kernel<R, B, NT, MODE, TAIL>), dim3(n), dim3(kBlock), lds, s, lins, units);
    return hipGetLastError();
}

// Instantiated shapes: R in {1, 2} tiles, B in {4, 8} blocks per wave step.
template <int MODE, bool NT, bool TAIL>
hipError_t dispatch_one(const W4Lin &L, const W4Cfg &c, hipStream_t s) {
    if (c.R == 1 && c.B == 8) return launch_one<1, 8, NT, MODE, TAIL>(L, s);
    if (c.R == 1 && c.B == 4) return launch_one<1, 4, NT, MODE, TAIL>(L, s);
    if (c.R == 2 && c.B == 8) return launch_one<2, 8, NT, MODE, TAIL>(L, s);
    if (c.R == 2 && c.B == 4) return launch_one<2, 4, NT, MODE, TAIL>(L, s);
    return hipErrorInvalidValue;
}

template <int MODE, bool NT, bool TAIL>
hipError_t dispatch_grp(const W4Lin *lins, const Unit *units, int n, int lds, const W4Cfg &c, hipStream_t s) {
    if (c.R == 1 && c.B == 8) return launch_grp<1, 8, NT, MODE, TAIL>(lins, units, n, lds, s);
    if (c.R == 1 && c.B == 4) return launch_grp<1, 4, NT, MODE, TAIL>(lins, units, n, lds, s);
    if (c.R == 2 && c.B == 8) return launch_grp<2, 8, NT, MODE, TAIL>(lins, units, n, lds, s);
    if (c.R == 2 && c.B == 4) return launch_grp<2, 4, NT, MODE, TAIL>(lins, units, n, lds, s);
    return hipErrorInvalidValue;
}

template <int MODE>
hipError_t one_mode(const W4Lin &L, const W4Cfg &c, hipStream_t s) {
    if (c.nt)
        return c.tail ? dispatch_one<MODE, true, true>(L, c, s) : dispatch_one<MODE, true, false>(L, c, s);
    return c.tail ? dispatch_one<MODE, false, true>(L, c, s) : dispatch_one<MODE, false, false>(L, c, s);
}

template <int MODE>
hipError_t grp_mode(const W4Lin *lins, const Unit *units, int n, int lds, const W4Cfg &c, hipStream_t s) {
    if (c.nt)
        return c.tail ? dispatch_grp<MODE, true, true>(lins, units, n, lds, c, s)
                      : dispatch_grp<MODE, true, false>(lins, units, n, lds, c, s);
    return c.tail ? dispatch_grp<MODE, false, true>(lins, units, n, lds, c, s)
                  : dispatch_grp<MODE, false, false>(lins, units, n, lds, c, s);
}

}  // namespace

hipError_t launch_w4(const W4Lin &L, int mode, const W4Cfg &c, hipStream_t s) {
    if (mode == kA8)
        return one_mode<kA8>(L, c, s);
    return mode == kMfma ? one_mode<kMfma>(L, c, s) : one_mode<kA16>(L, c, s);
}

hipError_t launch_w4_grouped(const W4Lin *lins, const Unit *units, int n_units, int lds_bytes, int mode,
                             const W4Cfg &c, hipStream_t s) {
    if (mode == kA8)
        return grp_mode<kA8>(lins, units, n_units, lds_bytes, c, s);
    return mode == kMfma ? grp_mode<kMfma>(lins, units, n_units, lds_bytes, c, s)
                         : grp_mode<kA16>(lins, units, n_units, lds_bytes, c, s);
}

int w4_reduce_blocks(int64_t M, int64_t N) { return (int)((M * N + kBlock - 1) / kBlock); }

hipError_t launch_w4_reduce(const W4Lin &L, hipStream_t s) {
    hipLaunchKernelGGL(w4_reduce_kernel, dim3((unsigned)w4_reduce_blocks(L.M, L.N)), dim3(kBlock), 0, s, L);
    return hipGetLastError();
}

hipError_t launch_pack_w4(const uint32_t *Wc, const uint16_t *s4, u32x4 *Wp, u32x2 *Sp, int64_t N, int32_t K,
                          hipStream_t s) {
    const int64_t n_rtiles = (N + 15) / 16;
    const int32_t kb = K / 128, kq = (kb + 3) / 4;
    const int64_t words = n_rtiles * kb * 256;
    const int64_t scales = n_rtiles * kq * 64;
    if (words > 0)
        hipLaunchKernelGGL(pack_w4_kernel, dim3((unsigned)((words + kBlock - 1) / kBlock)), dim3(kBlock), 0, s,
                           Wc, reinterpret_cast<uint32_t *>(Wp), N, K);
    if (scales > 0)
        hipLaunchKernelGGL(pack_s4_kernel, dim3((unsigned)((scales + kBlock - 1) / kBlock)), dim3(kBlock), 0, s,
                           s4, reinterpret_cast<uint16_t *>(Sp), N, K);
    return hipGetLastError();
}

}  // namespace wsg
