// Internal declarations shared by the wsgemv kernels and the host side of the
// library: device descriptors of one linear, launch configurations and the
// launcher functions each kernel file exports.  gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wsg {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kBlock = 256;        // 4 waves per workgroup for every streaming kernel
constexpr int kWavesPerBlock = kBlock / kWave;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum Kind : int32_t { kF16 = 0, kW8A8 = 1, kW4A16 = 2, kW4A8 = 3, kW8A8D = 4 };

// int4-weight kernel modes: fp16 activations on the VALU (M = 1), fp16
// activations on MFMA (M = 2..8), int8 activations quantised in-kernel (M = 1).
enum W4Mode : int32_t { kA16 = 0, kMfma = 1, kA8 = 2 };

// Reinterpret a 32-bit word as two fp16.  Always pass a scalar copy: with
// this toolchain, __builtin_bit_cast applied directly to an ext-vector
// element expression (v.y, v.z, ...) lowers to element 0 for every element.
__device__ __forceinline__ f16x2 as_h2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }

// fp32 -> fp16 bits, round to nearest even (overflow to inf).
__device__ __forceinline__ uint16_t f16_bits(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }

// The value that lane (l ^ stride) holds, for stride = 1, 2, 4, ..., 32, by
// DPP row operations and the gfx950 lane-swap instructions: plain vector
// instructions, where a generic shuffle goes through the LDS crossbar and
// waits for it.  Every lane of the wave must be active.  The stride must be a
// compile-time constant after unrolling (the switch then folds away).
__device__ __forceinline__ uint32_t xor_lane(uint32_t v, int stride) {
    const int lane = __lane_id();
    switch (stride) {
    case 1:
        return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    case 2:
        return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
    case 4: {
        const uint32_t up = __builtin_amdgcn_mov_dpp(v, 0x104, 0xF, 0xF, false);  // row_shl:4, lane i reads i + 4
        const uint32_t dn = __builtin_amdgcn_mov_dpp(v, 0x114, 0xF, 0xF, false);  // row_shr:4, lane i reads i - 4
        return (lane & 4) ? dn : up;
    }
    case 8:
        return __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false);  // row_ror:8
    case 16: {
        // swap(v, v): element 0 holds rows (0, 0, 2, 2), element 1 rows (1, 1, 3, 3)
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane & 16) ? r[0] : r[1];
    }
    default: {
        // swap(v, v): element 0 holds halves (0, 0), element 1 halves (1, 1)
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane & 32) ? r[0] : r[1];
    }
    }
}

__device__ __forceinline__ float xor_lane(float v, int stride) {
    return __builtin_bit_cast(float, xor_lane(__builtin_bit_cast(uint32_t, v), stride));
}

__device__ __forceinline__ int32_t xor_lane(int32_t v, int stride) {
    return (int32_t)xor_lane((uint32_t)v, stride);
}

// Per-token int8 activation codes c = clamp(rint(x / s), -127, 127), with the
// quotient the IEEE fp32 division x / s (rounded to nearest) and rint ties to
// even, for N values and s > 0; rs = fp32(1 / s).  The quotient is first
// taken as t = fp32(x * rs): with unit roundoff u = 2^-24, t and fp32(x / s)
// differ by at most about 3u|t|, so when t lies farther than 8u|t| from every
// half-integer both round to the same integer.  Only a lane holding a value
// inside that window (or a NaN) takes the exact division, for its N values.
// The distance 0.5 - |t - rint(t)| is exact where it matters (t - rint(t) is
// exact; the subtraction from 0.5 is exact once |t - rint(t)| >= 1/4), and
// no step is contracted into a fused multiply-add.
template <int N>
__device__ __forceinline__ void int8_codes(const float (&x)[N], float s, float rs, int (&c)[N]) {
#pragma clang fp contract(off)
    bool exact = false;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float t = x[i] * rs;
        const float r = rintf(t);
        exact |= !(0.5f - fabsf(t - r) > fabsf(t) * 0x1p-21f);
        c[i] = (int)fminf(fmaxf(r, -127.0f), 127.0f);
    }
    if (exact) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            c[i] = (int)fminf(fmaxf(rintf(x[i] / s), -127.0f), 127.0f);
    }
}

// The global-memory view of a device pointer.  The work-table kernels read
// their tensor pointers from memory, where the compiler cannot see that they
// point to global memory, and would access them with flat instructions.  A
// flat access also counts against the LDS wait counter, so each wait for an
// activation read from LDS would also wait for every weight load still in
// flight, which serialises the stream inside a wave.  Every kernel access to
// a tensor goes through glob(), which makes it a global load or store.
template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T *glob(T *p) {
    return (__attribute__((address_space(1))) T *)p;
}

// Fused greedy-token output of a linear (device functions in argmax.hpp).
// keys == nullptr: no token is taken.
struct ArgOut {
    unsigned long long *keys;  // [M][stride] best key of each publishing workgroup, per position
    int32_t *idx;              // out: [M] tokens (index of the largest logit of each output row)
    float *val;                // out, optional: [M] their logits
    int32_t n_keys;            // workgroups that publish in one launch
    int32_t stride;            // keys per position row (n_keys rounded up to 32)
    int32_t M;                 // positions (output rows of a verify block); 1 otherwise
    int32_t pad;
};

inline int32_t arg_key_stride(int32_t n_keys) { return (n_keys + 31) / 32 * 32; }

// Fused causal-conv1d decode step over a linear's output (conv1d.hpp).
// out == nullptr: none.
struct ConvOut {
    const uint16_t *w;     // fp16 [N][W] taps, oldest input first
    const float *bias;     // optional [N]
    float *state;          // [N][W-1] previous inputs, oldest first (updated)
    float *out;            // [N]
    int32_t W;             // taps, 2..8
    int32_t silu;          // apply SiLU to the output
};

// One row-major linear streamed 16 bytes per lane (fp16: 8 weights per
// vector, int8: 16 weights per vector).
struct DenseLin {
    const u32x4 *W;        // [N][kvec]
    const u32x4 *x;        // [kvec]
    float *y;              // [N]
    void *part;            // [S][N] fp32 (fp16) or int32 (int8) partial sums, S > 1
    const float *w_scale;  // int8: [N]
    const float *x_scale;  // int8: [1]
    int32_t *acc_out;      // int8: optional [N]
    int64_t N;
    int32_t kvec;          // 16-byte vectors per row
    int32_t S;             // k-slices
    int32_t kvs;           // vectors per slice (the last slice may be shorter)
    int32_t tile_rows;     // rows per work unit
    int32_t n_tiles;       // ceil(N / tile_rows)
    int32_t fuse;          // S > 1: 0 = a reduce kernel sums the partials; 1 = the last unit of each
                           // row tile does (partials written through at agent scope)
    ArgOut arg;            // optional greedy token over y (S = 1 or fused: the units; else the reduce)
    ConvOut conv;          // optional causal-conv1d step over y (same place as y is final)
    uint16_t *y16;         // optional fp16 copy of y [N] (same place as y is final)
    int8_t *xq_out;        // kW8A8D: optional int8 codes [K] (written by the first row tile)
    float *sx_out;         // kW8A8D: optional activation scale [1]
    float *sx_part;        // kW8A8D with S > 1: the activation scale, after the partials (for the reduce kernel)
    uint32_t *ctr;         // fuse != 0: [n_tiles] arrival counters, zero between launches
};

// One int4 linear in the packed tile layout (16 rows x 128 k per 1 KiB tile).
struct W4Lin {
    const u32x4 *Wp;       // [n_rtiles][kb][64 lanes] 16-byte words
    const u32x2 *Sp;       // [n_rtiles][kq][16 rows] 4 fp16 scales (blocks 4q..4q+3)
    const u32x4 *x;        // fp16 [M][K] as 16-byte vectors
    float *y;              // [M][N]
    float *part;           // [S][M][N], S > 1
    int8_t *xq_out;        // kA8: optional int8 codes [K] (written by the first row tile)
    float *sx_out;         // kA8: optional activation scale [1]
    int64_t N;
    int32_t K;
    int32_t M;
    int32_t kb;            // 128-wide k-blocks per row (K / 128)
    int32_t kq;            // ceil(kb / 4)
    int32_t S;
    int32_t kbs;           // k-blocks per slice, a multiple of 4 when S > 1
    int32_t tile_rtiles;   // 16-row tiles per work unit
    int32_t n_tiles;       // ceil(n_rtiles / tile_rtiles)
    ArgOut arg;            // optional greedy token of each output row (where y is final)
    ConvOut conv;          // optional causal-conv1d step over y (M = 1; where y is final)
    uint16_t *y16;         // optional fp16 copy of y [M][N] (where y is final)
    uint32_t *ctr;         // S > 1 and fuse: [n_tiles] arrival counters, zero between launches
    int32_t fuse;          // S > 1: 0 = a reduce kernel sums the partials; 1 = the last unit of each
                           // row tile does (partials written through at agent scope)
    int32_t pad;
};

// One work unit of a grouped launch: linear `lin`, row tile `tile`, k-slice `s`.
struct Unit {
    int32_t lin;
    int32_t tile;
    int32_t s;
    int32_t pad;
};

// One fp16 linear of a persistent dependency-respecting step (M = 1, whole
// k per unit).  Its input is either a plain fp16 vector (x) or the tagged
// output words of an earlier linear (x_tag): word k = (tag << 16) | fp16
// bits of input k, current when its tag is the step's.
struct ChainLin {
    const u32x4 *W;          // [N][kvec]
    const u32x4 *x;          // plain input [kvec] (x_tag == nullptr)
    const uint32_t *x_tag;   // tagged input words [8 * kvec], or nullptr
    float *y;                // [N]
    uint16_t *y16;           // optional fp16 copy of y [N]
    uint32_t *tag_out;       // optional tagged copy of y16 for later linears [N]
    int64_t N;
    int32_t kvec;            // 16-byte vectors per row
    int32_t tile_rows;       // rows per work unit
    int32_t n_tiles;
    int32_t pad;
};

// Control block of a persistent step (its own 256-byte line).
struct ChainCtl {
    uint32_t give_ups;       // waits that gave up (cumulative until the host clears it)
    uint32_t abort_epoch;    // epoch of the last step in which a wait gave up
    uint32_t pad[62];
};

// Per-launch arguments of the persistent step kernel.
struct ChainArgs {
    const ChainLin *lins;
    const Unit *units;
    ChainCtl *ctl;
    int32_t n_units;
    int32_t xs_vecs;         // 16-byte vectors of one LDS input buffer (two alternate)
    uint32_t epoch;          // step number (never 0)
    uint32_t tag;            // written with this step's outputs (1..65535)
    uint32_t want;           // inputs are current with this tag (== tag; tests may differ)
    uint32_t spin_limit;     // polls before a wait gives up
    int32_t sleep;           // s_sleep(1) calls between polls (0: poll again at once)
    uint64_t *trace;         // per-unit timestamps [4 * n_units], or nullptr
};

struct DenseCfg {
    int R;        // rows per wave step
    int CH;       // 16-byte vectors per lane per row per step
    bool nt;      // non-temporal weight loads
    bool tail;    // some k-slice is not a whole number of chunks (64 * CH vectors)
};

// True when a slice of this linear ends inside a chunk of 64 * CH vectors.
inline bool dense_needs_tail(const DenseLin &L, int CH) {
    const int chunk = kWave * CH;
    const int last = L.kvec - (L.S - 1) * L.kvs;
    return (L.kvs % chunk) != 0 || (last % chunk) != 0;
}

struct W4Cfg {
    int R;        // 16-row tiles per wave step
    int B;        // 128-wide k-blocks per wave step (4 or 8)
    bool nt;
    bool tail;    // some k-slice is not a whole number of B-block steps
};

// True when a slice of this linear ends inside a step of B blocks.
inline bool w4_needs_tail(const W4Lin &L, int B) {
    const int last = L.kb - (L.S - 1) * L.kbs;
    return (L.kbs % B) != 0 || (last % B) != 0;
}

// ----- launchers (each defined next to its kernels) -----
hipError_t launch_dense(int kind, const DenseLin &L, const DenseCfg &c, hipStream_t s);
hipError_t launch_dense_grouped(int kind, const DenseLin *lins, const Unit *units, int n_units,
                                int lds_bytes, const DenseCfg &c, hipStream_t s);
hipError_t launch_dense_reduce(int kind, const DenseLin &L, hipStream_t s);
int dense_reduce_blocks(int64_t N);
hipError_t launch_chain(const ChainArgs &a, int grid, int lds_bytes, bool tail, hipStream_t s);
hipError_t chain_blocks_per_cu(int lds_bytes, bool tail, int *blocks);
hipError_t launch_w4(const W4Lin &L, int mode, const W4Cfg &c, hipStream_t s);
hipError_t launch_w4_grouped(const W4Lin *lins, const Unit *units, int n_units, int lds_bytes,
                             int mode, const W4Cfg &c, hipStream_t s);
hipError_t launch_w4_reduce(const W4Lin &L, hipStream_t s);
int w4_reduce_blocks(int64_t M, int64_t N);
hipError_t launch_pack_w4(const uint32_t *Wc, const uint16_t *s4, u32x4 *Wp, u32x2 *Sp,
                          int64_t N, int32_t K, hipStream_t s);
struct ProbeCfg {
    int U;         // 16-byte loads in flight per lane per iteration (4, 8, 16)
    bool nt;       // non-temporal loads
    bool chunked;  // contiguous share per workgroup instead of grid-stride
};
hipError_t launch_read_probe(const u32x4 *buf, int64_t nvec, float *out, int grid, const ProbeCfg &c,
                             hipStream_t s);
hipError_t launch_zero_f32(float *p, int64_t n, hipStream_t s);
hipError_t launch_zero_u16(uint16_t *p, int64_t n, hipStream_t s);
hipError_t launch_argmax_finish(const ArgOut &a, hipStream_t s);
hipError_t launch_conv1d_step(const float *x, const ConvOut &cv, int64_t C, hipStream_t s);
int64_t topk_plan(int64_t N, int k, int64_t *max_keys, int *passes);
hipError_t launch_topk(const float *y, int64_t N, int k, int32_t *idx, float *val, unsigned long long *ws_a,
                       unsigned long long *ws_b, hipStream_t s);
hipError_t launch_argmax_f32(const float *y, int64_t N, ArgOut a, hipStream_t s);
int argmax_f32_blocks(int64_t N);

// LDS bytes a dense unit of this linear stages for x (whole slice, chunk-padded).
inline int dense_lds_bytes(const DenseLin &L, int CH) {
    int chunk = kWave * CH;
    int nch = (L.kvs + chunk - 1) / chunk;
    return nch * chunk * 16;
}

// int8-activation units whose fp16 row fits kA8HoldVec 16-byte vectors per
// thread hold it in registers, and stash it in LDS for the codes.
constexpr int kA8HoldVec = 2;
__host__ __device__ inline bool a8_row_held(int64_t K) { return K / 8 <= (int64_t)kA8HoldVec * kBlock; }

// Padding of each activation row of a verify block in LDS, in 16-byte vectors.
constexpr int kW4XRowPad = 4;

inline int w4_lds_bytes(const W4Lin &L, int mode) {
    if (mode == kA8)  // int8 codes of the slice, one int sum per (block, lane group), 4 floats[, the fp16 row]
        return L.kbs * 128 + L.kbs * 4 * 4 + 16 + (a8_row_held(L.K) ? L.K * 2 : 0);
    if (mode == kMfma)  // x slice for all M rows, each row padded
        return L.M * (L.kbs * 16 + kW4XRowPad) * 16;
    // x slice: kbs blocks of 128 fp16
    return L.M * L.kbs * 128 * 2;
}

}  // namespace wsg
