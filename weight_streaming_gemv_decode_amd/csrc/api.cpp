// C ABI of wsgemv: argument validation, the per-shape launch table, the
// GEMV entry points and the decode-step plan (hipGraph capture and replay).
//
// The launch table follows the operator implementation table of the EdgeFM
// summary (section 2B): an operator call is mapped to a kernel configuration
// by its tensor-shape signature.  Here the key is (kind, M, N, K) and the
// value is the k-split S, the rows per work unit and the kernel variant.
// Graph replay follows the same summary, section 2C: the launches of one
// decode step are captured once and replayed every step.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <unordered_set>
#include <vector>

#include "wsgemv.h"
#include "wsg_common.hpp"

using namespace wsg;

namespace {

thread_local int32_t g_last_hip = 0;

wsg_status hip_fail(hipError_t e) {
    g_last_hip = (int32_t)e;
    return WSG_ERR_HIP;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// HIP takes a launch's grid as a 32-bit count of work-items, so a launch of
// kBlock-thread workgroups holds at most this many workgroups.  Shapes whose
// launches would need more are rejected (WSG_ERR_UNSUPPORTED) before any
// size is narrowed to the kernels' 32-bit fields.
constexpr int64_t kMaxBlocks = (int64_t)UINT32_MAX / kBlock;
bool grid_ok(int64_t blocks) { return blocks <= kMaxBlocks; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Largest k-slice, in 16-byte vectors, a dense unit stages in LDS (32 KiB).
constexpr int kMaxSliceVec = 2048;
// Work units wanted per launch (4 per compute unit on 256 CUs).
constexpr int64_t kWantUnits = 1024;
constexpr int kMaxM = 8;

// Launch-table overrides for tuning sweeps (wsg_tune_set).  -1 = the
// table's own choice.  No result depends on them: every configuration
// computes the same sums (split-K changes only the summation order).
struct Tune {
    int64_t nt = -1;             // non-temporal weight loads
    int64_t dense_R = -1, dense_CH = -1, dense_rows = -1;
    int64_t group_R = -1, group_CH = -1, group_unit_kb = -1;
    int64_t w4_R = -1, w4_B = -1, w4_tiles = -1, group_w4_tiles = -1;
    int64_t w4_mfma_m1 = -1;     // 1: W4A16 at M = 1 on the matrix cores
    int64_t probe_U = -1, probe_chunked = -1;
    int64_t chain_unit_kb = -1;       // persistent step: weight bytes per work unit (KiB)
    int64_t chain_blocks_per_cu = -1; // persistent step: workgroups per compute unit (at most the resident count)
    int64_t chain_spin_limit = -1;    // persistent step: polls before a wait gives up
    int64_t chain_test_stale = -1;    // 1: consumers wait for a tag no producer writes (tests the give-up path)
    int64_t chain_sleep = -1;         // s_sleep(1) calls between polls of a waiting workgroup
    int64_t split_fuse = -1;          // split-K sum: 0 reduce kernel, 1 last unit of each row tile
};
Tune g_tune;

// Non-temporal weight loads by default: the weight stream has no reuse, and
// on MI355X they lift streaming reads from ~6.1 to ~7.1 TB/s.
bool use_nt() { return g_tune.nt != 0; }

bool dense_shape_ok(int64_t R, int64_t CH, bool grouped) {
    if (CH == 2)
        return R == 4 || R == 2 || (!grouped && R == 1);
    if (CH == 1)
        return R == 8 || (!grouped && R == 4);
    return false;
}

// ---------------------------------------------------------------- dense --

struct DensePlan {
    DenseCfg cfg;
    int S;
    int kvs;
    int tile_rows;
    int fuse;       // S > 1: how the partials are summed (DenseLin::fuse)
};

// How a split linear of any kind sums its partials (DenseLin::fuse,
// W4Lin::fuse): by default the last unit of each row tile does.  Measured on
// MI355X against the reduce kernel (bit-identical results): 6.7-7.1 against
// 9.3-9.7 us on fp16 linears of 128-896 rows that the launch table splits,
// 7.7-8.7 against 10.1 us on the int8 ones, and 76.9 against 77.0 us on the
// 248320x1024 lm_head at S = 2.
int split_fuse_mode() { return g_tune.split_fuse >= 0 ? (int)std::min<int64_t>(g_tune.split_fuse, 1) : 1; }

int elem_per_vec(int kind) { return kind == kF16 ? 8 : 16; }

int dense_min_splits(int64_t kvec) { return (int)std::max<int64_t>(1, cdiv(kvec, kMaxSliceVec)); }

// `token`: the linear also takes the greedy token, whose finish kernel reads
// one key per work unit.
DensePlan plan_dense(int kind, int64_t N, int64_t K, int splits, bool token = false) {
    const int64_t kvec = K / elem_per_vec(kind);
    DensePlan p;
    int S = splits > 0 ? splits : dense_min_splits(kvec);
    // Row tile: 4 waves x R rows per unit.  Small units keep many
    // workgroups in flight; split k only when the launch would have fewer
    // than 256 units even with 4-row units (slices stay whole 128-vector
    // chunks).
    if (splits <= 0 && cdiv(N, 4) * S < 256 && kvec >= 256) {
        const int64_t chunks = kvec / 128;
        for (int s = S + 1; s <= 16 && s <= chunks; ++s) {
            if (kvec % (128LL * s) == 0 || s == (int)chunks) {
                S = s;
                if (cdiv(N, 4) * S >= 256)
                    break;
            }
        }
    }
    p.S = S;
    p.kvs = (int)cdiv(kvec, S);
    int tr;
    if (p.kvs % 128 != 0 && p.kvs % 64 == 0) {
        // 64-vector slices (e.g. K = 1024 fp16 cut in two): 8 rows x 1 vector per step
        p.cfg = DenseCfg{8, 1, use_nt(), false};
        tr = 32;
    } else if (cdiv(N, 16) * S >= 1024 && kind == kF16 && !token) {
        // many rows: 4-row units (1 row per wave).  On the 248320x1024
        // lm_head they measured 70.6 us against 73.7 us for 16-row units;
        // with the token, 4x the units would be 4x the keys its finish reads.
        p.cfg = DenseCfg{1, 2, use_nt(), false};
        tr = 4;
    } else if (cdiv(N, 16) * S >= 1024) {
        p.cfg = DenseCfg{4, 2, use_nt(), false};
        tr = 16;
    } else if (cdiv(N, 8) * S >= 256) {
        p.cfg = DenseCfg{2, 2, use_nt(), false};
        tr = 8;
    } else {
        p.cfg = DenseCfg{1, 2, use_nt(), false};
        tr = 4;
    }
    if (g_tune.dense_R > 0 && g_tune.dense_CH > 0) {
        p.cfg.R = (int)g_tune.dense_R;
        p.cfg.CH = (int)g_tune.dense_CH;
    }
    if (g_tune.dense_rows > 0)
        tr = (int)g_tune.dense_rows;
    p.tile_rows = tr;
    p.fuse = p.S > 1 ? split_fuse_mode() : 0;
    return p;
}

// The partials of a split linear (and, for W8A8_DYN, the scale after them),
// and the arrival counters of a fused one.
void set_part(DenseLin &L, int kind, void *part, uint32_t *ctr) {
    L.part = part;
    L.sx_part = (kind == kW8A8D && part) ? reinterpret_cast<float *>(static_cast<char *>(part) +
                                                                      (size_t)L.S * (size_t)L.N * 4)
                                         : nullptr;
    L.ctr = L.fuse ? ctr : nullptr;
}

// Split-K workspace: S partial rows, and for fp16 activations quantised in
// the kernel one more float, the scale (which the reduce kernel of the
// unfused path reads); a fused linear's arrival counters follow (zero before
// the first call, and every call leaves them zero).
size_t dense_part_bytes(int kind, const DensePlan &p, int64_t N) {
    return p.S > 1 ? (size_t)p.S * (size_t)N * 4 + (kind == kW8A8D ? 256 : 0) : 0;
}

size_t dense_ctr_bytes(const DensePlan &p, int64_t N) {
    return p.S > 1 && p.fuse ? (size_t)cdiv(N, p.tile_rows) * 4 : 0;
}

size_t dense_ws_bytes(int kind, const DensePlan &p, int64_t N) {
    const size_t pb = dense_part_bytes(kind, p, N), cb = dense_ctr_bytes(p, N);
    return cb ? (pb + 255) / 256 * 256 + cb : pb;
}

uint32_t *dense_ws_ctr(int kind, const DensePlan &p, int64_t N, void *ws) {
    if (!ws || !dense_ctr_bytes(p, N))
        return nullptr;
    return reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + (dense_part_bytes(kind, p, N) + 255) / 256 * 256);
}

DenseLin make_dense(int kind, const void *W, const void *x, float *y, void *part, const float *w_scale,
                    const float *x_scale, int32_t *acc_out, int64_t N, int64_t K, const DensePlan &p) {
    DenseLin L{};
    L.W = static_cast<const u32x4 *>(W);
    L.x = static_cast<const u32x4 *>(x);
    L.y = y;
    L.w_scale = w_scale;
    L.x_scale = x_scale;
    L.acc_out = acc_out;
    L.N = N;
    L.kvec = (int32_t)(K / elem_per_vec(kind));
    L.S = p.S;
    L.kvs = p.kvs;
    L.tile_rows = p.tile_rows;
    L.n_tiles = (int32_t)cdiv(N, p.tile_rows);
    L.fuse = p.fuse;
    set_part(L, kind, part, dense_ws_ctr(kind, p, N, part));
    return L;
}

wsg_status check_dense_args(int kind, const void *W, const void *x, const float *y, int64_t N, int64_t K,
                            int32_t splits) {
    if (N < 0 || K < 0)
        return WSG_ERR_SHAPE;
    if (N > (int64_t)INT32_MAX * 16 || K > (1LL << 28) || !grid_ok(cdiv(N, kBlock)))
        return WSG_ERR_UNSUPPORTED;
    if (K % elem_per_vec(kind))
        return WSG_ERR_SHAPE;
    if (N == 0)
        return WSG_OK;
    if (!y)
        return WSG_ERR_NULL;
    if (!aligned(y, 4))
        return WSG_ERR_ALIGN;
    if (K == 0)
        return WSG_OK;
    if (!W || !x)
        return WSG_ERR_NULL;
    if (!aligned(W, 16) || !aligned(x, 16))
        return WSG_ERR_ALIGN;
    const int64_t kvec = K / elem_per_vec(kind);
    if (splits < 0 || (splits > 0 && (splits > kvec || cdiv(kvec, splits) > kMaxSliceVec)))
        return WSG_ERR_SHAPE;
    // every slice must hold at least one vector
    if (splits > 0 && (int64_t)(splits - 1) * cdiv(kvec, splits) >= kvec)
        return WSG_ERR_SHAPE;
    const DensePlan p = plan_dense(kind, N, K, splits);
    if (!grid_ok(cdiv(N, p.tile_rows) * p.S))
        return WSG_ERR_UNSUPPORTED;
    return WSG_OK;
}



wsg_status check_ws(const void *ws, size_t ws_bytes, size_t need) {
    if (need == 0)
        return WSG_OK;
    if (!ws || ws_bytes < need)
        return WSG_ERR_WORKSPACE;
    if (!aligned(ws, 256))
        return WSG_ERR_ALIGN;
    return WSG_OK;
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

ArgOut arg_out(void *keys, int32_t n_keys, int32_t *token, float *token_logit, int32_t M = 1) {
    ArgOut a{};
    a.keys = static_cast<unsigned long long *>(keys);
    a.n_keys = n_keys;
    a.stride = arg_key_stride(n_keys);
    a.M = M;
    a.idx = token;
    a.val = token_logit;
    return a;
}

// Workgroups that publish a key for a dense linear's token: its units (or
// the last unit of each row tile), or the reduce's workgroups when a reduce
// kernel sums the split partials.
int32_t dense_token_keys(const DenseLin &L) { return L.S > 1 && !L.fuse ? dense_reduce_blocks(L.N) : L.n_tiles; }

int32_t dense_token_keys(const DensePlan &p, int64_t N) {
    return p.S > 1 && !p.fuse ? dense_reduce_blocks(N) : (int32_t)cdiv(N, p.tile_rows);
}

// Key array bytes (M rows of keys) at the start of a token-taking workspace.
size_t token_key_bytes(int32_t n_keys, int32_t M = 1) { return align256((size_t)M * arg_key_stride(n_keys) * 8); }

wsg_status check_token_args(int64_t N, const int32_t *token, const float *token_logit) {
    if (N < 1)
        return WSG_ERR_SHAPE;
    if (N > (int64_t)INT32_MAX)
        return WSG_ERR_UNSUPPORTED;
    if (!token)
        return WSG_ERR_NULL;
    if (!aligned(token, 4) || (token_logit && !aligned(token_logit, 4)))
        return WSG_ERR_ALIGN;
    return WSG_OK;
}

// Causal-conv1d step arguments: W taps (2..8), C channels (or the N of the
// linear it follows); bias optional.
wsg_status check_conv(int64_t C, int32_t W, const void *w, const float *bias, const float *state, const float *out) {
    if (C < 0)
        return WSG_ERR_SHAPE;
    if (W < 2 || W > 8 || !grid_ok(cdiv(C, kBlock)))
        return WSG_ERR_UNSUPPORTED;
    if (C == 0)
        return WSG_OK;
    if (!w || !state || !out)
        return WSG_ERR_NULL;
    if (!aligned(w, 2) || !aligned(state, 4) || !aligned(out, 4) || (bias && !aligned(bias, 4)))
        return WSG_ERR_ALIGN;
    return WSG_OK;
}

ConvOut conv_out(const void *w, const float *bias, float *state, float *out, int32_t W, int32_t silu) {
    ConvOut c{};
    c.w = static_cast<const uint16_t *>(w);
    c.bias = bias;
    c.state = state;
    c.out = out;
    c.W = W;
    c.silu = silu != 0;
    return c;
}

wsg_status enqueue_dense(int kind, const DenseLin &L, const DenseCfg &cfg, hipStream_t s) {
    hipError_t e = launch_dense(kind, L, cfg, s);
    if (e != hipSuccess)
        return hip_fail(e);
    if (L.S > 1 && !L.fuse) {
        e = launch_dense_reduce(kind, L, s);
        if (e != hipSuccess)
            return hip_fail(e);
    }
    return WSG_OK;
}

// ------------------------------------------------ allocation-free scratch --

// Device scratch of gemv_f16_static: the split-K partials live in this
// file-scope array instead of a caller workspace.  Each GPU holds its own
// copy, at its own address, until the process ends.  In host code the name
// `scratch` is only a host-side stand-in: its device address comes from
// hipGetSymbolAddress, taken once per device and kept in g_scratch_dev.
__attribute__((used)) static __device__ __align__(256) unsigned char scratch[WSG_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on its first use on
// that device, with that device current).
wsg_status static_scratch(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices)
        return WSG_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return hip_fail(e);
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return WSG_OK;
}

// ------------------------------------------------------------------- w4 --

struct W4Plan {
    W4Cfg cfg;
    int S;
    int kbs;
    int tile_rtiles;
    int fuse;       // S > 1: how the partials are summed (W4Lin::fuse)
};

W4Plan plan_w4(int64_t M, int64_t N, int64_t K, int splits) {
    const int64_t kb = K / 128;
    const int64_t n_rtiles = cdiv(N, 16);
    W4Plan p;
    p.cfg = W4Cfg{1, 4, use_nt(), false};
    // LDS holds M rows of the slice: M * kbs * 256 bytes <= 32 KiB.
    const int64_t max_kbs = std::max<int64_t>(4, (32 * 1024 / (256 * std::max<int64_t>(1, M))) / 4 * 4);
    int S;
    if (splits > 0) {
        S = splits;
    } else {
        S = (int)std::max<int64_t>(1, cdiv(kb, max_kbs));
        // underfilled: split k in whole 4-block quads
        while (n_rtiles * S < 512 && (int64_t)(S + 1) * 4 <= kb)
            ++S;
        // never leave a slice empty (slices are whole 4-block quads)
        while (S > 1 && (int64_t)(S - 1) * (cdiv(cdiv(kb, S), 4) * 4) >= kb)
            --S;
    }
    p.S = S;
    p.kbs = S > 1 ? (int)(cdiv(cdiv(kb, S), 4) * 4) : (int)kb;
    // 16-row tiles per unit: 8 (M = 1) or 16 (verify blocks), fewer when the
    // launch would otherwise have under 1024 units.
    int64_t tt = M > 1 ? 16 : 8;
    while (tt > 1 && cdiv(n_rtiles, tt) * S < kWantUnits)
        tt = tt / 2;
    if (g_tune.w4_tiles > 0)
        tt = g_tune.w4_tiles;
    p.tile_rtiles = (int)tt;
    p.fuse = p.S > 1 ? split_fuse_mode() : 0;
    if (g_tune.w4_R > 0)
        p.cfg.R = (int)g_tune.w4_R;
    if (g_tune.w4_B > 0)
        p.cfg.B = (int)g_tune.w4_B;
    return p;
}

// Split-K workspace of an int4 linear: S x M x N partials, then (fused)
// one arrival counter per row tile from the next 256-byte boundary.
size_t w4_part_bytes(const W4Plan &p, int64_t M, int64_t N) {
    return p.S > 1 ? (size_t)p.S * (size_t)M * (size_t)N * 4 : 0;
}

size_t w4_ctr_bytes(const W4Plan &p, int64_t N) {
    return p.S > 1 && p.fuse ? (size_t)cdiv(cdiv(N, 16), p.tile_rtiles) * 4 : 0;
}

W4Lin make_w4(const void *Wp, const void *Sp, const void *x, float *y, float *part, int64_t M, int64_t N,
              int64_t K, const W4Plan &p) {
    W4Lin L{};
    L.Wp = static_cast<const u32x4 *>(Wp);
    L.Sp = static_cast<const u32x2 *>(Sp);
    L.x = static_cast<const u32x4 *>(x);
    L.y = y;
    L.part = part;
    L.N = N;
    L.K = (int32_t)K;
    L.M = (int32_t)M;
    L.kb = (int32_t)(K / 128);
    L.kq = (int32_t)cdiv(L.kb, 4);
    L.S = p.S;
    L.kbs = p.kbs;
    L.tile_rtiles = p.tile_rtiles;
    L.n_tiles = (int32_t)cdiv(cdiv(N, 16), p.tile_rtiles);
    L.fuse = p.fuse;
    const size_t pb = w4_part_bytes(p, M, N);
    L.ctr = (p.fuse && part) ? reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(part) + (pb + 255) / 256 * 256)
                             : nullptr;
    return L;
}

wsg_status check_w4_args(const void *Wp, const void *Sp, const void *x, const float *y, int64_t M, int64_t N,
                         int64_t K, int64_t group, int32_t splits) {
    if (M < 0 || N < 0 || K < 0)
        return WSG_ERR_SHAPE;
    if (group != 128)
        return WSG_ERR_UNSUPPORTED;
    if (K % 128)
        return WSG_ERR_SHAPE;
    if (M < 1 || M > kMaxM)
        return M == 0 ? WSG_ERR_SHAPE : WSG_ERR_UNSUPPORTED;
    if (N > (int64_t)INT32_MAX * 16 || K > (1LL << 24) || !grid_ok(cdiv(M * N, kBlock)))
        return WSG_ERR_UNSUPPORTED;
    if (N == 0)
        return WSG_OK;
    if (!y)
        return WSG_ERR_NULL;
    if (!aligned(y, 4))
        return WSG_ERR_ALIGN;
    if (K == 0)
        return WSG_OK;
    if (!Wp || !Sp || !x)
        return WSG_ERR_NULL;
    if (!aligned(Wp, 16) || !aligned(Sp, 16) || !aligned(x, 16))
        return WSG_ERR_ALIGN;
    const int64_t kb = K / 128;
    if (splits < 0 || splits > kb)
        return WSG_ERR_SHAPE;
    if (splits > 1) {
        const int64_t kbs = cdiv(cdiv(kb, splits), 4) * 4;
        if ((int64_t)(splits - 1) * kbs >= kb)  // an empty slice
            return WSG_ERR_SHAPE;
        if ((int64_t)M * kbs * 256 > 48 * 1024)
            return WSG_ERR_SHAPE;
    } else if (splits == 1 && (int64_t)M * kb * 256 > 48 * 1024) {
        return WSG_ERR_SHAPE;
    }
    const W4Plan p = plan_w4(M, N, K, splits);
    if (!grid_ok(cdiv(cdiv(N, 16), p.tile_rtiles) * p.S))
        return WSG_ERR_UNSUPPORTED;
    return WSG_OK;
}

size_t w4_ws_bytes(const W4Plan &p, int64_t M, int64_t N) {
    const size_t pb = w4_part_bytes(p, M, N), cb = w4_ctr_bytes(p, N);
    return cb ? (pb + 255) / 256 * 256 + cb : pb;
}

wsg_status enqueue_w4(const W4Lin &L, int mode, const W4Cfg &cfg, hipStream_t s) {
    hipError_t e = launch_w4(L, mode, cfg, s);
    if (e != hipSuccess)
        return hip_fail(e);
    if (L.S > 1 && !L.fuse) {
        e = launch_w4_reduce(L, s);
        if (e != hipSuccess)
            return hip_fail(e);
    }
    return WSG_OK;
}

template <typename F>
wsg_status guarded(F &&f) {
    try {
        return f();
    } catch (const std::bad_alloc &) {
        return WSG_ERR_NOMEM;
    } catch (...) {
        return WSG_ERR_STATE;
    }
}

}  // namespace

// ================================================================ C ABI ==

extern "C" {

const char *wsg_status_string(wsg_status s) {
    switch (s) {
    case WSG_OK: return "ok";
    case WSG_ERR_NULL: return "a required pointer is NULL";
    case WSG_ERR_SHAPE: return "invalid or inconsistent shape";
    case WSG_ERR_ALIGN: return "pointer not aligned";
    case WSG_ERR_UNSUPPORTED: return "unsupported request";
    case WSG_ERR_WORKSPACE: return "workspace missing or too small";
    case WSG_ERR_HIP: return "HIP runtime error";
    case WSG_ERR_NOMEM: return "out of memory";
    case WSG_ERR_STATE: return "invalid plan state";
    default: return "unknown status";
    }
}

int32_t wsg_last_hip_error(void) { return g_last_hip; }

const char *wsg_build_info(void) { return "wsgemv for gfx950"; }

int32_t wsg_plan_splits(int32_t kind, int64_t M, int64_t N, int64_t K) {
    if (N <= 0 || K <= 0)
        return 1;
    if (kind == kF16 || kind == kW8A8 || kind == kW8A8D) {
        if (K % elem_per_vec(kind))
            return 1;
        return plan_dense(kind, N, K, 0).S;
    }
    if (kind == kW4A16 || kind == kW4A8) {
        if (K % 128 || M < 1)
            return 1;
        return plan_w4(M, N, K, 0).S;
    }
    return 1;
}

size_t wsg_workspace_bytes(int32_t kind, int64_t M, int64_t N, int64_t K, int32_t splits) {
    if (kind & WSG_WITH_ARGMAX) {
        const int32_t base = kind & ~WSG_WITH_ARGMAX;
        if ((base != kF16 && base != kW8A8) || M != 1 || N < 1 || N > (int64_t)INT32_MAX || K < 0 || splits < 0)
            return 0;
        if (K == 0 || K % elem_per_vec(base))
            return token_key_bytes(argmax_f32_blocks(N));
        const DensePlan p = plan_dense(base, N, K, splits, true);
        return token_key_bytes(dense_token_keys(p, N)) + dense_ws_bytes(base, p, N);
    }
    if (N <= 0 || K <= 0 || splits < 0)
        return 0;
    if (kind == kF16 || kind == kW8A8 || kind == kW8A8D) {
        if (K % elem_per_vec(kind))
            return 0;
        return dense_ws_bytes(kind, plan_dense(kind, N, K, splits), N);
    }
    if (kind == kW4A16 || kind == kW4A8) {
        if (K % 128 || M < 1)
            return 0;
        return w4_ws_bytes(plan_w4(M, N, K, splits), M, N);
    }
    return 0;
}

wsg_status gemv_f16(const void *W, const void *x, float *y, int64_t N, int64_t K, int32_t splits, void *ws,
                    size_t ws_bytes, wsg_stream_t stream) {
    return guarded([&]() -> wsg_status {
        wsg_status st = check_dense_args(kF16, W, x, y, N, K, splits);
        if (st != WSG_OK || N == 0)
            return st;
        hipStream_t s = static_cast<hipStream_t>(stream);
        if (K == 0) {
            hipError_t e = launch_zero_f32(y, N, s);
            return e == hipSuccess ? WSG_OK : hip_fail(e);
        }
        DensePlan p = plan_dense(kF16, N, K, splits);
        st = check_ws(ws, ws_bytes, dense_ws_bytes(kF16, p, N));
        if (st != WSG_OK)
            return st;
        DenseLin L = make_dense(kF16, W, x, y, ws, nullptr, nullptr, nullptr, N, K, p);
        p.cfg.tail = dense_needs_tail(L, p.cfg.CH);
        return enqueue_dense(kF16, L, p.cfg, s);
    });
}

wsg_status gemv_f16_static(const void *W, const void *x, float *y, int64_t N, int64_t K, int32_t splits,
                           wsg_stream_t stream) {
    return guarded([&]() -> wsg_status {
        wsg_status st = check_dense_args(kF16, W, x, y, N, K, splits);
        if (st != WSG_OK || N == 0)
            return st;
        DensePlan p = plan_dense(kF16, N, K, splits);
        p.fuse = 0;  // the shared array keeps no counters: a reduce kernel sums the partials
        const size_t need = K == 0 ? 0 : dense_ws_bytes(kF16, p, N);
        if (need > (size_t)WSG_STATIC_SCRATCH_BYTES)
            return WSG_ERR_WORKSPACE;
        hipStream_t s = static_cast<hipStream_t>(stream);
        if (K == 0) {
            hipError_t e = launch_zero_f32(y, N, s);
            return e == hipSuccess ? WSG_OK : hip_fail(e);
        }
        void *part = nullptr;
        if (need > 0) {
            st = static_scratch(&part);
            if (st != WSG_OK)
                return st;
        }
        DenseLin L = make_dense(kF16, W, x, y, part, nullptr, nullptr, nullptr, N, K, p);
        p.cfg.tail = dense_needs_tail(L, p.cfg.CH);
        return enqueue_dense(kF16, L, p.cfg, s);
    });
}

wsg_status wsg_argmax_f32(const float *y, int64_t N, int32_t *token, float *token_logit, void *ws,
                          size_t ws_bytes, wsg_stream_t stream) {
    return guarded([&]() -> wsg_status {
        wsg_status st = check_token_args(N, token, token_logit);
        if (st != WSG_OK)
            return st;
        if (!y)
            return WSG_ERR_NULL;
        if (!aligned(y, 4))
            return WSG_ERR_ALIGN;
        const int32_t nk = argmax_f32_blocks(N);
        st = check_ws(ws, ws_bytes, token_key_bytes(nk));
        if (st != WSG_OK)
            return st;
        hipError_t e = launch_argmax_f32(y, N, arg_out(ws, nk, token, token_logit), static_cast<hipStream_t>(stream));
        return e == hipSuccess ? WSG_OK : hip_fail(e);
    });
}

wsg_status causal_conv1d_step(const float *x, const void *w, const float *bias, float *state, float *out, int64_t C,
                              int32_t W, int32_t silu, wsg_stream_t stream) {
    return guarded([&]() -> wsg_status {
        wsg_status st = check_conv(C, W, w, bias, state, out);
        if (st != WSG_OK || C == 0)
            return st;
        if (!x)
            return WSG_ERR_NULL;
        if (!aligned(x, 4))
            return WSG_ERR_ALIGN;
        hipError_t e = launch_conv1d_step(x, conv_out(w, bias, state, out, W, silu), C,
                                          static_cast<hipStream_t>(stream));
        return e == hipSuccess ? WSG_OK : hip_fail(e);
    });
}

size_t wsg_topk_ws_bytes(int64_t N, int32_t k) {
    if (N < 1 || N > (int64_t)INT32_MAX || k < 1 || k > WSG_TOPK_MAX || k > N)
        return 0;
    int64_t max_keys = 0;
    topk_plan(N, k, &max_keys, nullptr);
    const size_t need = 2 * align256((size_t)max_keys * 8);
    // k = 1 runs as the greedy token (its key array must fit too)
    return k == 1 ? std::max(need, token_key_bytes(argmax_f32_blocks(N))) : need;
}

wsg_status wsg_topk_f32(const float *y, int64_t N, int32_t k, int32_t *idx, float *val, void *ws, size_t ws_bytes,
                        wsg_stream_t stream) {
    return guarded([&]() -> wsg_status {
        wsg_status st = check_token_args(N, idx, val);
        if (st != WSG_OK)
            return st;
        if (k < 1 || k > N)
            return WSG_ERR_SHAPE;
        if (k > WSG_TOPK_MAX)
            return WSG_ERR_UNSUPPORTED;
        if (!y)
            return WSG_ERR_NULL;
        if (!aligned(y, 4))
            return WSG_ERR_ALIGN;
        const size_t need = wsg_topk_ws_bytes(N, k);
        st = check_ws(ws, ws_bytes, need);
        if (st != WSG_OK)
            return st;
        hipStream_t s = static_cast<hipStream_t>(stream);
        hipError_t e;
        if (k == 1) {  // the greedy token: one reduce over y and the finish
            e = launch_argmax_f32(y, N, arg_out(ws, argmax_f32_blocks(N), idx, val), s);
        } else {
            auto *a = static_cast<unsigned long long *>(ws);
            int64_t max_keys = 0;
            topk_plan(N, k, &max_keys, nullptr);
            auto *b = reinterpret_cast<unsigned long long *>(static_cast<char *>(ws) + align256((size_t)max_keys * 8));
            e = launch_topk(y, N, k, idx, val, a, b, s);
        }
        return e == hipSuccess ? WSG_OK : hip_fail(e);
    });
}

wsg_status gemv_f16_argmax(const void *W, const void *x, float *y, int32_t *token, float *token_logit,
                           int64_t N, int64_t K, int32_t splits, void *ws, size_t ws_bytes, wsg_stream_t stream) {
    return guarded([&]() -> wsg_status {
        wsg_status st = check_dense_args(kF16, W, x, y, N, K, splits);
        if (st != WSG_OK)
            return st;
        st = check_token_args(N, token, token_logit);
        if (st != WSG_OK)
            return st;
        hipStream_t s = static_cast<hipStream_t>(stream);
        if (K == 0) {
            const int32_t nk = argmax_f32_blocks(N);
            st = check_ws(ws, ws_bytes, token_key_bytes(nk));
            if (st != WSG_OK)
                return st;
            hipError_t e = launch_zero_f32(y, N, s);
            if (e == hipSuccess)
                e = launch_argmax_f32(y, N, arg_out(ws, nk, token, token_logit), s);
            return e == hipSuccess ? WSG_OK : hip_fail(e);
        }
        DensePlan p = plan_dense(kF16, N, K, splits, true);
        const int32_t nk = dense_token_keys(p, N);
        const size_t kb = token_key_bytes(nk);
        st = check_ws(ws, ws_bytes, kb + dense_ws_bytes(kF16, p, N));
        if (st != WSG_OK)
            return st;
        DenseLin L = make_dense(kF16, W, x, y, static_cast<char *>(ws) + kb, nullptr, nullptr, nullptr, N, K, p);
        L.arg = arg_out(ws, nk, token, token_logit);
        p.cfg.tail = dense_needs_tail(L, p.cfg.CH);
        st = enqueue_dense(kF16, L, p.cfg, s);
        if (st != WSG_OK)
            return st;
        hipError_t e = launch_argmax_finish(L.arg, s);
        return e == hipSuccess ? WSG_OK : hip_fail(e);
    });
}

wsg_status gemv_w8a8(const int8_t *Wq, const float *w_scale, const int8_t *xq, const float *x_scale, float *y,
                     int32_t *acc_out, int64_t N, int64_t K, int32_t splits, void *ws, size_t ws_bytes,
                     wsg_stream_t stream) {
    return guarded([&]() -> wsg_status {
        wsg_status st = check_dense_args(kW8A8, Wq, xq, y, N, K, splits);
        if (st != WSG_OK || N == 0)
            return st;
        if (acc_out && !aligned(acc_out, 4))
            return WSG_ERR_ALIGN;
        hipStream_t s = static_cast<hipStream_t>(stream);
        if (K == 0) {
            hipError_t e = launch_zero_f32(y, N, s);
            if (e == hipSuccess && acc_out)
                e = launch_zero_f32(reinterpret_cast<float *>(acc_out), N, s);
            return e == hipSuccess ? WSG_OK : hip_fail(e);
        }
        if (!w_scale || !x_scale)
            return WSG_ERR_NULL;
        if (!aligned(w_scale, 4) || !aligned(x_scale, 4))
            return WSG_ERR_ALIGN;
        DensePlan p = plan_dense(kW8A8, N, K, splits);
        st = check_ws(ws, ws_bytes, dense_ws_bytes(kW8A8, p, N));
        if (st != WSG_OK)
            return st;
        DenseLin L = make_dense(kW8A8, Wq, xq, y, ws, w_scale, x_scale, acc_out, N, K, p);
        p.cfg.tail = dense_needs_tail(L, p.cfg.CH);
        return enqueue_dense(kW8A8, L, p.cfg, s);
    });
}

wsg_status gemv_w8a8_dyn(const int8_t *Wq, const float *w_scale, const void *x, float *y, int32_t *acc_out,
                         int8_t *xq_out, float *sx_out, int64_t N, int64_t K, int32_t splits, void *ws,
                         size_t ws_bytes, wsg_stream_t stream) {
    return guarded([&]() -> wsg_status {
        wsg_status st = check_dense_args(kW8A8D, Wq, x, y, N, K, splits);
        if (st != WSG_OK)
            return st;
        if ((acc_out && !aligned(acc_out, 4)) || (xq_out && !aligned(xq_out, 16)) || (sx_out && !aligned(sx_out, 4)))
            return WSG_ERR_ALIGN;
        if (N == 0)
            return WSG_OK;
        hipStream_t s = static_cast<hipStream_t>(stream);
        if (K == 0) {  // the empty sum, and s_x = max of nothing / 127 = 0
            hipError_t e = launch_zero_f32(y, N, s);
            if (e == hipSuccess && acc_out)
                e = launch_zero_f32(reinterpret_cast<float *>(acc_out), N, s);
            if (e == hipSuccess && sx_out)
                e = launch_zero_f32(sx_out, 1, s);
            return e == hipSuccess ? WSG_OK : hip_fail(e);
        }
        if (!w_scale)
            return WSG_ERR_NULL;
        if (!aligned(w_scale, 4))
            return WSG_ERR_ALIGN;
        DensePlan p = plan_dense(kW8A8D, N, K, splits);
        st = check_ws(ws, ws_bytes, dense_ws_bytes(kW8A8D, p, N));
        if (st != WSG_OK)
            return st;
        DenseLin L = make_dense(kW8A8D, Wq, x, y, ws, w_scale, nullptr, acc_out, N, K, p);
        L.xq_out = xq_out;
        L.sx_out = sx_out;
        p.cfg.tail = dense_needs_tail(L, p.cfg.CH);
        return enqueue_dense(kW8A8D, L, p.cfg, s);
    });
}

size_t wsg_w4_packed_weight_bytes(int64_t N, int64_t K) {
    if (N <= 0 || K <= 0 || K % 128)
        return 0;
    return (size_t)cdiv(N, 16) * 16 * (size_t)(K / 2);
}

size_t wsg_w4_packed_scale_bytes(int64_t N, int64_t K, int64_t group) {
    if (N <= 0 || K <= 0 || group != 128 || K % 128)
        return 0;
    return (size_t)cdiv(N, 16) * 16 * (size_t)cdiv(K / 128, 4) * 4 * 2;
}

wsg_status wsg_pack_w4(const uint32_t *Wc, const void *s4, void *Wp, void *Sp, int64_t N, int64_t K,
                       int64_t group, wsg_stream_t stream) {
    return guarded([&]() -> wsg_status {
        if (N < 0 || K < 0)
            return WSG_ERR_SHAPE;
        if (group != 128)
            return WSG_ERR_UNSUPPORTED;
        if (K % 128)
            return WSG_ERR_SHAPE;
        if (K > (1LL << 24) || N > (int64_t)INT32_MAX * 16 || !grid_ok(cdiv(N, 16) * (K / 128)))
            return WSG_ERR_UNSUPPORTED;
        if (N == 0 || K == 0)
            return WSG_OK;
        if (!Wc || !s4 || !Wp || !Sp)
            return WSG_ERR_NULL;
        if (!aligned(Wc, 4) || !aligned(s4, 2) || !aligned(Wp, 16) || !aligned(Sp, 16))
            return WSG_ERR_ALIGN;
        hipError_t e = launch_pack_w4(Wc, static_cast<const uint16_t *>(s4), static_cast<u32x4 *>(Wp),
                                      static_cast<u32x2 *>(Sp), N, (int32_t)K, static_cast<hipStream_t>(stream));
        return e == hipSuccess ? WSG_OK : hip_fail(e);
    });
}

wsg_status gemv_w4a16(const void *Wp, const void *Sp, const void *x, float *y, int64_t M, int64_t N, int64_t K,
                      int64_t group, int32_t splits, void *ws, size_t ws_bytes, wsg_stream_t stream) {
    return guarded([&]() -> wsg_status {
        wsg_status st = check_w4_args(Wp, Sp, x, y, M, N, K, group, splits);
        if (st != WSG_OK || N == 0)
            return st;
        hipStream_t s = static_cast<hipStream_t>(stream);
        if (K == 0) {
            hipError_t e = launch_zero_f32(y, M * N, s);
            return e == hipSuccess ? WSG_OK : hip_fail(e);
        }
        W4Plan p = plan_w4(M, N, K, splits);
        st = check_ws(ws, ws_bytes, w4_ws_bytes(p, M, N));
        if (st != WSG_OK)
            return st;
        W4Lin L = make_w4(Wp, Sp, x, y, static_cast<float *>(ws), M, N, K, p);
        p.cfg.tail = w4_needs_tail(L, p.cfg.B);
        return enqueue_w4(L, (M > 1 || g_tune.w4_mfma_m1 == 1) ? kMfma : kA16, p.cfg, s);
    });
}

wsg_status wsg_tune_set(const char *key, int64_t value) {
    if (!key)
        return WSG_ERR_NULL;
    struct {
        const char *name;
        int64_t *slot;
    } table[] = {{"nt", &g_tune.nt},
                 {"dense_R", &g_tune.dense_R},
                 {"dense_CH", &g_tune.dense_CH},
                 {"dense_rows", &g_tune.dense_rows},
                 {"group_R", &g_tune.group_R},
                 {"group_CH", &g_tune.group_CH},
                 {"group_unit_kb", &g_tune.group_unit_kb},
                 {"w4_R", &g_tune.w4_R},
                 {"w4_B", &g_tune.w4_B},
                 {"w4_tiles", &g_tune.w4_tiles},
                 {"group_w4_tiles", &g_tune.group_w4_tiles},
                 {"w4_mfma_m1", &g_tune.w4_mfma_m1},
                 {"probe_U", &g_tune.probe_U},
                 {"probe_chunked", &g_tune.probe_chunked},
                 {"chain_unit_kb", &g_tune.chain_unit_kb},
                 {"chain_blocks_per_cu", &g_tune.chain_blocks_per_cu},
                 {"chain_spin_limit", &g_tune.chain_spin_limit},
                 {"chain_test_stale", &g_tune.chain_test_stale},
                 {"chain_sleep", &g_tune.chain_sleep},
                 {"split_fuse", &g_tune.split_fuse}};
    for (auto &t : table) {
        if (std::strcmp(key, t.name) == 0) {
            *t.slot = value < 0 ? -1 : value;
            if ((g_tune.dense_R > 0 && g_tune.dense_CH > 0 &&
                 !dense_shape_ok(g_tune.dense_R, g_tune.dense_CH, false)) ||
                (g_tune.group_R > 0 && g_tune.group_CH > 0 &&
                 !dense_shape_ok(g_tune.group_R, g_tune.group_CH, true)) ||
                (g_tune.w4_R > 0 && g_tune.w4_R != 1 && g_tune.w4_R != 2) ||
                (g_tune.w4_B > 0 && g_tune.w4_B != 4 && g_tune.w4_B != 8) ||
                (g_tune.probe_U > 0 && g_tune.probe_U != 4 && g_tune.probe_U != 8 && g_tune.probe_U != 16)) {
                *t.slot = -1;
                return WSG_ERR_UNSUPPORTED;
            }
            return WSG_OK;
        }
    }
    return WSG_ERR_UNSUPPORTED;
}

wsg_status gemv_w4a8(const void *Wp, const void *Sp, const void *x, float *y, int8_t *xq_out, float *sx_out,
                     int64_t N, int64_t K, int64_t group, int32_t splits, void *ws, size_t ws_bytes,
                     wsg_stream_t stream) {
    return guarded([&]() -> wsg_status {
        wsg_status st = check_w4_args(Wp, Sp, x, y, 1, N, K, group, splits);
        if (st != WSG_OK || N == 0)
            return st;
        if ((xq_out && !aligned(xq_out, 8)) || (sx_out && !aligned(sx_out, 4)))
            return WSG_ERR_ALIGN;
        hipStream_t s = static_cast<hipStream_t>(stream);
        if (K == 0) {
            hipError_t e = launch_zero_f32(y, N, s);
            if (e == hipSuccess && sx_out)
                e = launch_zero_f32(sx_out, 1, s);
            return e == hipSuccess ? WSG_OK : hip_fail(e);
        }
        W4Plan p = plan_w4(1, N, K, splits);
        st = check_ws(ws, ws_bytes, w4_ws_bytes(p, 1, N));
        if (st != WSG_OK)
            return st;
        W4Lin L = make_w4(Wp, Sp, x, y, static_cast<float *>(ws), 1, N, K, p);
        L.xq_out = xq_out;
        L.sx_out = sx_out;
        p.cfg.tail = w4_needs_tail(L, p.cfg.B);
        return enqueue_w4(L, kA8, p.cfg, s);
    });
}

int32_t wsg_read_probe_grid(size_t bytes) {
    (void)bytes;
    return 2048;  // 8 workgroups per compute unit on 256 CUs
}

wsg_status wsg_read_probe(const void *buf, size_t bytes, float *out, int32_t grid, wsg_stream_t stream) {
    return guarded([&]() -> wsg_status {
        if (bytes % 16 || grid < 0)
            return WSG_ERR_SHAPE;
        if (!buf || !out)
            return WSG_ERR_NULL;
        if (!aligned(buf, 16) || !aligned(out, 4))
            return WSG_ERR_ALIGN;
        const int g = grid > 0 ? grid : wsg_read_probe_grid(bytes);
        const ProbeCfg pc{g_tune.probe_U > 0 ? (int)g_tune.probe_U : 8, use_nt(), g_tune.probe_chunked == 1};
        hipError_t e = launch_read_probe(static_cast<const u32x4 *>(buf), (int64_t)(bytes / 16), out, g, pc,
                                         static_cast<hipStream_t>(stream));
        return e == hipSuccess ? WSG_OK : hip_fail(e);
    });
}

}  // extern "C"

// ========================================================== decode step ==

struct wsg_step {
    int32_t mode = 0;
    bool use_graph = true;
    bool fake = false;    // built in host memory by the test mode: never launched
    hipStream_t cap = nullptr;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    void *dev = nullptr;  // one device allocation: partials, descriptor and unit tables

    struct Op {
        enum Type { kDense, kDenseGroup, kW4, kW4Group, kZero, kZero16, kArgmax, kArgFinish, kConv } type;
        int kind = 0;
        DenseLin d{};
        DenseCfg dc{};
        W4Lin w{};
        W4Cfg wc{};
        const void *lins = nullptr;   // device tables for grouped ops
        const Unit *units = nullptr;
        int n_units = 0;
        int lds = 0;
        int mode = 0;                 // W4 kernel mode (kA16, kMfma, kA8)
        float *zero_p = nullptr;
        uint16_t *zero16_p = nullptr;  // kZero16
        int64_t zero_n = 0;
        ArgOut arg{};                 // kArgmax: token over zero_p[0..zero_n); kArgFinish: token from keys
        ConvOut conv{};               // kConv: conv step over zero_p[0..zero_n)
        int fix = -1;                 // key array this op's token descriptor waits for (plan building)
    };
    std::vector<Op> ops;
    int32_t launches = 0;
    int64_t units = 0;

    // persistent dependency-respecting plan (WSG_STEP_PERSISTENT)
    bool chain = false;
    ChainArgs chain_args{};
    int chain_grid = 0;
    int chain_lds = 0;
    bool chain_tail = false;
    uint32_t chain_epoch = 0;
    uint64_t *chain_trace = nullptr;  // caller's per-unit timestamp buffer, or nullptr
};

namespace {

// ------------------------------------------------------ live plans --
// Handles of plans that exist: calls on a NULL, destroyed or foreign handle
// return WSG_ERR_STATE instead of touching freed memory.  (A new plan may
// later be allocated at the address of a destroyed one.)
std::mutex g_plans_mu;
std::unordered_set<const wsg_step *> g_plans;

void plan_register(const wsg_step *st) {
    std::lock_guard<std::mutex> lock(g_plans_mu);
    g_plans.insert(st);
}

bool plan_live(const wsg_step *st) {
    std::lock_guard<std::mutex> lock(g_plans_mu);
    return st != nullptr && g_plans.count(st) != 0;
}

bool plan_unregister(const wsg_step *st) {
    std::lock_guard<std::mutex> lock(g_plans_mu);
    return st != nullptr && g_plans.erase(st) != 0;
}

// ------------------------------------- device actions of plan creation --
// Plan creation allocates one device block, uploads its tables and may
// capture a graph.  The test mode (wsg_test_set_fault, enabled by the
// environment) builds plans in host memory instead and can make one of these
// actions fail, so that every failure path of creation runs on the CPU.
enum Fault : int { kFaultNone = 0, kFaultAlloc = 1, kFaultUpload = 2, kFaultCapture = 3 };
std::atomic<int> g_fake{0};            // 1: plans are built in host memory
std::atomic<int> g_fault{kFaultNone};  // the action that fails in the test mode
std::atomic<int64_t> g_fake_live{0};   // host blocks of test-mode plans not yet freed

hipError_t dev_alloc(wsg_step *st, size_t bytes) {
    if (st->fake) {
        if (g_fault.load() == kFaultAlloc)
            return hipErrorOutOfMemory;
        st->dev = std::malloc(std::max<size_t>(bytes, 1));
        if (!st->dev)
            return hipErrorOutOfMemory;
        ++g_fake_live;
        return hipSuccess;
    }
    hipError_t e = hipMalloc(&st->dev, bytes);
    if (e != hipSuccess)
        st->dev = nullptr;
    return e;
}

hipError_t dev_upload(wsg_step *st, const void *src, size_t bytes, hipStream_t s) {
    if (st->fake) {
        if (g_fault.load() == kFaultUpload)
            return hipErrorInvalidValue;
        std::memcpy(st->dev, src, bytes);
        return hipSuccess;
    }
    hipError_t e = hipMemcpyAsync(st->dev, src, bytes, hipMemcpyHostToDevice, s);
    return e == hipSuccess ? hipStreamSynchronize(s) : e;
}

void dev_free(wsg_step *st) {
    if (!st->dev)
        return;
    if (st->fake) {
        std::free(st->dev);
        --g_fake_live;
    } else {
        (void)hipFree(st->dev);
    }
    st->dev = nullptr;
}

// Workgroups that publish keys for an int4 linear's tokens.
int32_t w4_token_keys(const W4Lin &L) { return L.S > 1 && !L.fuse ? w4_reduce_blocks(L.M, L.N) : L.n_tiles; }

// True when some linear's x overlaps some linear's y16: the list chains
// linears, which only the ORDERED plan runs in order.
bool feeds_another(const wsg_linear *L, int32_t n) {
    for (int32_t j = 0; j < n; ++j) {
        if (!L[j].y16 || L[j].N == 0)
            continue;
        const auto *y0 = static_cast<const char *>(L[j].y16);
        const auto *y1 = y0 + (size_t)L[j].M * (size_t)L[j].N * 2;
        for (int32_t i = 0; i < n; ++i) {
            if (!L[i].x || L[i].K == 0)
                continue;
            const size_t xb = (size_t)L[i].M * (size_t)L[i].K * (L[i].kind == kW8A8 ? 1 : 2);
            const auto *x0 = static_cast<const char *>(L[i].x);
            if (x0 < y1 && y0 < x0 + xb)
                return true;
        }
    }
    return false;
}

wsg_status validate_linear(const wsg_linear &l) {
    if (l.y16 && !aligned(l.y16, 2))
        return WSG_ERR_ALIGN;
    if (l.conv_out || l.conv_w || l.conv_state || l.conv_bias || l.conv_width) {
        if (l.kind < kF16 || l.kind > kW8A8D || l.M != 1)
            return WSG_ERR_UNSUPPORTED;
        wsg_status st = check_conv(l.N, l.conv_width, l.conv_w, l.conv_bias, l.conv_state, l.conv_out);
        if (st != WSG_OK)
            return st;
    }
    if (l.argmax_idx || l.argmax_val) {
        if (l.kind < kF16 || l.kind > kW8A8D)
            return WSG_ERR_UNSUPPORTED;
        wsg_status st = check_token_args(l.N, l.argmax_idx, l.argmax_val);
        if (st != WSG_OK)
            return st;
    }
    switch (l.kind) {
    case kF16: {
        if (l.M != 1)
            return WSG_ERR_UNSUPPORTED;
        return check_dense_args(kF16, l.W, l.x, l.y, l.N, l.K, l.splits);
    }
    case kW8A8: {
        if (l.M != 1)
            return WSG_ERR_UNSUPPORTED;
        wsg_status st = check_dense_args(kW8A8, l.W, l.x, l.y, l.N, l.K, l.splits);
        if (st != WSG_OK || l.N == 0 || l.K == 0)
            return st;
        if (!l.scale || !l.x_scale)
            return WSG_ERR_NULL;
        if (!aligned(l.scale, 4) || !aligned(l.x_scale, 4) || (l.acc_out && !aligned(l.acc_out, 4)))
            return WSG_ERR_ALIGN;
        return WSG_OK;
    }
    case kW8A8D: {
        if (l.M != 1)
            return WSG_ERR_UNSUPPORTED;
        wsg_status st = check_dense_args(kW8A8D, l.W, l.x, l.y, l.N, l.K, l.splits);
        if (st != WSG_OK || l.N == 0 || l.K == 0)
            return st;
        if (l.x_scale)
            return WSG_ERR_UNSUPPORTED;  // the activation scale is computed, not given
        if (!l.scale)
            return WSG_ERR_NULL;
        if (!aligned(l.scale, 4) || (l.acc_out && !aligned(l.acc_out, 4)))
            return WSG_ERR_ALIGN;
        return WSG_OK;
    }
    case kW4A16:
        return check_w4_args(l.W, l.scale, l.x, l.y, l.M, l.N, l.K, l.group, l.splits);
    case kW4A8:
        if (l.M != 1)
            return WSG_ERR_UNSUPPORTED;
        return check_w4_args(l.W, l.scale, l.x, l.y, 1, l.N, l.K, l.group, l.splits);
    default:
        return WSG_ERR_UNSUPPORTED;
    }
}

hipError_t run_ops(const wsg_step *st, hipStream_t s) {
    for (const auto &op : st->ops) {
        hipError_t e = hipSuccess;
        switch (op.type) {
        case wsg_step::Op::kDense:
            e = launch_dense(op.kind, op.d, op.dc, s);
            if (e == hipSuccess && op.d.S > 1 && !op.d.fuse)
                e = launch_dense_reduce(op.kind, op.d, s);
            break;
        case wsg_step::Op::kDenseGroup:
            e = launch_dense_grouped(op.kind, static_cast<const DenseLin *>(op.lins), op.units, op.n_units, op.lds,
                                     op.dc, s);
            break;
        case wsg_step::Op::kW4:
            e = launch_w4(op.w, op.mode, op.wc, s);
            if (e == hipSuccess && op.w.S > 1 && !op.w.fuse)
                e = launch_w4_reduce(op.w, s);
            break;
        case wsg_step::Op::kW4Group:
            e = launch_w4_grouped(static_cast<const W4Lin *>(op.lins), op.units, op.n_units, op.lds, op.mode,
                                  op.wc, s);
            break;
        case wsg_step::Op::kZero:
            e = launch_zero_f32(op.zero_p, op.zero_n, s);
            break;
        case wsg_step::Op::kZero16:
            e = launch_zero_u16(op.zero16_p, op.zero_n, s);
            break;
        case wsg_step::Op::kArgmax:
            e = launch_argmax_f32(op.zero_p, op.zero_n, op.arg, s);
            break;
        case wsg_step::Op::kArgFinish:
            e = launch_argmax_finish(op.arg, s);
            break;
        case wsg_step::Op::kConv:
            e = launch_conv1d_step(op.zero_p, op.conv, op.zero_n, s);
            break;
        }
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

void free_step(wsg_step *st) {
    if (!st)
        return;
    if (st->exec)
        (void)hipGraphExecDestroy(st->exec);
    if (st->graph)
        (void)hipGraphDestroy(st->graph);
    if (st->cap)
        (void)hipStreamDestroy(st->cap);
    dev_free(st);
    delete st;
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Owns a plan until it is handed to the caller.
struct StepOwner {
    wsg_step *p;
    explicit StepOwner(wsg_step *s) : p(s) {}
    ~StepOwner() { free_step(p); }
    // hand the plan to the caller: it becomes a live handle
    wsg_status give(wsg_step **out) {
        plan_register(p);
        *out = p;
        p = nullptr;
        return WSG_OK;
    }
    StepOwner(const StepOwner &) = delete;
    StepOwner &operator=(const StepOwner &) = delete;
};

// The step's launch count and work units (graph or not).
void count_launches(wsg_step &st) {
    for (const auto &op : st.ops) {
        st.launches += 1;
        if (op.type == wsg_step::Op::kDense) {
            st.units += (int64_t)op.d.n_tiles * op.d.S;
            st.launches += op.d.S > 1 && !op.d.fuse;
        } else if (op.type == wsg_step::Op::kW4) {
            st.units += (int64_t)op.w.n_tiles * op.w.S;
            st.launches += op.w.S > 1 && !op.w.fuse;
        } else if (op.type == wsg_step::Op::kDenseGroup || op.type == wsg_step::Op::kW4Group) {
            st.units += op.n_units;
        } else if (op.type == wsg_step::Op::kArgmax) {
            st.launches += 1;  // the reduce over y, then the finish kernel
        }
    }
}

// Captures the step's launches into a graph on an internal stream, when the
// plan uses one.
hipError_t capture_graph(wsg_step &st) {
    if (!st.use_graph || st.ops.empty())
        return hipSuccess;
    if (st.fake) {  // the test mode never launches: the capture only fails on request
        st.use_graph = false;
        return g_fault.load() == kFaultCapture ? hipErrorStreamCaptureInvalidated : hipSuccess;
    }
    hipError_t e = hipStreamCreateWithFlags(&st.cap, hipStreamNonBlocking);
    if (e == hipSuccess)
        e = hipStreamBeginCapture(st.cap, hipStreamCaptureModeThreadLocal);
    if (e == hipSuccess) {
        hipError_t le = run_ops(&st, st.cap);
        e = hipStreamEndCapture(st.cap, &st.graph);
        if (le != hipSuccess)
            e = le;
    }
    if (e == hipSuccess)
        e = hipGraphInstantiate(&st.exec, st.graph, nullptr, nullptr, 0);
    return e;
}

wsg_status alloc_status(hipError_t e) { return e == hipErrorOutOfMemory ? WSG_ERR_NOMEM : hip_fail(e); }

// ------------------------------------------- ORDERED and GROUPED plans --

// Host-side plan of an ORDERED or GROUPED step: its launches, and for a
// GROUPED plan the work tables of each kernel kind, before the device block
// exists; then the layout of that block.
struct PlanBuild {
    int base_mode = 0;
    std::vector<DenseLin> dl[3];   // grouped dense linears per kind (F16, W8A8, W8A8D)
    std::vector<Unit> du[3];
    int dlds[3] = {0, 0, 0};
    bool dtail[3] = {false, false, false};
    std::vector<W4Lin> wl[3];      // grouped int4 linears per kernel mode (kA16, kMfma, kA8)
    std::vector<Unit> wu[3];
    int wlds[3] = {0, 0, 0};
    bool wtail[3] = {false, false, false};
    W4Cfg wcfg[3] = {};
    DenseCfg gcfg[3] = {};
    bool f16_hybrid = true;
    size_t part_bytes = 0;         // split-K partials shared by the ORDERED linears (they run in order)
    size_t ctr_bytes = 0;          // their arrival counters (fused sums), zero between linears
    // Greedy-token key arrays (one per linear that takes a token) open the
    // device block; descriptors get their addresses once it exists.
    std::vector<size_t> key_off;   // per key array: offset in the keys region
    size_t keys_bytes = 0;
    struct TableFix {
        bool w4;                   // false: dl[ki][li]; true: wl[ki][li]
        int ki, li, keys;
    };
    std::vector<TableFix> table_fix;         // grouped descriptors that take a token
    std::vector<wsg_step::Op> finish_after;  // their finish kernels, after the grouped launches
    // the device block: [token keys][partials][counters][dense tables x3][int4 tables x3]
    size_t keys_off = 0, part_off = 0, ctr_off = 0, dl_off[3] = {}, du_off[3] = {}, wl_off[3] = {}, wu_off[3] = {};
    size_t bytes = 0;

    int new_keys(int32_t n_keys, int32_t M = 1) {
        key_off.push_back(keys_bytes);
        keys_bytes += token_key_bytes(n_keys, M);
        return (int)key_off.size() - 1;
    }
};

// Grouped launches, one per kind: 8 rows x 1 vector per wave step, units of
// at least 32 rows (64 KiB at K = 1024 fp16).  An fp16 launch whose linears
// run no epilogue (token, conv) takes 2 rows x 2 vectors per step instead,
// units of about 128 KiB (64 rows at K = 1024), and of 16 KiB (8 rows) for
// linears of 16384 rows or more (the lm_head): interleaved on MI355X the
// 113-linear step took 173.0-173.5 us against 174.0-174.8 us.  With the
// lm_head taking the token that shape measured 181-182 us against
// 178.6-179.3 us (at 8-, 32- and 64-row units), so plans with epilogues keep
// the 8 x 1 shape.
void plan_config(PlanBuild &pb, const wsg_linear *L, int32_t n) {
    bool f16_epilogue = false;
    for (int32_t i = 0; i < n; ++i)
        f16_epilogue |= L[i].kind == kF16 && (L[i].argmax_idx || L[i].conv_out);
    pb.f16_hybrid = !f16_epilogue;
    for (auto &c : pb.gcfg)
        c = DenseCfg{8, 1, use_nt(), false};
    if (pb.f16_hybrid)
        pb.gcfg[0] = DenseCfg{2, 2, use_nt(), false};
    if (g_tune.group_R > 0 && g_tune.group_CH > 0) {
        for (auto &c : pb.gcfg) {
            c.R = (int)g_tune.group_R;
            c.CH = (int)g_tune.group_CH;
        }
    }
}

// A linear with K = 0: y = 0 (and its copies and epilogues) by small kernels.
void plan_k_zero(wsg_step &st, PlanBuild &pb, const wsg_linear &l) {
    wsg_step::Op z{};
    z.type = wsg_step::Op::kZero;
    z.zero_p = l.y;
    z.zero_n = (int64_t)l.M * l.N;
    st.ops.push_back(z);
    if ((l.kind == kW8A8 || l.kind == kW8A8D) && l.acc_out) {
        z.zero_p = reinterpret_cast<float *>(l.acc_out);
        z.zero_n = l.N;
        st.ops.push_back(z);
    }
    if (l.y16) {
        wsg_step::Op z16{};
        z16.type = wsg_step::Op::kZero16;
        z16.zero16_p = static_cast<uint16_t *>(l.y16);
        z16.zero_n = (int64_t)l.M * l.N;
        st.ops.push_back(z16);
    }
    if (l.conv_out) {
        wsg_step::Op c{};
        c.type = wsg_step::Op::kConv;
        c.zero_p = l.y;
        c.zero_n = l.N;
        c.conv = conv_out(l.conv_w, l.conv_bias, l.conv_state, l.conv_out, l.conv_width, l.conv_silu);
        st.ops.push_back(c);
    }
    for (int32_t m = 0; l.argmax_idx && m < l.M; ++m) {
        wsg_step::Op g{};
        g.type = wsg_step::Op::kArgmax;
        g.zero_p = l.y + (int64_t)m * l.N;
        g.zero_n = l.N;
        g.arg = arg_out(nullptr, argmax_f32_blocks(l.N), l.argmax_idx + m, l.argmax_val ? l.argmax_val + m : nullptr);
        g.fix = pb.new_keys(g.arg.n_keys);
        st.ops.push_back(g);
    }
}

// An fp16 or int8-weight linear: its own launch (ORDERED) or units of the
// kind's grouped launch (GROUPED).
wsg_status plan_dense_linear(wsg_step &st, PlanBuild &pb, const wsg_linear &l) {
    const int ki = l.kind == kF16 ? 0 : (l.kind == kW8A8 ? 1 : 2);
    if (pb.base_mode == WSG_STEP_ORDERED) {
        DensePlan p = plan_dense(l.kind, l.N, l.K, l.splits, l.argmax_idx != nullptr);
        pb.part_bytes = std::max(pb.part_bytes, dense_part_bytes(l.kind, p, l.N));
        pb.ctr_bytes = std::max(pb.ctr_bytes, dense_ctr_bytes(p, l.N));
        wsg_step::Op o{};
        o.type = wsg_step::Op::kDense;
        o.kind = l.kind;
        o.dc = p.cfg;
        o.d = make_dense(l.kind, l.W, l.x, l.y, nullptr, static_cast<const float *>(l.scale), l.x_scale, l.acc_out,
                         l.N, l.K, p);
        o.dc.tail = dense_needs_tail(o.d, o.dc.CH);
        o.d.y16 = static_cast<uint16_t *>(l.y16);
        if (l.conv_out)
            o.d.conv = conv_out(l.conv_w, l.conv_bias, l.conv_state, l.conv_out, l.conv_width, l.conv_silu);
        if (l.argmax_idx) {
            o.d.arg = arg_out(nullptr, dense_token_keys(o.d), l.argmax_idx, l.argmax_val);
            o.fix = pb.new_keys(o.d.arg.n_keys);
        }
        st.ops.push_back(o);
        if (l.argmax_idx) {
            wsg_step::Op f{};
            f.type = wsg_step::Op::kArgFinish;
            f.arg = o.d.arg;
            f.fix = o.fix;
            st.ops.push_back(f);
        }
        return WSG_OK;
    }
    DensePlan p{};
    p.cfg = pb.gcfg[ki];
    p.S = 1;
    p.kvs = (int)(l.K / elem_per_vec(l.kind));
    if (p.kvs > kMaxSliceVec)
        return WSG_ERR_UNSUPPORTED;
    {
        const int q = kWavesPerBlock * pb.gcfg[ki].R;
        int64_t unit_bytes;
        if (g_tune.group_unit_kb > 0)
            unit_bytes = g_tune.group_unit_kb * 1024;
        else if (l.kind != kF16 || !pb.f16_hybrid)
            unit_bytes = 32 * 1024;
        else
            unit_bytes = l.N >= 16384 ? 16 * 1024 : 128 * 1024;
        int64_t rows = unit_bytes / ((int64_t)p.kvs * 16);
        // short rows do not fill a wave step: at most 64 rows per unit keeps
        // such linears spread over workgroups
        if (ki == 0 && pb.f16_hybrid && g_tune.group_unit_kb <= 0)
            rows = std::min<int64_t>(rows, 64);
        p.tile_rows = (int)std::min<int64_t>(1 << 20, std::max<int64_t>(q, rows / q * q));
    }
    DenseLin L = make_dense(l.kind, l.W, l.x, l.y, nullptr, static_cast<const float *>(l.scale), l.x_scale, l.acc_out,
                            l.N, l.K, p);
    const int li = (int)pb.dl[ki].size();
    L.y16 = static_cast<uint16_t *>(l.y16);
    if (l.conv_out)
        L.conv = conv_out(l.conv_w, l.conv_bias, l.conv_state, l.conv_out, l.conv_width, l.conv_silu);
    if (l.argmax_idx) {
        L.arg = arg_out(nullptr, dense_token_keys(L), l.argmax_idx, l.argmax_val);
        wsg_step::Op f{};
        f.type = wsg_step::Op::kArgFinish;
        f.arg = L.arg;
        f.fix = pb.new_keys(L.arg.n_keys);
        pb.table_fix.push_back(PlanBuild::TableFix{false, ki, li, f.fix});
        pb.finish_after.push_back(f);
    }
    pb.dl[ki].push_back(L);
    for (int t = 0; t < L.n_tiles; ++t)
        pb.du[ki].push_back(Unit{li, t, 0, 0});
    pb.dlds[ki] = std::max(pb.dlds[ki], dense_lds_bytes(L, pb.gcfg[ki].CH));
    pb.dtail[ki] = pb.dtail[ki] || dense_needs_tail(L, pb.gcfg[ki].CH);
    return WSG_OK;
}

// An int4-weight linear: its own launch (ORDERED) or units of its kernel
// mode's grouped launch (GROUPED).
wsg_status plan_w4_linear(wsg_step &st, PlanBuild &pb, const wsg_linear &l) {
    const int wmode = l.kind == kW4A8 ? kA8 : ((l.M > 1 || g_tune.w4_mfma_m1 == 1) ? kMfma : kA16);
    if (pb.base_mode == WSG_STEP_ORDERED) {
        W4Plan p = plan_w4(l.M, l.N, l.K, l.splits);
        pb.part_bytes = std::max(pb.part_bytes, w4_part_bytes(p, l.M, l.N));
        pb.ctr_bytes = std::max(pb.ctr_bytes, w4_ctr_bytes(p, l.N));
        wsg_step::Op o{};
        o.type = wsg_step::Op::kW4;
        o.mode = wmode;
        o.wc = p.cfg;
        o.w = make_w4(l.W, l.scale, l.x, l.y, nullptr, l.M, l.N, l.K, p);
        o.wc.tail = w4_needs_tail(o.w, o.wc.B);
        o.w.y16 = static_cast<uint16_t *>(l.y16);
        if (l.conv_out)
            o.w.conv = conv_out(l.conv_w, l.conv_bias, l.conv_state, l.conv_out, l.conv_width, l.conv_silu);
        if (l.argmax_idx) {
            o.w.arg = arg_out(nullptr, w4_token_keys(o.w), l.argmax_idx, l.argmax_val, l.M);
            o.fix = pb.new_keys(o.w.arg.n_keys, l.M);
        }
        st.ops.push_back(o);
        if (l.argmax_idx) {
            wsg_step::Op f{};
            f.type = wsg_step::Op::kArgFinish;
            f.arg = o.w.arg;
            f.fix = o.fix;
            st.ops.push_back(f);
        }
        return WSG_OK;
    }
    W4Plan p = plan_w4(l.M, l.N, l.K, 1);
    p.S = 1;
    p.kbs = (int)(l.K / 128);
    // fp16 activations, M = 1: 1 tile x 8 blocks per step, 4 tiles per unit;
    // int8 activations: 1 tile x 4 blocks per step, 8 tiles per unit (the
    // per-unit quantisation is amortised over more rows); verify blocks: 2
    // tiles x 4 blocks per step, 8 tiles per unit
    const bool a8 = wmode == kA8;
    const bool mfma = wmode == kMfma;
    p.tile_rtiles = g_tune.group_w4_tiles > 0 ? (int)g_tune.group_w4_tiles : (mfma || a8 ? 8 : 4);
    p.cfg.R = g_tune.w4_R > 0 ? (int)g_tune.w4_R : (mfma ? 2 : 1);
    p.cfg.B = g_tune.w4_B > 0 ? (int)g_tune.w4_B : (mfma || a8 ? 4 : 8);
    W4Lin L = make_w4(l.W, l.scale, l.x, l.y, nullptr, l.M, l.N, l.K, p);
    if (w4_lds_bytes(L, wmode) > 64 * 1024)
        return WSG_ERR_UNSUPPORTED;
    const int li = (int)pb.wl[wmode].size();
    L.y16 = static_cast<uint16_t *>(l.y16);
    if (l.conv_out)
        L.conv = conv_out(l.conv_w, l.conv_bias, l.conv_state, l.conv_out, l.conv_width, l.conv_silu);
    if (l.argmax_idx) {
        L.arg = arg_out(nullptr, w4_token_keys(L), l.argmax_idx, l.argmax_val, l.M);
        wsg_step::Op f{};
        f.type = wsg_step::Op::kArgFinish;
        f.arg = L.arg;
        f.fix = pb.new_keys(L.arg.n_keys, l.M);
        pb.table_fix.push_back(PlanBuild::TableFix{true, wmode, li, f.fix});
        pb.finish_after.push_back(f);
    }
    pb.wl[wmode].push_back(L);
    for (int t = 0; t < L.n_tiles; ++t)
        pb.wu[wmode].push_back(Unit{li, t, 0, 0});
    pb.wlds[wmode] = std::max(pb.wlds[wmode], w4_lds_bytes(L, wmode));
    pb.wtail[wmode] = pb.wtail[wmode] || w4_needs_tail(L, p.cfg.B);
    pb.wcfg[wmode] = p.cfg;
    return WSG_OK;
}

// Every linear of the list, in order.
wsg_status plan_linears(wsg_step &st, PlanBuild &pb, const wsg_linear *L, int32_t n) {
    for (int32_t i = 0; i < n; ++i) {
        const wsg_linear &l = L[i];
        if (l.N == 0)
            continue;
        wsg_status v = WSG_OK;
        if (l.K == 0)
            plan_k_zero(st, pb, l);
        else if (l.kind == kF16 || l.kind == kW8A8 || l.kind == kW8A8D)
            v = plan_dense_linear(st, pb, l);
        else
            v = plan_w4_linear(st, pb, l);
        if (v != WSG_OK)
            return v;
    }
    // a grouped launch covers every unit of its kind
    for (int k = 0; k < 3; ++k)
        if (!grid_ok((int64_t)pb.du[k].size()) || !grid_ok((int64_t)pb.wu[k].size()))
            return WSG_ERR_UNSUPPORTED;
    return WSG_OK;
}

// Offsets of the device block's parts and its size.
void layout_block(PlanBuild &pb) {
    size_t off = 0;
    pb.keys_off = off;
    off = align_up(off + pb.keys_bytes, 256);
    pb.part_off = off;
    off = align_up(off + pb.part_bytes, 256);
    pb.ctr_off = off;  // zero in the uploaded image
    off = align_up(off + pb.ctr_bytes, 256);
    for (int k = 0; k < 3; ++k) {
        pb.dl_off[k] = off;
        off = align_up(off + pb.dl[k].size() * sizeof(DenseLin), 256);
        pb.du_off[k] = off;
        off = align_up(off + pb.du[k].size() * sizeof(Unit), 256);
    }
    for (int k = 0; k < 3; ++k) {
        pb.wl_off[k] = off;
        off = align_up(off + pb.wl[k].size() * sizeof(W4Lin), 256);
        pb.wu_off[k] = off;
        off = align_up(off + pb.wu[k].size() * sizeof(Unit), 256);
    }
    pb.bytes = off;
}

// With the device block at st.dev: the addresses of key arrays and
// partials in every descriptor, the block's host image, and the grouped
// launches (then the token finish kernels that follow them).
void fill_block(wsg_step &st, PlanBuild &pb, std::vector<char> &host) {
    char *base = static_cast<char *>(st.dev);
    auto keys_at = [&](int fix) {
        return reinterpret_cast<unsigned long long *>(base + pb.keys_off + pb.key_off[fix]);
    };
    for (const PlanBuild::TableFix &t : pb.table_fix)
        (t.w4 ? pb.wl[t.ki][t.li].arg : pb.dl[t.ki][t.li].arg).keys = keys_at(t.keys);
    for (auto &op : st.ops) {
        if (op.fix < 0)
            continue;
        if (op.type == wsg_step::Op::kDense)
            op.d.arg.keys = keys_at(op.fix);
        else if (op.type == wsg_step::Op::kW4)
            op.w.arg.keys = keys_at(op.fix);
        else
            op.arg.keys = keys_at(op.fix);
    }
    for (auto &op : pb.finish_after)
        op.arg.keys = keys_at(op.fix);
    auto put = [&](size_t o, const void *src, size_t bytes) {
        if (bytes)
            std::memcpy(host.data() + o, src, bytes);
    };
    for (int k = 0; k < 3; ++k) {
        put(pb.dl_off[k], pb.dl[k].data(), pb.dl[k].size() * sizeof(DenseLin));
        put(pb.du_off[k], pb.du[k].data(), pb.du[k].size() * sizeof(Unit));
        put(pb.wl_off[k], pb.wl[k].data(), pb.wl[k].size() * sizeof(W4Lin));
        put(pb.wu_off[k], pb.wu[k].data(), pb.wu[k].size() * sizeof(Unit));
    }
    // partials of ORDERED linears share one buffer (the ops run in order)
    for (auto &op : st.ops) {
        if (op.type == wsg_step::Op::kDense && op.d.S > 1)
            set_part(op.d, op.kind, base + pb.part_off, reinterpret_cast<uint32_t *>(base + pb.ctr_off));
        if (op.type == wsg_step::Op::kW4 && op.w.S > 1) {
            op.w.part = reinterpret_cast<float *>(base + pb.part_off);
            op.w.ctr = op.w.fuse ? reinterpret_cast<uint32_t *>(base + pb.ctr_off) : nullptr;
        }
    }
    for (int k = 0; k < 3; ++k) {
        if (pb.du[k].empty())
            continue;
        wsg_step::Op o{};
        o.type = wsg_step::Op::kDenseGroup;
        o.kind = k == 0 ? kF16 : (k == 1 ? kW8A8 : kW8A8D);
        o.dc = pb.gcfg[k];
        o.dc.tail = pb.dtail[k];
        o.lins = base + pb.dl_off[k];
        o.units = reinterpret_cast<const Unit *>(base + pb.du_off[k]);
        o.n_units = (int)pb.du[k].size();
        o.lds = pb.dlds[k];
        st.ops.push_back(o);
    }
    for (int k = 0; k < 3; ++k) {
        if (pb.wu[k].empty())
            continue;
        wsg_step::Op o{};
        o.type = wsg_step::Op::kW4Group;
        o.wc = pb.wcfg[k];
        o.wc.tail = pb.wtail[k];
        o.lins = base + pb.wl_off[k];
        o.units = reinterpret_cast<const Unit *>(base + pb.wu_off[k]);
        o.n_units = (int)pb.wu[k].size();
        o.lds = pb.wlds[k];
        o.mode = k;
        st.ops.push_back(o);
    }
    for (const auto &op : pb.finish_after)
        st.ops.push_back(op);
}

// An ORDERED or GROUPED plan: plan, lay out and allocate the device block,
// upload it, count the launches and capture them when a graph pays off.
wsg_status create_list(const wsg_linear *L, int32_t n, int32_t mode, hipStream_t s, wsg_step **out) {
    StepOwner st(new wsg_step());
    st.p->fake = g_fake.load() != 0;
    st.p->mode = mode;
    st.p->use_graph = !(mode & WSG_STEP_EAGER);
    PlanBuild pb;
    pb.base_mode = mode & 0xFF;
    plan_config(pb, L, n);
    wsg_status v = plan_linears(*st.p, pb, L, n);
    if (v != WSG_OK)
        return v;
    layout_block(pb);
    std::vector<char> host(pb.bytes);
    if (pb.bytes > 0) {
        hipError_t e = dev_alloc(st.p, pb.bytes);
        if (e != hipSuccess)
            return alloc_status(e);
    }
    fill_block(*st.p, pb, host);
    if (pb.bytes > 0) {
        hipError_t e = dev_upload(st.p, host.data(), pb.bytes, s);
        if (e != hipSuccess)
            return hip_fail(e);
    }
    count_launches(*st.p);
    // a graph pays off only when it replaces enough direct launches
    if (!(mode & WSG_STEP_FORCE_GRAPH) && st.p->launches < WSG_STEP_GRAPH_MIN_LAUNCHES)
        st.p->use_graph = false;
    hipError_t e = capture_graph(*st.p);
    if (e != hipSuccess)
        return hip_fail(e);
    return st.give(out);
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const auto *p = static_cast<const char *>(a), *q = static_cast<const char *>(b);
    return na > 0 && nb > 0 && p < q + nb && q < p + na;
}

// Largest input a persistent unit stages (16-byte vectors): K <= 4096.
constexpr int kChainMaxVec = 512;
constexpr uint32_t kChainSpinLimit = 1u << 18;
// Workgroups per compute unit (at most the resident count): on MI355X the C3
// chain took 568-571 us with 3 or 4, 580-595 with 1 or 2.
constexpr int kChainBlocksPerCu = 4;

// The persistent dependency-respecting plan: see WSG_STEP_PERSISTENT.
wsg_status create_chain(const wsg_linear *L, int32_t n, hipStream_t s, wsg_step **out) {
    // every linear: fp16, M = 1, whole k, no epilogue, K <= 4096
    for (int32_t i = 0; i < n; ++i) {
        const wsg_linear &l = L[i];
        if (l.kind != kF16 || l.M != 1 || l.splits > 1 || l.argmax_idx || l.argmax_val || l.conv_out)
            return WSG_ERR_UNSUPPORTED;
        if (l.N > 0 && (l.K == 0 || l.K / 8 > kChainMaxVec))
            return WSG_ERR_UNSUPPORTED;
    }
    // where each input comes from: nowhere in the list (a plain input), or
    // wholly inside the fp16 output of one earlier linear
    std::vector<int> prod(n, -1);
    std::vector<int64_t> prod_off(n, 0);
    std::vector<char> feeds(n, 0);
    for (int32_t i = 0; i < n; ++i) {
        const wsg_linear &l = L[i];
        if (l.N == 0)
            continue;
        const size_t xb = (size_t)l.K * 2;
        for (int32_t j = 0; j < n; ++j) {
            if (L[j].N == 0)
                continue;
            if (overlaps(l.x, xb, L[j].y, (size_t)L[j].N * 4))
                return WSG_ERR_UNSUPPORTED;  // fp32 outputs never feed, and are never overwritten while read
            if (!L[j].y16 || !overlaps(l.x, xb, L[j].y16, (size_t)L[j].N * 2))
                continue;
            const auto *x0 = static_cast<const char *>(l.x), *y0 = static_cast<const char *>(L[j].y16);
            // whole 8-value groups of the producer's outputs (aligned 64-bit tagged loads)
            const bool inside = x0 >= y0 && x0 + xb <= y0 + (size_t)L[j].N * 2 && (x0 - y0) % 16 == 0;
            if (j >= i || !inside || prod[i] >= 0)
                return WSG_ERR_UNSUPPORTED;
            prod[i] = j;
            prod_off[i] = (x0 - y0) / 2;
            feeds[j] = 1;
        }
    }

    constexpr int chunk = kWave * 2;  // the kernel's vectors per row step
    int max_nx = 0;
    bool tail = false;
    for (int32_t i = 0; i < n; ++i) {
        if (L[i].N == 0)
            continue;
        const int kvec = (int)(L[i].K / 8);
        max_nx = std::max(max_nx, (kvec + chunk - 1) / chunk * chunk);
        tail = tail || kvec % chunk != 0;
    }
    const int lds = 2 * max_nx * 16;
    int dev = 0, cus = 256, per_cu = kChainBlocksPerCu;  // the test mode's stand-in device
    if (!g_fake.load()) {
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess)
            e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e == hipSuccess)
            e = chain_blocks_per_cu(lds, tail, &per_cu);
        if (e != hipSuccess)
            return hip_fail(e);
    }
    const int cap = g_tune.chain_blocks_per_cu > 0 ? (int)g_tune.chain_blocks_per_cu : kChainBlocksPerCu;
    if (wsg_chain_grid(INT64_MAX, per_cu, cus, cap) < 1)
        return WSG_ERR_UNSUPPORTED;

    // units: whole rows, sized so that each linear spreads over the grid
    std::vector<ChainLin> lins;
    std::vector<Unit> units;
    std::vector<int> lin_of(n, -1);
    for (int32_t i = 0; i < n; ++i) {
        const wsg_linear &l = L[i];
        if (l.N == 0)
            continue;
        // about 32 KiB of weights per unit: both of a unit's first weight
        // steps cover most of it, so little streaming is left once its input
        // arrives; on MI355X the C3 chain took 568 us with 32 KiB units
        // against 588 with units of the linear's bytes over the grid (16 to
        // 128 KiB), 680 with 64 KiB and 896 with 128 KiB
        const int64_t row_bytes = l.K * 2;
        const int64_t want = g_tune.chain_unit_kb > 0 ? g_tune.chain_unit_kb * 1024 : 32 * 1024;
        int64_t rows = std::max<int64_t>(8, want / row_bytes / 8 * 8);
        rows = std::min<int64_t>(rows, cdiv(l.N, 8) * 8);
        ChainLin c{};
        c.W = static_cast<const u32x4 *>(l.W);
        c.x = static_cast<const u32x4 *>(l.x);
        c.y = l.y;
        c.y16 = static_cast<uint16_t *>(l.y16);
        c.N = l.N;
        c.kvec = (int32_t)(l.K / 8);
        c.tile_rows = (int32_t)rows;
        c.n_tiles = (int32_t)cdiv(l.N, rows);
        lin_of[i] = (int)lins.size();
        for (int t = 0; t < c.n_tiles; ++t)
            units.push_back(Unit{lin_of[i], t, 0, 0});
        lins.push_back(c);
    }
    if (!grid_ok((int64_t)units.size()))
        return WSG_ERR_UNSUPPORTED;

    // device block: [control][tagged outputs][linears][units]
    size_t off = 0;
    const size_t ctl_off = off;
    off = align_up(off + sizeof(ChainCtl), 256);
    std::vector<size_t> tag_off(n, 0);
    for (int32_t i = 0; i < n; ++i) {
        if (!feeds[i])
            continue;
        tag_off[i] = off;
        off = align_up(off + (size_t)L[i].N * 4, 256);
    }
    const size_t lin_off = off;
    off = align_up(off + lins.size() * sizeof(ChainLin), 256);
    const size_t unit_off = off;
    off = align_up(off + units.size() * sizeof(Unit), 256);

    StepOwner st(new wsg_step());
    st.p->fake = g_fake.load() != 0;
    st.p->mode = WSG_STEP_PERSISTENT;
    st.p->use_graph = false;
    st.p->chain = true;
    hipError_t e = dev_alloc(st.p, off);
    if (e != hipSuccess)
        return alloc_status(e);
    char *base = static_cast<char *>(st.p->dev);
    for (int32_t i = 0; i < n; ++i) {
        if (lin_of[i] < 0)
            continue;
        ChainLin &c = lins[lin_of[i]];
        if (feeds[i])
            c.tag_out = reinterpret_cast<uint32_t *>(base + tag_off[i]);
        if (prod[i] >= 0) {
            c.x_tag = reinterpret_cast<const uint32_t *>(base + tag_off[prod[i]]) + prod_off[i];
            c.x = nullptr;
        }
    }
    std::vector<char> host(off, 0);  // the control block and every tag start at zero
    if (!lins.empty())
        std::memcpy(host.data() + lin_off, lins.data(), lins.size() * sizeof(ChainLin));
    if (!units.empty())
        std::memcpy(host.data() + unit_off, units.data(), units.size() * sizeof(Unit));
    e = dev_upload(st.p, host.data(), off, s);
    if (e != hipSuccess)
        return hip_fail(e);

    ChainArgs &a = st.p->chain_args;
    a.lins = reinterpret_cast<const ChainLin *>(base + lin_off);
    a.units = reinterpret_cast<const Unit *>(base + unit_off);
    a.ctl = reinterpret_cast<ChainCtl *>(base + ctl_off);
    a.n_units = (int32_t)units.size();
    a.xs_vecs = max_nx;
    st.p->chain_grid = (int)wsg_chain_grid((int64_t)units.size(), per_cu, cus, cap);
    st.p->chain_lds = lds;
    st.p->chain_tail = tail;
    st.p->units = (int64_t)units.size();
    st.p->launches = units.empty() ? 0 : 1;
    return st.give(out);
}

hipError_t run_chain(wsg_step *st, hipStream_t s) {
    if (st->chain_args.n_units == 0)
        return hipSuccess;
    if (++st->chain_epoch == 0)
        st->chain_epoch = 1;
    ChainArgs &a = st->chain_args;
    a.epoch = st->chain_epoch;
    a.tag = (st->chain_epoch - 1) % 65535u + 1u;
    a.want = g_tune.chain_test_stale == 1 ? a.tag % 65535u + 1u : a.tag;
    a.spin_limit = g_tune.chain_spin_limit >= 0 ? (uint32_t)std::min<int64_t>(g_tune.chain_spin_limit, UINT32_MAX)
                                                : kChainSpinLimit;
    // polling again at once measured fastest on the C3 chain (sleeps of 2, 8
    // and 16 between polls cost 1, 3 and 7 %)
    a.sleep = g_tune.chain_sleep >= 0 ? (int)std::min<int64_t>(g_tune.chain_sleep, 64) : 0;
    a.trace = st->chain_trace;
    return launch_chain(a, st->chain_grid, st->chain_lds, st->chain_tail, s);
}

}  // namespace

extern "C" {

wsg_status wsg_decode_step_create(const wsg_linear *linears, int32_t n, int32_t mode, wsg_stream_t stream,
                                  wsg_step **out) {
    return guarded([&]() -> wsg_status {
        if (!out)
            return WSG_ERR_NULL;
        *out = nullptr;
        if (n < 0)
            return WSG_ERR_SHAPE;
        if (n > 0 && !linears)
            return WSG_ERR_NULL;
        const int base_mode = mode & 0xFF;
        if (base_mode != WSG_STEP_ORDERED && base_mode != WSG_STEP_GROUPED && base_mode != WSG_STEP_PERSISTENT)
            return WSG_ERR_UNSUPPORTED;
        if (mode & ~(0xFF | WSG_STEP_EAGER | WSG_STEP_FORCE_GRAPH))
            return WSG_ERR_UNSUPPORTED;
        if ((mode & WSG_STEP_EAGER) && (mode & WSG_STEP_FORCE_GRAPH))
            return WSG_ERR_UNSUPPORTED;
        if (base_mode == WSG_STEP_PERSISTENT && mode != WSG_STEP_PERSISTENT)
            return WSG_ERR_UNSUPPORTED;  // one direct launch per step: no graph flags
        for (int32_t i = 0; i < n; ++i) {
            wsg_status v = validate_linear(linears[i]);
            if (v != WSG_OK)
                return v;
            if (base_mode == WSG_STEP_GROUPED && linears[i].splits > 1)
                return WSG_ERR_UNSUPPORTED;
        }
        hipStream_t s = static_cast<hipStream_t>(stream);
        if (base_mode == WSG_STEP_PERSISTENT)
            return create_chain(linears, n, s, out);
        if (base_mode == WSG_STEP_GROUPED && feeds_another(linears, n))
            return WSG_ERR_UNSUPPORTED;
        return create_list(linears, n, mode, s, out);
    });
}

wsg_status decode_step_linears(wsg_step *step, wsg_stream_t stream) {
    return guarded([&]() -> wsg_status {
        if (!plan_live(step) || step->fake)
            return WSG_ERR_STATE;
        hipStream_t s = static_cast<hipStream_t>(stream);
        hipError_t e = hipSuccess;
        if (step->chain)
            e = run_chain(step, s);
        else if (step->exec)
            e = hipGraphLaunch(step->exec, s);
        else
            e = run_ops(step, s);
        return e == hipSuccess ? WSG_OK : hip_fail(e);
    });
}

wsg_status wsg_decode_step_destroy(wsg_step *step) {
    return guarded([&]() -> wsg_status {
        if (!plan_unregister(step))
            return WSG_ERR_STATE;
        free_step(step);
        return WSG_OK;
    });
}

wsg_status wsg_decode_step_status(wsg_step *step, wsg_stream_t stream, uint32_t *give_ups) {
    return guarded([&]() -> wsg_status {
        if (!plan_live(step))
            return WSG_ERR_STATE;
        if (!give_ups)
            return WSG_ERR_NULL;
        *give_ups = 0;
        if (!step->chain || step->fake)
            return WSG_OK;
        hipStream_t s = static_cast<hipStream_t>(stream);
        ChainCtl *ctl = step->chain_args.ctl;
        uint32_t v = 0;
        hipError_t e = hipStreamSynchronize(s);
        if (e == hipSuccess)
            e = hipMemcpy(&v, &ctl->give_ups, sizeof(v), hipMemcpyDeviceToHost);
        if (e == hipSuccess && v != 0)
            e = hipMemset(&ctl->give_ups, 0, sizeof(v));
        if (e != hipSuccess)
            return hip_fail(e);
        *give_ups = v;
        return WSG_OK;
    });
}

wsg_status wsg_decode_step_trace(wsg_step *step, uint64_t *trace, int64_t capacity) {
    return guarded([&]() -> wsg_status {
        if (!plan_live(step))
            return WSG_ERR_STATE;
        if (!step->chain)
            return WSG_ERR_UNSUPPORTED;
        if (trace == nullptr) {
            step->chain_trace = nullptr;
            return WSG_OK;
        }
        if (!aligned(trace, 8))
            return WSG_ERR_ALIGN;
        if (capacity < 4 * step->units)
            return WSG_ERR_SHAPE;
        step->chain_trace = trace;
        return WSG_OK;
    });
}

int64_t wsg_chain_grid(int64_t units, int32_t blocks_per_cu, int32_t cus, int32_t cap_per_cu) {
    if (units <= 0 || blocks_per_cu <= 0 || cus <= 0)
        return 0;
    const int64_t per = cap_per_cu > 0 ? std::min(blocks_per_cu, cap_per_cu) : blocks_per_cu;
    return std::min(units, per * (int64_t)cus);
}

wsg_status wsg_decode_step_info(const wsg_step *step, int32_t *launches, int64_t *units, int32_t *graph) {
    if (!plan_live(step))
        return WSG_ERR_STATE;
    if (launches)
        *launches = step->launches;
    if (units)
        *units = step->units;
    if (graph)
        *graph = step->exec != nullptr;
    return WSG_OK;
}

wsg_status wsg_test_set_fault(int32_t mode) {
    const char *env = std::getenv("WSG_ENABLE_TEST_HOOKS");
    if (!env || std::strcmp(env, "1") != 0)
        return WSG_ERR_UNSUPPORTED;
    if (mode < -1 || mode > kFaultCapture)
        return WSG_ERR_SHAPE;
    g_fake.store(mode >= 0 ? 1 : 0);
    g_fault.store(mode >= 0 ? mode : kFaultNone);
    return WSG_OK;
}

int64_t wsg_test_live_blocks(void) { return g_fake_live.load(); }

}  // extern "C"
