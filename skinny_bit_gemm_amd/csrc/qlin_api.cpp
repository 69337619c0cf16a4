// qlin_api.cpp -- the C ABI: argument validation, schedule planning and
// dispatch to the gfx950 kernels.  Every check runs before the first HIP
// call, so a rejected call touches neither the device nor the stream.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <new>

#include <hip/hip_runtime_api.h>

#include "qlin_internal.h"

namespace qlin {
namespace {

thread_local int g_last_hip_error = 0;

bool fmt_ok(int fmt) { return fmt == QLIN_FP8_DYNAMIC || fmt == QLIN_W8A8_INT8 || fmt == QLIN_BLOCK_FP8; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// int32 sums of int8 products stay exact while 127 * 127 * K < 2^31
constexpr int kMaxKInt8 = 133120;
constexpr int kMaxDim = 1 << 20;

qlin_status shape_ok(int fmt, int M, int N, int K) {
    if (M < 0 || M > kMaxDim || N < 16 || N > kMaxDim || K < 16 || K > kMaxDim) return QLIN_ERR_SHAPE;
    if (N % 16 != 0 || K % 16 != 0) return QLIN_ERR_SHAPE;
    if (fmt == QLIN_BLOCK_FP8 && (N % kGroup != 0 || K % kGroup != 0)) return QLIN_ERR_SHAPE;
    if (fmt == QLIN_W8A8_INT8 && K > kMaxKInt8) return QLIN_ERR_SHAPE;
    return QLIN_OK;
}

// The format argument of the GEMM calls: a number format, optionally with
// QLIN_PACKED_WEIGHTS (the weight codes' layout) OR-ed in.
qlin_format base_format(qlin_format f) { return (qlin_format)((int)f & ~QLIN_PACKED_WEIGHTS); }
bool packed_weights(qlin_format f) { return ((int)f & QLIN_PACKED_WEIGHTS) != 0; }

qlin_status hip_status(hipError_t e) {
    if (e == hipSuccess) return QLIN_OK;
    g_last_hip_error = (int)e;
    return QLIN_ERR_HIP;
}

qlin_status resolve_config(qlin_format fmt, int M, int N, int K, const qlin_config *cfg,
                           qlin_config *out) {
    if (cfg) {
        *out = *cfg;
        return QLIN_OK;
    }
    bool found = false;
    qlin_status st = table_lookup(fmt, M, N, K, out, &found);
    if (st != QLIN_OK) return st;
    if (found) return QLIN_OK;
    if (strict_mode()) return QLIN_ERR_NO_CONFIG;
    st = table_nearest(fmt, M, N, K, out, &found);
    if (st != QLIN_OK) return st;
    if (found) return QLIN_OK;
    default_config(fmt, M, N, K, out);
    return QLIN_OK;
}

}  // namespace

// workspace: [arrival counters][packed int64 sums, or one slice of 32-bit
// partial sums per partition]; all of it is zero between calls
static void set_workspace(Plan *p, int M, int N) {
    if (p->nsplit > 1) {
        p->ws_counter_bytes = align256((size_t)p->n_tiles * p->m_tiles * 4);
        const size_t sums = p->packed ? (size_t)M * N * 8 : (size_t)p->nsplit * M * N * 4;
        p->ws_bytes = p->ws_counter_bytes + align256(sums);
    } else {
        p->ws_counter_bytes = 0;
        p->ws_bytes = 0;
    }
}

qlin_status make_plan(qlin_format fmt, int M, int N, int K, const qlin_config &c, bool fused,
                      Plan *p, bool grouped) {
    if (!fmt_ok(fmt)) return QLIN_ERR_INVALID_ARG;
    if (M < 1) M = 1;
    if (c.swap_ab != 0 && c.swap_ab != 1) return QLIN_ERR_INVALID_ARG;
    if (c.split_k < 1 || c.split_k > kMaxSplit) return QLIN_ERR_INVALID_ARG;
    if (c.tile_m != 16 && c.tile_m != 32 && c.tile_m != 64 && c.tile_m != 128) return QLIN_ERR_INVALID_ARG;
    if (c.waves < 1 || c.waves > kMaxWaves) return QLIN_ERR_INVALID_ARG;
    if (c.k_waves < 1 || c.k_waves > c.waves || c.waves % c.k_waves != 0) return QLIN_ERR_INVALID_ARG;
    if (c.reduce != 0 && c.reduce != 1) return QLIN_ERR_INVALID_ARG;
    if (c.act_path < QLIN_ACT_STAGED || c.act_path > QLIN_ACT_DIRECT) return QLIN_ERR_INVALID_ARG;
    // int8 sums (K <= 133120) and fp8 sums in units of 2^-18 stay below 2^51
    // in magnitude while K <= 40960: only those partials can be added as
    // packed 64-bit integers
    if (c.reduce == 1 && !(fmt == QLIN_W8A8_INT8 || (fmt == QLIN_FP8_DYNAMIC && K <= 40960)))
        return QLIN_ERR_INVALID_ARG;
    const bool fuse = fused && c.act_path == QLIN_ACT_FUSED;
    const bool direct = c.act_path == QLIN_ACT_DIRECT;
    if (c.act_path == QLIN_ACT_FUSED && c.tile_m != 16) return QLIN_ERR_INVALID_ARG;
    if (direct && c.tile_m >= 64) return QLIN_ERR_INVALID_ARG;   // 16- or 32-token tiles only
    // The large-M kernel: 64- or 128-token tiles of 128 channels, 4 waves in
    // a 2 x 2 grid, Standard operand roles, slice reduction, static LDS.  A
    // 64-token tile with any other layout is the skinny kernel's.
    const bool big_layout = c.tile_n == 128 && c.waves == 4 && c.k_waves == 1 && c.swap_ab == 0 &&
                            c.reduce == 0 && c.act_path == QLIN_ACT_STAGED;
    if (c.tile_m == 128 || (c.tile_m == 64 && big_layout)) {
        if (!big_layout) return QLIN_ERR_INVALID_ARG;
        if (!gemm_variant_exists(fmt, false, c.tile_m, 0, 0)) return QLIN_ERR_INVALID_ARG;
        p->tile_m = c.tile_m;
        p->tile_n = 128;
        p->sub_rows = 16;
        p->nr = 0;
        p->nw = 2;
        p->kw = 1;
        p->waves = 4;
        p->fuse = 0;
        p->xc = 0;
        p->nkb = (K + kGroup - 1) / kGroup;
        p->kb_per_split = (p->nkb + c.split_k - 1) / c.split_k;
        p->nsplit = (p->nkb + p->kb_per_split - 1) / p->kb_per_split;
        p->phase_blocks = p->kb_per_split;
        p->lds_bytes = 0;
        p->n_tiles = (N + 127) / 128;
        p->m_tiles = (M + c.tile_m - 1) / c.tile_m;
        p->packed = 0;
        set_workspace(p, M, N);
        return QLIN_OK;
    }
    const int nw = c.waves / c.k_waves;
    // weight sub-tiles of 16 rows (the matrix core's), or of 8 rows where
    // tile_n = 8 x nw: the other 8 rows of each sub-tile read zeros, which
    // doubles the workgroups a narrow layer spreads over
    if (c.tile_n < 8 || c.tile_n > 256) return QLIN_ERR_INVALID_ARG;
    int sub_rows = 16;
    if (c.tile_n % (16 * nw) != 0) {
        if (c.tile_n != 8 * nw) return QLIN_ERR_INVALID_ARG;
        sub_rows = 8;
    }
    const int nr = c.tile_n / (sub_rows * nw);
    const int mt = c.tile_m / 16;
    p->tile_m = c.tile_m;
    p->tile_n = c.tile_n;
    p->sub_rows = sub_rows;
    p->nr = nr;
    p->nw = nw;
    p->kw = c.k_waves;
    p->waves = c.waves;
    p->fuse = fuse;
    p->nkb = (K + kGroup - 1) / kGroup;
    p->kb_per_split = (p->nkb + c.split_k - 1) / c.split_k;
    p->nsplit = (p->nkb + p->kb_per_split - 1) / p->kb_per_split;
    // activation codes of the tile's existing token rows (128 bytes per row
    // and K block, and one more 16-byte slot per row, which makes the row
    // stride odd) plus, for the block format, one fp32 scale per row and block
    // A launch with at most one workgroup per compute unit may use most of
    // the CU's LDS: fewer phases, so the weight stream runs dry less often
    // (the stream stops at each phase boundary); measured 3-12 % faster
    // at 16-32 tokens on the 8B- and 32B-class layers.
    const int rows = M < c.tile_m ? M : c.tile_m;
    const int per_block = rows * kGroup + (fmt == QLIN_BLOCK_FP8 ? rows * 4 : 0);
    const int64_t wgs = (int64_t)((N + c.tile_n - 1) / c.tile_n) * ((M + c.tile_m - 1) / c.tile_m) * p->nsplit;
    const int budget = !grouped && wgs <= kComputeUnits ? kLdsBudgetOnePerCU : kLdsBudget;
    int pb = (budget - rows * 16) / per_block;
    if (pb > p->kb_per_split || direct) pb = p->kb_per_split;   // direct: nothing staged, one phase
    p->phase_blocks = pb;
    // In-kernel quantization: one phase (the workgroup's K range fits the
    // LDS), and the tile's activation chunks of 8 values, spread over the
    // workgroup's threads, fit in 8 register chunks per thread: whole rows
    // for the per-token formats (the amax is over all of K; rows are padded
    // to a multiple of 64 chunks), the range for the block format.
    int xc = 0;
    if (fuse) {
        if (pb < p->kb_per_split) return QLIN_ERR_INVALID_ARG;
        const int chunks = fmt == QLIN_BLOCK_FP8 ? p->kb_per_split * 16 : (K / 8 + 63) / 64 * 64;
        const int threads = 64 * c.waves;
        const int need = (rows * chunks + threads - 1) / threads;
        xc = need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : 0;
        if (xc == 0) return QLIN_ERR_INVALID_ARG;
    }
    if (direct) xc = -1;
    p->xc = xc;
    if (!gemm_variant_exists(fmt, c.swap_ab != 0, c.tile_m, nr, xc)) return QLIN_ERR_INVALID_ARG;
    size_t lds = direct ? 0 : (size_t)pb * per_block + (size_t)rows * 16;
    const size_t red = (size_t)(c.k_waves - 1) * nw * nr * mt * 64 * 16;
    if (red > lds) lds = red;
    p->lds_bytes = lds;
    p->n_tiles = (N + c.tile_n - 1) / c.tile_n;
    p->m_tiles = (M + c.tile_m - 1) / c.tile_m;
    p->packed = p->nsplit > 1 && c.reduce == 1;
    set_workspace(p, M, N);
    return QLIN_OK;
}

}  // namespace qlin

using namespace qlin;

extern "C" {

qlin_status qlin_quantize_act(qlin_format fmt, int M, int K, const void *x, int64_t ldx, void *xq,
                              float *x_scales, void *stream) {
    if (!fmt_ok(fmt)) return QLIN_ERR_INVALID_ARG;
    if (M < 0 || M > kMaxDim || K < 16 || K > kMaxDim || K % 16 != 0) return QLIN_ERR_SHAPE;
    if (fmt == QLIN_BLOCK_FP8 && K % kGroup != 0) return QLIN_ERR_SHAPE;
    if (ldx < K || ldx % 8 != 0) return QLIN_ERR_ALIGNMENT;
    if (!x || !xq || !x_scales) return QLIN_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(xq) || !aligned4(x_scales)) return QLIN_ERR_ALIGNMENT;
    if (M == 0) return QLIN_OK;
    return hip_status(launch_quant_act(fmt, M, K, x, ldx, xq, x_scales,
                                       static_cast<hipStream_t>(stream)));
}

qlin_status qlin_quantize_act_cfg(qlin_format fmt, int M, int K, const void *x, int64_t ldx, void *xq,
                                  float *x_scales, int threads, void *stream) {
    if (!fmt_ok(fmt)) return QLIN_ERR_INVALID_ARG;
    if (threads != 0 && !quant_threads_valid(fmt, threads)) return QLIN_ERR_INVALID_ARG;
    if (M < 0 || M > kMaxDim || K < 16 || K > kMaxDim || K % 16 != 0) return QLIN_ERR_SHAPE;
    if (fmt == QLIN_BLOCK_FP8 && K % kGroup != 0) return QLIN_ERR_SHAPE;
    if (ldx < K || ldx % 8 != 0) return QLIN_ERR_ALIGNMENT;
    if (!x || !xq || !x_scales) return QLIN_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(xq) || !aligned4(x_scales)) return QLIN_ERR_ALIGNMENT;
    if (M == 0) return QLIN_OK;
    return hip_status(launch_quant_act(fmt, M, K, x, ldx, xq, x_scales, static_cast<hipStream_t>(stream),
                                       threads));
}

qlin_status qlin_quantize_weight(qlin_format fmt, int N, int K, const float *w, void *wq,
                                 float *w_scales, void *stream) {
    if (!fmt_ok(fmt)) return QLIN_ERR_INVALID_ARG;
    qlin_status st = shape_ok(fmt, 1, N, K);
    if (st != QLIN_OK) return st;
    if (!w || !wq || !w_scales) return QLIN_ERR_INVALID_ARG;
    if (!aligned16(w) || !aligned16(wq) || !aligned4(w_scales)) return QLIN_ERR_ALIGNMENT;
    return hip_status(launch_quant_weight(fmt, N, K, w, wq, w_scales,
                                          static_cast<hipStream_t>(stream)));
}

qlin_status qlin_validate_config(qlin_format fmt, int M, int N, int K, const qlin_config *cfg) {
    fmt = base_format(fmt);   // the weight layout does not change the schedule
    if (!fmt_ok(fmt)) return QLIN_ERR_INVALID_ARG;
    qlin_status st = shape_ok(fmt, M, N, K);
    if (st != QLIN_OK) return st;
    if (!cfg) return QLIN_ERR_INVALID_ARG;
    Plan p;
    return make_plan(fmt, M, N, K, *cfg, true, &p);
}

qlin_status qlin_select_variant(qlin_format fmt, int M, int N, int K, qlin_config *out) {
    fmt = base_format(fmt);   // the weight layout does not change the schedule
    if (!fmt_ok(fmt)) return QLIN_ERR_INVALID_ARG;
    if (!out) return QLIN_ERR_INVALID_ARG;
    qlin_status st = shape_ok(fmt, M, N, K);
    if (st != QLIN_OK) return st;
    return resolve_config(fmt, M, N, K, nullptr, out);
}

qlin_status qlin_workspace_bytes(qlin_format fmt, int M, int N, int K, const qlin_config *cfg,
                                 size_t *bytes) {
    fmt = base_format(fmt);   // the weight layout does not change the schedule
    if (!fmt_ok(fmt) || !bytes) return QLIN_ERR_INVALID_ARG;
    qlin_status st = shape_ok(fmt, M, N, K);
    if (st != QLIN_OK) return st;
    qlin_config c;
    st = resolve_config(fmt, M, N, K, cfg, &c);
    if (st != QLIN_OK) return st;
    Plan p;
    st = make_plan(fmt, M, N, K, c, true, &p);
    if (st != QLIN_OK) return st;
    *bytes = p.ws_bytes;
    return QLIN_OK;
}

// Checks shared by qlin_gemm and qlin_linear (everything but the
// activations and the workspace); fills *c and *p.
static qlin_status check_gemm_args(qlin_format fmt, int M, int N, int K, const float *x_scales,
                                   const void *wq, const float *w_scales, void *y,
                                   qlin_out_type out_type, const qlin_config *cfg, bool fused,
                                   qlin_config *c, Plan *p) {
    if (!fmt_ok(fmt)) return QLIN_ERR_INVALID_ARG;
    if (out_type != QLIN_OUT_BF16 && out_type != QLIN_OUT_F32_ACC && out_type != QLIN_OUT_I32_ACC)
        return QLIN_ERR_INVALID_ARG;
    if (out_type == QLIN_OUT_I32_ACC && fmt != QLIN_W8A8_INT8) return QLIN_ERR_INVALID_ARG;
    qlin_status st = shape_ok(fmt, M, N, K);
    if (st != QLIN_OK) return st;
    if (!x_scales || !wq || !w_scales || !y) return QLIN_ERR_INVALID_ARG;
    if (!aligned16(wq) || !aligned16(y) || !aligned4(x_scales) || !aligned4(w_scales))
        return QLIN_ERR_ALIGNMENT;
    st = resolve_config(fmt, M, N, K, cfg, c);
    if (st != QLIN_OK) return st;
    return make_plan(fmt, M, N, K, *c, fused, p);
}

static qlin_status check_workspace(const Plan &p, void *workspace, size_t ws_bytes) {
    if (p.ws_bytes > 0) {
        if (!workspace || ws_bytes < p.ws_bytes) return QLIN_ERR_WORKSPACE;
        if (!aligned16(workspace)) return QLIN_ERR_ALIGNMENT;
    }
    return QLIN_OK;
}

static qlin_status check_gemm(qlin_format fmt, int M, int N, int K, const float *x_scales,
                              const void *wq, const float *w_scales, void *y,
                              qlin_out_type out_type, const qlin_config *cfg, void *workspace,
                              size_t ws_bytes, bool fused, qlin_config *c, Plan *p) {
    qlin_status st = check_gemm_args(fmt, M, N, K, x_scales, wq, w_scales, y, out_type, cfg, fused, c, p);
    if (st != QLIN_OK) return st;
    return check_workspace(*p, workspace, ws_bytes);
}

static GemmLaunch launch_args(const Plan &p, int M, int N, int K, const void *wq, bool w_packed,
                              const float *w_scales, void *y, qlin_out_type out_type,
                              void *workspace) {
    GemmLaunch g = {};
    g.w_packed = w_packed;
    g.w_group_stride = w_packed ? packed_weight_bytes(N, K) : (int64_t)N * K;
    g.wq = static_cast<const uint8_t *>(wq);
    g.wsc = w_scales;
    g.y = y;
    g.counters = p.ws_bytes ? static_cast<uint32_t *>(workspace) : nullptr;
    g.acc_ws = p.ws_bytes ? static_cast<char *>(workspace) + p.ws_counter_bytes : nullptr;
    g.M = M;
    g.N = N;
    g.K = K;
    g.nkb = p.nkb;
    g.kb_per_split = p.kb_per_split;
    g.nsplit = p.nsplit;
    g.phase_blocks = p.phase_blocks;
    g.out_type = out_type;
    g.packed = p.packed;
    g.n_tiles = p.n_tiles;
    g.m_tiles = p.m_tiles;
    g.nw = p.nw;
    g.kw = p.kw;
    g.sub_rows = p.sub_rows;
    g.slice = (int64_t)M * N;
    return g;
}

qlin_status qlin_gemm(qlin_format fmt, int M, int N, int K, const void *xq, const float *x_scales,
                      const void *wq, const float *w_scales, void *y, qlin_out_type out_type,
                      const qlin_config *cfg, void *workspace, size_t ws_bytes, void *stream) {
    const bool wpk = packed_weights(fmt);
    fmt = base_format(fmt);
    qlin_config c;
    Plan p;
    qlin_status st = check_gemm(fmt, M, N, K, x_scales, wq, w_scales, y, out_type, cfg, workspace,
                                ws_bytes, false, &c, &p);
    if (st != QLIN_OK) return st;
    if (!xq) return QLIN_ERR_INVALID_ARG;
    if (!aligned16(xq)) return QLIN_ERR_ALIGNMENT;
    if (M == 0) return QLIN_OK;
    GemmLaunch g = launch_args(p, M, N, K, wq, wpk, w_scales, y, out_type, workspace);
    g.xq = static_cast<const uint8_t *>(xq);
    g.xs = x_scales;
    return hip_status(launch_gemm(fmt, c.swap_ab != 0, c.tile_m, p.nr, p.xc, g, p.lds_bytes,
                                  static_cast<hipStream_t>(stream)));
}

// Validates a qlin_linear call (everything but the workspace) and plans it:
// fills *c and *p, with the in-kernel quantization turned off where the
// tile's rows of x are too far apart for its 32-bit offsets.
static qlin_status plan_linear(qlin_format fmt, int M, int N, int K, const void *x, int64_t ldx,
                               void *xq, const float *x_scales, const void *wq, const float *w_scales,
                               void *y, qlin_out_type out_type, const qlin_config *cfg, qlin_config *c,
                               Plan *p) {
    qlin_status st = check_gemm_args(fmt, M, N, K, x_scales, wq, w_scales, y, out_type, cfg, true, c, p);
    if (st != QLIN_OK) return st;
    if (!x || !xq) return QLIN_ERR_INVALID_ARG;
    if (ldx < K || ldx % 8 != 0) return QLIN_ERR_ALIGNMENT;
    if (!aligned16(x) || !aligned16(xq)) return QLIN_ERR_ALIGNMENT;
    // the in-kernel quantization addresses the tile's rows of x with 32-bit
    // byte offsets; a very wide row stride takes the two-kernel path
    if (p->fuse && ((int64_t)((M < c->tile_m ? M : c->tile_m) - 1) * ldx + K) * 2 >= ((int64_t)1 << 31)) {
        c->act_path = QLIN_ACT_STAGED;
        st = make_plan(fmt, M, N, K, *c, true, p);
        if (st != QLIN_OK) return st;
    }
    return QLIN_OK;
}

// Enqueues a planned qlin_linear call (quantize + GEMM, or the fused GEMM).
static qlin_status run_linear(qlin_format fmt, int M, int N, int K, const void *x, int64_t ldx, void *xq,
                              float *x_scales, const void *wq, bool w_packed, const float *w_scales, void *y,
                              qlin_out_type out_type, const qlin_config &c, const Plan &p, void *workspace,
                              hipStream_t s) {
    GemmLaunch g = launch_args(p, M, N, K, wq, w_packed, w_scales, y, out_type, workspace);
    if (p.fuse) {
        g.x = static_cast<const uint16_t *>(x);
        g.ldx = ldx;
        g.xq_out = static_cast<uint8_t *>(xq);
        g.xs_out = x_scales;
    } else {
        qlin_status st = hip_status(launch_quant_act(fmt, M, K, x, ldx, xq, x_scales, s));
        if (st != QLIN_OK) return st;
        g.xq = static_cast<const uint8_t *>(xq);
        g.xs = x_scales;
    }
    return hip_status(launch_gemm(fmt, c.swap_ab != 0, c.tile_m, p.nr, p.xc, g, p.lds_bytes, s));
}

qlin_status qlin_linear(qlin_format fmt, int M, int N, int K, const void *x, int64_t ldx, void *xq,
                        float *x_scales, const void *wq, const float *w_scales, void *y,
                        qlin_out_type out_type, const qlin_config *cfg, void *workspace,
                        size_t ws_bytes, void *stream) {
    const bool wpk = packed_weights(fmt);
    fmt = base_format(fmt);
    qlin_config c;
    Plan p;
    qlin_status st = plan_linear(fmt, M, N, K, x, ldx, xq, x_scales, wq, w_scales, y, out_type, cfg, &c, &p);
    if (st != QLIN_OK) return st;
    st = check_workspace(p, workspace, ws_bytes);
    if (st != QLIN_OK) return st;
    if (M == 0) return QLIN_OK;
    return run_linear(fmt, M, N, K, x, ldx, xq, x_scales, wq, wpk, w_scales, y, out_type, c, p, workspace,
                      static_cast<hipStream_t>(stream));
}

qlin_status qlin_linear_scratch(qlin_format fmt, int M, int N, int K, const void *x, int64_t ldx, void *xq,
                                float *x_scales, const void *wq, const float *w_scales, void *y,
                                qlin_out_type out_type, const qlin_config *cfg, void *stream) {
    const bool wpk = packed_weights(fmt);
    fmt = base_format(fmt);
    qlin_config c;
    Plan p;
    qlin_status st = plan_linear(fmt, M, N, K, x, ldx, xq, x_scales, wq, w_scales, y, out_type, cfg, &c, &p);
    if (st != QLIN_OK) return st;
    if (p.ws_bytes > kScratchBytes) return QLIN_ERR_WORKSPACE;
    if (M == 0) return QLIN_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void *ws = nullptr;
    if (p.ws_bytes > 0) {
        st = hip_status(static_scratch(s, &ws));
        if (st != QLIN_OK) return st;
    }
    return run_linear(fmt, M, N, K, x, ldx, xq, x_scales, wq, wpk, w_scales, y, out_type, c, p, ws, s);
}

// ---------------------------------------------------------------- grouped

// Built-in rule for grouped launches.  The groups already give the grid
// many workgroups (active groups x channel tiles), so no split: 16- or
// 32-token tiles (the largest group decides), Swap-AB, 64-column tiles of
// four waves with two K waves.  Three cases differ, all measured on the
// 128-expert layers:
// - at most 2 rows per group and K >= 2048: 32-column tiles with four K
//   waves (twice the workgroups, each wave's K range halved), ~10% faster;
// - more than 2 rows per group and K <= 1024: 48-column tiles of three
//   waves, each with the whole K range (a short K split over waves leaves
//   each wave a few blocks and adds a reduction), 15-20% faster on
//   768-deep rows from 32 tokens on, a few % for the block format;
// - 32-token tiles on longer rows: Standard operand roles, 2-7% faster at
//   24-32 tokens.
static void grouped_default_config(int max_group_rows, int K, qlin_config *c) {
    const int tm = max_group_rows <= 16 ? 16 : 32;
    if (max_group_rows <= 2 && K >= 2048) *c = qlin_config{1, 1, 16, 32, 4, 4, 0, 0};
    else if (max_group_rows > 2 && K <= 1024) *c = qlin_config{1, 1, tm, 48, 3, 1, 0, 0};
    else if (tm == 32) *c = qlin_config{0, 1, 32, 64, 4, 2, 0, 0};
    else *c = qlin_config{1, 1, 16, 64, 4, 2, 0, 0};
}

// Token tiles of a grouped launch: tiles of min(tile_m, max_group_rows)
// rows (the rows the LDS staging is sized for).  Group e has
// ceil(rows_e / tile rows) of them, fewer than rows_e / tile rows + 1, so
// ceil(total_rows / tile rows) + (groups with rows) bounds every routing.
static int64_t grouped_grid_y(int groups, int total_rows, int group_rows) {
    return (total_rows + (int64_t)group_rows - 1) / group_rows + std::min(groups, total_rows);
}

// Plans a grouped launch; the workspace holds one arrival counter per
// (token tile, channel tile) and the split-K sums of all rows.
static qlin_status grouped_plan(qlin_format fmt, int groups, int N, int K, int total_rows,
                                int max_group_rows, const qlin_config *cfg, qlin_config *c, Plan *p) {
    if (!fmt_ok(fmt)) return QLIN_ERR_INVALID_ARG;
    if (groups < 1 || groups > kMaxDim || total_rows < 0 || total_rows > kMaxDim || max_group_rows < 1)
        return QLIN_ERR_SHAPE;
    qlin_status st = shape_ok(fmt, max_group_rows, N, K);
    if (st != QLIN_OK) return st;
    if (cfg) *c = *cfg;
    else grouped_default_config(max_group_rows, K, c);
    // the skinny kernel only (16- or 32-token tiles), codes quantized beforehand
    if (c->tile_m > 32 || c->act_path == QLIN_ACT_FUSED) return QLIN_ERR_INVALID_ARG;
    st = make_plan(fmt, max_group_rows, N, K, *c, false, p, true);
    if (st != QLIN_OK) return st;
    p->m_tiles = (int)std::min<int64_t>(grouped_grid_y(groups, total_rows, std::min(c->tile_m, max_group_rows)),
                                        INT32_MAX);
    if (p->m_tiles > 65535) return QLIN_ERR_SHAPE;   // grid y
    if (p->nsplit > 1) {
        p->ws_counter_bytes = align256((size_t)p->m_tiles * p->n_tiles * 4);
        const size_t sums = p->packed ? (size_t)total_rows * N * 8 : (size_t)p->nsplit * total_rows * N * 4;
        p->ws_bytes = p->ws_counter_bytes + align256(sums);
    } else {
        p->ws_counter_bytes = 0;
        p->ws_bytes = 0;
    }
    return QLIN_OK;
}

qlin_status qlin_grouped_select_variant(qlin_format fmt, int groups, int N, int K, int max_group_rows,
                                        qlin_config *out) {
    fmt = base_format(fmt);
    if (!out) return QLIN_ERR_INVALID_ARG;
    Plan p;
    return grouped_plan(fmt, groups, N, K, 0, max_group_rows, nullptr, out, &p);
}

qlin_status qlin_grouped_workspace_bytes(qlin_format fmt, int groups, int N, int K, int total_rows,
                                         int max_group_rows, const qlin_config *cfg, size_t *bytes) {
    fmt = base_format(fmt);
    if (!bytes) return QLIN_ERR_INVALID_ARG;
    qlin_config c;
    Plan p;
    const qlin_status st = grouped_plan(fmt, groups, N, K, total_rows, max_group_rows, cfg, &c, &p);
    if (st != QLIN_OK) return st;
    *bytes = p.ws_bytes;
    return QLIN_OK;
}

qlin_status qlin_grouped_gemm(qlin_format fmt, int groups, int N, int K, const int *group_offsets,
                              int total_rows, int max_group_rows, const void *xq, const float *x_scales,
                              const void *wq, const float *w_scales, void *y, qlin_out_type out_type,
                              const qlin_config *cfg, void *workspace, size_t ws_bytes, void *stream) {
    const bool wpk = packed_weights(fmt);
    fmt = base_format(fmt);
    if (out_type != QLIN_OUT_BF16 && out_type != QLIN_OUT_F32_ACC && out_type != QLIN_OUT_I32_ACC)
        return QLIN_ERR_INVALID_ARG;
    if (out_type == QLIN_OUT_I32_ACC && fmt != QLIN_W8A8_INT8) return QLIN_ERR_INVALID_ARG;
    qlin_config c;
    Plan p;
    qlin_status st = grouped_plan(fmt, groups, N, K, total_rows, max_group_rows, cfg, &c, &p);
    if (st != QLIN_OK) return st;
    if (!group_offsets || !xq || !x_scales || !wq || !w_scales || !y) return QLIN_ERR_INVALID_ARG;
    if (!aligned4(group_offsets) || !aligned16(xq) || !aligned16(wq) || !aligned16(y) ||
        !aligned4(x_scales) || !aligned4(w_scales))
        return QLIN_ERR_ALIGNMENT;
    if (p.ws_bytes && (!workspace || ws_bytes < p.ws_bytes)) return QLIN_ERR_WORKSPACE;
    if (p.ws_bytes && !aligned16(workspace)) return QLIN_ERR_ALIGNMENT;
    if (total_rows == 0) return QLIN_OK;
    GemmLaunch g = launch_args(p, total_rows, N, K, wq, wpk, w_scales, y, out_type, workspace);
    g.xq = static_cast<const uint8_t *>(xq);
    g.xs = x_scales;
    g.group_off = group_offsets;
    g.groups = groups;
    g.group_rows = std::min(c.tile_m, max_group_rows);
    g.m_tiles = p.m_tiles;   // grid y
    return hip_status(launch_gemm(fmt, c.swap_ab != 0, c.tile_m, p.nr, p.xc, g, p.lds_bytes,
                                  static_cast<hipStream_t>(stream)));
}

qlin_status qlin_packed_weight_bytes(int N, int K, size_t *bytes) {
    if (!bytes) return QLIN_ERR_INVALID_ARG;
    if (N < 16 || N > kMaxDim || K < 16 || K > kMaxDim || N % 16 != 0 || K % 16 != 0) return QLIN_ERR_SHAPE;
    *bytes = (size_t)packed_weight_bytes(N, K);
    return QLIN_OK;
}

qlin_status qlin_pack_weight(int batch, int N, int K, const void *wq, void *wq_packed, void *stream) {
    if (batch < 0 || batch > 65535) return QLIN_ERR_SHAPE;
    if (N < 16 || N > kMaxDim || K < 16 || K > kMaxDim || N % 16 != 0 || K % 16 != 0) return QLIN_ERR_SHAPE;
    if (!wq || !wq_packed) return QLIN_ERR_INVALID_ARG;
    if (!aligned16(wq) || !aligned16(wq_packed)) return QLIN_ERR_ALIGNMENT;
    if (batch == 0) return QLIN_OK;
    return hip_status(launch_pack_weight(batch, N, K, wq, wq_packed, static_cast<hipStream_t>(stream)));
}

struct qlin_graph_s {
    hipGraphExec_t exec;
};

qlin_status qlin_graph_begin(void *stream) {
    if (!stream) return QLIN_ERR_INVALID_ARG;
    return hip_status(hipStreamBeginCapture(static_cast<hipStream_t>(stream),
                                            hipStreamCaptureModeThreadLocal));
}

qlin_status qlin_graph_end(void *stream, qlin_graph *graph) {
    if (!stream || !graph) return QLIN_ERR_INVALID_ARG;
    hipGraph_t g = nullptr;
    qlin_status st = hip_status(hipStreamEndCapture(static_cast<hipStream_t>(stream), &g));
    if (st != QLIN_OK) return st;
    hipGraphExec_t exec = nullptr;
    st = hip_status(hipGraphInstantiate(&exec, g, nullptr, nullptr, 0));
    (void)hipGraphDestroy(g);   // the executable graph keeps what it needs
    if (st != QLIN_OK) return st;
    qlin_graph h = new (std::nothrow) qlin_graph_s;
    if (!h) {
        (void)hipGraphExecDestroy(exec);
        return QLIN_ERR_INVALID_ARG;
    }
    h->exec = exec;
    *graph = h;
    return QLIN_OK;
}

qlin_status qlin_graph_launch(qlin_graph graph, void *stream) {
    if (!graph) return QLIN_ERR_INVALID_ARG;
    return hip_status(hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream)));
}

qlin_status qlin_graph_destroy(qlin_graph graph) {
    if (!graph) return QLIN_ERR_INVALID_ARG;
    qlin_status st = hip_status(hipGraphExecDestroy(graph->exec));
    delete graph;
    return st;
}

const char *qlin_status_str(qlin_status st) {
    switch (st) {
    case QLIN_OK: return "ok";
    case QLIN_ERR_INVALID_ARG: return "invalid argument";
    case QLIN_ERR_ALIGNMENT: return "misaligned pointer or stride";
    case QLIN_ERR_SHAPE: return "unsupported shape";
    case QLIN_ERR_WORKSPACE: return "workspace missing or too small";
    case QLIN_ERR_NO_CONFIG: return "no tuned configuration for this shape (strict mode)";
    case QLIN_ERR_TABLE: return "selection table unreadable or malformed";
    case QLIN_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

int qlin_abi_version(void) { return QLIN_ABI_VERSION; }

int qlin_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
