/*
 * qlin.h -- C ABI of the MI355X (gfx950) quantized skinny linear layer.
 *
 * One quantized linear layer y[M,N] = dequant(quant(x)[M,K] . W_q[N,K]^T)
 * for LLM decode at small token counts M, in the three 8-bit formats of
 * "Building a High-Performance and Portable vLLM Linear Backend with Helion",
 * section "Scope":
 *   QLIN_FP8_DYNAMIC  fp8 E4M3 codes, one activation scale per token
 *                     (computed at run time), one weight scale per output
 *                     channel;
 *   QLIN_W8A8_INT8    int8 codes, the same scale granularity, int32 sums;
 *   QLIN_BLOCK_FP8    fp8 E4M3 codes, one activation scale per token and
 *                     128-wide K group (1x128), one weight scale per 128x128
 *                     block of W.
 * The product is the one of section "Kernel Implementation" (out = a @ b
 * with a wide accumulator); Standard, Split-K and Swap-AB are schedules of
 * it that give the same result, chosen per shape and token count from an
 * offline table (sections "Kernel Implementation" and "Per-shape Config
 * Tuning").
 *
 * Numbers: fp8 is OCP E4M3FN (largest finite 448, no infinity); int8 is
 * symmetric in [-127, 127].  A scale is amax / qmax as one fp32 division
 * (qmax = 448 or 127); a zero run has scale 0 and all-zero codes.  A code is
 * the fp32 quotient x / scale rounded to nearest-even and saturated.
 *
 * Conventions for every call:
 *   - all tensor arguments are device pointers (hipMalloc'ed or torch CUDA
 *     tensors), dense row-major unless a leading dimension is given, owned by
 *     the caller; the library never allocates, frees, synchronizes or reads
 *     device memory on the host inside these calls;
 *   - `stream` is a hipStream_t (NULL = the default stream); work is only
 *     enqueued on it, so every call may be captured into a hipGraph;
 *   - arguments are validated before any HIP call; on error nothing is
 *     enqueued and a qlin_status other than QLIN_OK is returned; nothing
 *     aborts and nothing throws across this interface;
 *   - device pointers must be 16-byte aligned; K must be a multiple of 16
 *     (128 for QLIN_BLOCK_FP8, which also needs N % 128 == 0);
 *   - activations must be finite; results for inf/NaN inputs are unspecified.
 */
#ifndef QLIN_H
#define QLIN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QLIN_ABI_VERSION 1
/* Largest token count served by the tuned decode path (the pages' hybrid
 * dispatch threshold, section "Hybrid Dispatch"). */
#define QLIN_MAX_DECODE_M 32

typedef enum {
    QLIN_FP8_DYNAMIC = 0,
    QLIN_W8A8_INT8 = 1,
    QLIN_BLOCK_FP8 = 2
} qlin_format;

/* Weight layout flag: OR-ed into the format argument of qlin_gemm,
 * qlin_linear, qlin_linear_scratch and qlin_grouped_gemm (and accepted,
 * without effect, by the schedule queries), it says that wq holds the codes
 * in the packed layout of qlin_pack_weight instead of [N, K] row-major.
 * Results are identical; only the memory traffic pattern changes. */
#define QLIN_PACKED_WEIGHTS 0x100

typedef enum {
    QLIN_OUT_BF16 = 0,    /* y: bf16 [M,N], the product                     */
    QLIN_OUT_F32_ACC = 1, /* y: fp32 [M,N], scaled sums before bf16 rounding */
    QLIN_OUT_I32_ACC = 2  /* y: int32 [M,N], raw sums (W8A8_INT8 only)       */
} qlin_out_type;

typedef enum {
    QLIN_OK = 0,
    QLIN_ERR_INVALID_ARG = 1, /* null pointer, unknown enum, bad config      */
    QLIN_ERR_ALIGNMENT = 2,   /* pointer not 16-byte aligned or bad stride   */
    QLIN_ERR_SHAPE = 3,       /* M, N, K out of range or not multiples       */
    QLIN_ERR_WORKSPACE = 4,   /* workspace missing or too small              */
    QLIN_ERR_NO_CONFIG = 5,   /* strict mode: no table entry for this shape  */
    QLIN_ERR_TABLE = 6,       /* table file unreadable, malformed, wrong arch */
    QLIN_ERR_HIP = 7          /* a HIP runtime call failed                   */
} qlin_status;

/* act_path values of qlin_config */
#define QLIN_ACT_STAGED 0
#define QLIN_ACT_FUSED 1
#define QLIN_ACT_DIRECT 2

/* One schedule of the contraction (section "Kernel Implementation": the
 * split_k and swap_ab tunables, plus the tile shape and how the pieces are
 * put back together).
 *   swap_ab    0: tokens fill the matrix-core row operand (Standard);
 *              1: weight rows fill it and the result is transposed back,
 *                 y = (W_q . x_q^T)^T (Swap-AB).
 *   split_k    number of K partitions handled by separate workgroups, 1..64;
 *              each covers ceil(K / split_k) rounded up to 128 (the effective
 *              count can be lower).
 *   tile_m     tokens per tile: 16, 32 or 64 (the skinny kernel; 64 with
 *              codes staged in the LDS only, act_path 0, and 1 or 2
 *              sub-tiles per wave), or 64 or 128 with tile_n 128, waves 4,
 *              k_waves 1, swap_ab 0, reduce 0 and act_path 0 (the large-M
 *              kernel for token counts past the skinny range; 128 takes only
 *              that layout, and that exact layout with 64 selects it).
 *   tile_n     output channels per workgroup, <= 256: 1, 2 or 4 times
 *              16 x (waves / k_waves) (16-row weight sub-tiles, the matrix
 *              core's), or exactly 8 x (waves / k_waves) (8-row sub-tiles:
 *              twice the workgroups for the same layer).
 *   waves      64-lane waves per workgroup: 1 to 8.  Column-wave counts
 *              (waves / k_waves) of 3, 5, 6 or 7 give tile widths such as
 *              24, 48, 96 or 224 that split a layer's N into about one tile
 *              per compute unit.
 *   k_waves    how many of those waves split the workgroup's K range
 *              (the rest split tile_n); divides waves.
 *   reduce     how Split-K partitions are combined: 0 = every partition
 *              stores its partial sums in its own workspace slice and the
 *              last to arrive adds them in partition order (any format);
 *              1 = exact packed 64-bit integer atomics (W8A8_INT8, and
 *              FP8_DYNAMIC with K <= 40960).  Both give results that do
 *              not depend on the order partitions finish in.
 *   act_path   how the GEMM workgroups get their activation codes:
 *              QLIN_ACT_STAGED (0): quantized beforehand (qlin_linear
 *                enqueues qlin_quantize_act first) and copied into the
 *                LDS in K-block stages that all of the workgroup's waves
 *                read;
 *              QLIN_ACT_FUSED (1), qlin_linear only (qlin_gemm takes it
 *                as 0): each workgroup quantizes the rows it needs itself
 *                (one kernel instead of two; needs tile_m 16, the K range
 *                in one LDS stage and the tile's activation rows within 8
 *                register chunks of 8 values per thread);
 *              QLIN_ACT_DIRECT (2): quantized beforehand, and each wave
 *                loads the fragments of its own K blocks from memory with
 *                the weight blocks they multiply (no LDS stage and no
 *                prologue that waits for one); the skinny kernel only
 *                (tile_m 16 or 32), and for QLIN_BLOCK_FP8 only with
 *                swap_ab 1.                                                  */
typedef struct {
    int32_t swap_ab;
    int32_t split_k;
    int32_t tile_m;
    int32_t tile_n;
    int32_t waves;
    int32_t k_waves;
    int32_t reduce;
    int32_t act_path;
} qlin_config;

/* Activation quantization (per token, or per token and 1x128 group for
 * QLIN_BLOCK_FP8), the dynamic step of section "Scope".
 *   x        bf16 [M, ldx] (row stride ldx >= K elements, ldx % 8 == 0)
 *   xq       [M, K] codes: int8 (W8A8_INT8) or fp8 E4M3 bytes
 *   x_scales fp32 [M], or [M][K/128] for QLIN_BLOCK_FP8
 * M may be 0 (nothing is enqueued). */
qlin_status qlin_quantize_act(qlin_format fmt, int M, int K, const void *x, int64_t ldx,
                              void *xq, float *x_scales, void *stream);

/* qlin_quantize_act with the kernel's launch shape chosen by the caller (the
 * small config set the built-in rule picks from, exposed for measuring it):
 *   threads  per-token formats: threads per token row, 64, 128, 256 or 512
 *            (one wave per row needs no exchange between waves);
 *            QLIN_BLOCK_FP8: threads per workgroup, 64 or 256 (16 per group);
 *            0: the built-in rule (what qlin_quantize_act does).
 * Codes and scales do not depend on it.  Other values: QLIN_ERR_INVALID_ARG. */
qlin_status qlin_quantize_act_cfg(qlin_format fmt, int M, int K, const void *x, int64_t ldx,
                                  void *xq, float *x_scales, int threads, void *stream);

/* Weight quantization (offline preparation; same rules, one scale per output
 * channel, or per 128x128 block for QLIN_BLOCK_FP8).
 *   w        fp32 [N, K], row n = output channel n
 *   wq       [N, K] codes
 *   w_scales fp32 [N], or [N/128][K/128] for QLIN_BLOCK_FP8 */
qlin_status qlin_quantize_weight(qlin_format fmt, int N, int K, const float *w, void *wq,
                                 float *w_scales, void *stream);

/* Packed weight layout (offline preparation, like the quantization): the
 * codes of each 16-row x 128-K block of W become 2 KiB of consecutive
 * bytes, in the order in which the GEMM kernels' 64-lane waves hold them,
 * so that every weight load of a wave reads 1 KiB of consecutive memory.
 * For 16-row group s, K block kb (nkb = ceil(K / 128) blocks), half h and
 * lane l, the 16 bytes at offset 1024 ((s nkb + kb) 2 + h) + 16 l are codes
 * [16 s + l % 16][128 kb + 32 (l / 16) + 16 h + 0 .. 15] of the row-major
 * matrix, zeros past K.  The product ("Building a High-Performance and
 * Portable vLLM Linear Backend with Helion", section "Kernel
 * Implementation") does not depend on how the weights are stored.
 *   batch      matrices back to back (a grouped layer's experts): wq is
 *              [batch][N][K], wq_packed [batch][qlin_packed_weight_bytes]
 *   N, K       multiples of 16
 * wq and wq_packed must not overlap.  batch 0 enqueues nothing. */
qlin_status qlin_packed_weight_bytes(int N, int K, size_t *bytes);
qlin_status qlin_pack_weight(int batch, int N, int K, const void *wq, void *wq_packed, void *stream);

/* The quantized GEMM y = dequant(xq . wq^T).
 *   xq, x_scales  as produced by qlin_quantize_act
 *   wq, w_scales  as produced by qlin_quantize_weight ([N,K] row-major), or
 *                 wq packed by qlin_pack_weight with QLIN_PACKED_WEIGHTS in fmt
 *   y             [M, N] row-major of the out_type's element type
 *   cfg           NULL: look the schedule up with qlin_select_variant;
 *                 otherwise that schedule is forced (it must be valid)
 *   workspace     needed when the schedule splits K: at least
 *                 qlin_workspace_bytes(...) bytes, zero-filled before its
 *                 first use; every call leaves it zero again, so one buffer
 *                 can serve calls of any shape and schedule that fit it.
 *                 Calls that overlap in time must not share a workspace.
 * Returns QLIN_ERR_NO_CONFIG in strict mode when cfg is NULL and the table
 * has no entry for (fmt, N, K, bucket(M)). */
qlin_status qlin_gemm(qlin_format fmt, int M, int N, int K, const void *xq,
                      const float *x_scales, const void *wq, const float *w_scales, void *y,
                      qlin_out_type out_type, const qlin_config *cfg, void *workspace,
                      size_t ws_bytes, void *stream);

/* The whole layer: quantize x (as qlin_quantize_act; xq and x_scales are
 * written) and compute y (as qlin_gemm).  With act_path QLIN_ACT_FUSED in
 * cfg (or in the table's choice when cfg is NULL) this is one kernel
 * launch, else two.
 * Arguments, layouts and errors are those of the two calls; x must not
 * alias xq, x_scales or y. */
qlin_status qlin_linear(qlin_format fmt, int M, int N, int K, const void *x, int64_t ldx, void *xq,
                        float *x_scales, const void *wq, const float *w_scales, void *y,
                        qlin_out_type out_type, const qlin_config *cfg, void *workspace,
                        size_t ws_bytes, void *stream);

/* Bytes of the static split-K workspace that qlin_linear_scratch uses on
 * each GPU. */
#define QLIN_SCRATCH_BYTES (8u << 20)

/* qlin_linear for callers that cannot allocate device memory: code under
 * hipGraph capture, tight serving loops, harnesses that forbid allocation.
 * Arguments, layouts, results and errors are qlin_linear's, minus the
 * workspace: a schedule that splits K keeps its partial sums and arrival
 * counters in a static array of QLIN_SCRATCH_BYTES that the library holds
 * on each GPU until the process ends.  Nothing is allocated or freed.
 *   - a schedule whose workspace (qlin_workspace_bytes) exceeds
 *     QLIN_SCRATCH_BYTES is rejected with QLIN_ERR_WORKSPACE before any
 *     HIP call (every M <= 32 entry of the shipped table fits);
 *   - the array must hold zeros between calls, and every call leaves it so;
 *     the first call on a GPU that needs it enqueues one fill kernel on
 *     `stream` that zeroes it (a call made while `stream` is captured puts
 *     the fill into the graph, and the next call outside capture fills it
 *     once more);
 *   - every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (other streams, other threads, or a graph replay
 *     beside an eager call) race on it and their results are undefined. */
qlin_status qlin_linear_scratch(qlin_format fmt, int M, int N, int K, const void *x, int64_t ldx,
                                void *xq, float *x_scales, const void *wq, const float *w_scales,
                                void *y, qlin_out_type out_type, const qlin_config *cfg,
                                void *stream);

/* Schedule lookup (host only, no device work).  M rounds up to the next
 * tuned token bucket {1,2,4,8,16,24,32} (section "Per-shape Config Tuning"),
 * or {64,128,256,512} above 32.  In strict mode a missing entry is
 * QLIN_ERR_NO_CONFIG (the opt-in rule that start-up fails without tuned
 * configurations); in permissive mode a built-in rule answers. */
qlin_status qlin_select_variant(qlin_format fmt, int M, int N, int K, qlin_config *out);

/* Workspace bytes qlin_gemm needs for this schedule (0 when split_k is 1).
 * cfg NULL: for the schedule qlin_select_variant picks. */
qlin_status qlin_workspace_bytes(qlin_format fmt, int M, int N, int K, const qlin_config *cfg,
                                 size_t *bytes);

/* Checks a schedule against (fmt, M, N, K) without launching anything. */
qlin_status qlin_validate_config(qlin_format fmt, int M, int N, int K, const qlin_config *cfg);

/* Grouped (mixture-of-experts) GEMM: `groups` independent products of the
 * same shape in one launch, group e computing y_e = dequant(xq_e . wq_e^T).
 * The pages name MoE layers as the next target, and each group's product is
 * the one they define ("Building a High-Performance and Portable vLLM
 * Linear Backend with Helion", sections "Future work", model-coverage
 * paragraph, and "Kernel Implementation").
 *   group_offsets  device int32 [groups + 1], non-decreasing, from 0 to
 *                  total_rows: group e owns rows [off[e], off[e+1]) of xq,
 *                  x_scales and y.  Read by the kernel, so a captured graph
 *                  can be replayed after the routing changes.  A group
 *                  with no rows reads none of its weights.  (The kernel
 *                  clamps the offsets into [0, total_rows] and takes
 *                  running maxima, so whatever the array holds, groups
 *                  never overlap and nothing outside y is written; rows in
 *                  no group are left as they were.)
 *   total_rows     rows of xq / x_scales / y (0: nothing is enqueued)
 *   max_group_rows the expected largest group: token tiles hold
 *                  min(tile_m, max_group_rows) rows.  Larger groups are
 *                  still computed whole, in more tiles.  In decode with
 *                  top-k routing, the token count bounds every group.
 *   xq, x_scales   [total_rows, K] codes and their scales (qlin_quantize_act
 *                  layouts), rows grouped by group
 *   wq, w_scales   [groups][N][K] codes (or [groups] packed matrices with
 *                  QLIN_PACKED_WEIGHTS) and [groups][N] (or
 *                  [groups][N/128][K/128] for QLIN_BLOCK_FP8) scales
 *   y              [total_rows, N]
 *   cfg            NULL: qlin_grouped_select_variant's rule; otherwise
 *                  forced (tile_m 16 or 32, act_path QLIN_ACT_STAGED or
 *                  QLIN_ACT_DIRECT)
 *   workspace      as qlin_gemm, qlin_grouped_workspace_bytes(...) bytes
 * The grid covers ceil(total_rows / tile rows) + min(groups, total_rows)
 * token tiles, a bound on the tiles of any routing; workgroups past the
 * routing's own tiles exit without reading anything.
 * Errors as qlin_gemm, plus QLIN_ERR_SHAPE for groups < 1, total_rows < 0,
 * max_group_rows < 1 or a grid of more than 65535 token tiles. */
qlin_status qlin_grouped_gemm(qlin_format fmt, int groups, int N, int K, const int *group_offsets,
                              int total_rows, int max_group_rows, const void *xq,
                              const float *x_scales, const void *wq, const float *w_scales, void *y,
                              qlin_out_type out_type, const qlin_config *cfg, void *workspace,
                              size_t ws_bytes, void *stream);

/* The grouped launches' built-in schedule (no table: the groups already
 * fill the GPU): Swap-AB, 16- or 32-token tiles, 64 channels by 4 waves
 * (32 channels by 4 K waves when max_group_rows <= 2 and K >= 2048), no
 * split. */
qlin_status qlin_grouped_select_variant(qlin_format fmt, int groups, int N, int K, int max_group_rows,
                                        qlin_config *out);

/* Workspace bytes qlin_grouped_gemm needs (0 without split-K). */
qlin_status qlin_grouped_workspace_bytes(qlin_format fmt, int groups, int N, int K, int total_rows,
                                         int max_group_rows, const qlin_config *cfg, size_t *bytes);

/* Selection table.  qlin_load_table parses a text table (replacing any loaded
 * one; path NULL = the table installed next to the library); the table is
 * immutable afterwards, so lookups are thread-safe.  qlin_set_strict(1)
 * makes a missing entry an error (the default is 0, permissive). */
qlin_status qlin_load_table(const char *path);
qlin_status qlin_set_strict(int strict);
int qlin_table_entries(void);

/* hipGraph capture of a decode step (section "Hybrid Dispatch": the tuned
 * path runs only under graph replay).  qlin_graph_begin starts capturing
 * `stream` (not the NULL stream); every qlin call on it until
 * qlin_graph_end is recorded instead of run; qlin_graph_end instantiates
 * the graph into *graph.  qlin_graph_launch replays it on a stream. */
typedef struct qlin_graph_s *qlin_graph;
qlin_status qlin_graph_begin(void *stream);
qlin_status qlin_graph_end(void *stream, qlin_graph *graph);
qlin_status qlin_graph_launch(qlin_graph graph, void *stream);
qlin_status qlin_graph_destroy(qlin_graph graph);

/* Helpers. */
const char *qlin_status_str(qlin_status st);
int qlin_abi_version(void);
/* Last HIP error code seen by a call that returned QLIN_ERR_HIP (0 if none). */
int qlin_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif
