// qlin_internal.h -- declarations shared by the library's host and device
// sources (not part of the public ABI).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "../../include/qlin.h"

namespace qlin {

constexpr int kGroup = 128;          // K block: one fp8 MFMA, one 1x128 scale group
// packed weights (QLIN_PACKED_WEIGHTS): 16-row x 128-K blocks of 2 KiB
constexpr int kPackRows = 16;
constexpr int kPackBlock = kPackRows * kGroup;
// bytes of one [N, K] weight matrix in the packed layout (N % 16 == 0)
inline int64_t packed_weight_bytes(int N, int K) {
    return (int64_t)(N / kPackRows) * ((K + kGroup - 1) / kGroup) * kPackBlock;
}
constexpr int kMaxWaves = 8;         // waves per workgroup
constexpr int kLdsBudget = 78 * 1024; // bytes of LDS a GEMM workgroup may use (two fit a CU)
// ... and when the launch has no more workgroups than the GPU has compute
// units (each gets a CU of its own, with 160 KiB of LDS)
constexpr int kLdsBudgetOnePerCU = 150 * 1024;
constexpr int kComputeUnits = 256;
constexpr int kMaxSplit = 64;
// size of the static split-K workspace of qlin_linear_scratch (per GPU)
constexpr size_t kScratchBytes = QLIN_SCRATCH_BYTES;

// Everything a GEMM launch needs, resolved on the host.
struct GemmLaunch {
    const uint8_t *xq;   // activation codes and scales (unfused path)
    const float *xs;
    const uint16_t *x;   // fused path: bf16 activations [M][ldx] ...
    int64_t ldx;
    uint8_t *xq_out;     // ... and where the codes and scales it makes go
    float *xs_out;
    const uint8_t *wq;   // weight codes: [N][K] row-major, or packed (w_packed)
    const float *wsc;
    void *y;
    void *acc_ws;        // split-K: packed int64 sums [M][N] (zero between calls), or
                         // per-partition slices [nsplit][M][N] of int32 / fp32
    uint32_t *counters;  // split-K arrival counters, one per output tile, zero between calls
    int M, N, K;
    int nkb;             // K blocks of 128 (last one may be partial)
    int kb_per_split;    // K blocks per split-K partition
    int nsplit;          // effective number of partitions (grid z)
    int phase_blocks;    // K blocks of activations staged in LDS at once
    int out_type;
    int packed;          // split-K through packed 64-bit integer atomics (exact formats)
    int n_tiles, m_tiles;
    int nw, kw;          // waves along N and along K
    int64_t slice;       // split-K slice stride in elements (M x N; total rows x N when grouped)
    // grouped launches (mixture of experts): group e's rows are
    // [group_off[e], group_off[e + 1]) of the call's M rows, its weights and
    // scales the e-th of the call's; grid y covers the (group, token tile)
    // pairs of the groups that have rows, in group order (workgroups past
    // the last pair exit at once)
    int sub_rows;        // weight rows per 16-row sub-tile that are real (16, or 8)
    int w_packed;        // weight codes in the packed layout (2 KiB blocks)
    int64_t w_group_stride;   // bytes between the groups' weight matrices
    const int *group_off;
    int groups;
    int group_rows;      // rows per token tile of a grouped launch (<= tile_m)
};

// Derived launch geometry for (fmt, M, N, K, cfg).
struct Plan {
    int tile_m, tile_n, nr, nw, kw, waves;
    int sub_rows;         // weight rows per sub-tile: 16, or 8 (tile_n = 8 x nw)
    int nkb, kb_per_split, nsplit, phase_blocks;
    int n_tiles, m_tiles;
    size_t lds_bytes;
    int packed;           // split-K reduction through packed 64-bit atomics
    int fuse;             // activation quantization inside the GEMM kernel
    int xc;               // ... with this many 8-value chunks per lane in registers
                          // (-1: direct activation fragments, no LDS staging)
    size_t ws_bytes;          // workspace bytes (0 without split)
    size_t ws_counter_bytes;  // of which arrival counters (the rest: sums)
};

// Fills *plan; returns QLIN_OK or the reason the schedule is invalid.
// `fused`: planned for qlin_linear (cfg.act_path applies) or qlin_gemm.
// `grouped`: for a grouped launch, whose grid is not the plan's own (its
// workgroups keep the smaller LDS budget).
qlin_status make_plan(qlin_format fmt, int M, int N, int K, const qlin_config &cfg, bool fused,
                      Plan *plan, bool grouped = false);

// Host-side selection table (qlin_table.cpp).
qlin_status table_lookup(qlin_format fmt, int M, int N, int K, qlin_config *out, bool *found);
qlin_status table_nearest(qlin_format fmt, int M, int N, int K, qlin_config *out, bool *found);
void default_config(qlin_format fmt, int M, int N, int K, qlin_config *out);
int token_bucket(int M);
bool strict_mode();

// Kernel launchers (qlin_kernels.hip); they only enqueue.
// threads: per token row (per-token formats: 64, 128, 256 or 512) or per
// workgroup (1x128 groups: 64 or 256); 0 = quant_threads_rule
hipError_t launch_quant_act(int fmt, int M, int K, const void *x, int64_t ldx, void *xq,
                            float *xs, hipStream_t s, int threads = 0);
int quant_threads_rule(int fmt, int M, int K);
bool quant_threads_valid(int fmt, int threads);
hipError_t launch_quant_weight(int fmt, int N, int K, const float *w, void *wq, float *ws,
                               hipStream_t s);
// [batch][N][K] row-major codes -> [batch][packed_weight_bytes(N, K)]
hipError_t launch_pack_weight(int batch, int N, int K, const void *wq, void *out, hipStream_t s);
// xc: register chunks per lane of the in-kernel quantization (0: codes
// staged in LDS; -1: direct, each wave loads its own activation fragments)
hipError_t launch_gemm(int fmt, bool swap, int tile_m, int nr, int xc, const GemmLaunch &g,
                       size_t lds_bytes, hipStream_t s);
bool gemm_variant_exists(int fmt, bool swap, int tile_m, int nr, int xc);
// this device's static scratch array (kScratchBytes, zero between calls);
// see qlin_linear_scratch
hipError_t static_scratch(hipStream_t s, void **out);

}  // namespace qlin
