// qlin_gemm.h -- the skinny quantized GEMM kernel for gfx950 (CDNA4), with
// its Standard / Split-K / Swap-AB schedules and the optional in-kernel
// activation quantization.  Included by one source file per format, each of
// which instantiates the variants it dispatches to.
//
// Product: "Building a High-Performance and Portable vLLM Linear Backend
// with Helion", section "Scope" (FP8_Dynamic, W8A8_INT8, Block_FP8 scale
// granularities) and section "Kernel Implementation" (one contraction with
// a float32 accumulator, split_k / swap_ab as schedule choices, Split-K
// partials added into a zeroed output).
//
// Data layout (all row-major): activations x bf16 [M][ldx], codes xq [M][K],
// weights wq [N][K] (K contiguous, as a torch Linear weight), output y [M][N].
#pragma once

#include "qlin_device.h"

namespace qlin {

// ---------------------------------------------------------------------------
//
// Work decomposition.  A workgroup owns a tile of up to TM = 16*MT tokens by
// TN = SR*NR*nw output channels and a range of 128-wide K blocks (all of K,
// or one Split-K partition).  Its waves form an nw x kw grid: a wave owns NR
// sub-tiles of SR channels and every kw-th K block of the range, so the kw
// waves of a column stream neighbouring K blocks of the same weight rows at
// the same time; their partial sums are added through LDS at the end.  A
// sub-tile is the matrix core's 16 rows (SR = 16), or 8 of them (SR = 8: the
// other 8 read zeros and are never stored), which halves the weight bytes
// per workgroup and doubles the workgroups a narrow layer spreads over.
//
// Operand fragments.  For one 128-wide K block a lane l (row r = l % 16,
// quarter q = l / 16) holds 32 consecutive bytes k = 32q .. 32q+31 of its
// row, for the weight row (channel n0 + r) and for the activation row
// (token m0 + r).  Both matrix-core operands use the same lane -> (row, k)
// assignment, so whatever order the hardware sums the k slots in, every
// weight byte meets the activation byte of the same k.  fp8 uses one
// 16x16x128 MFMA per block (32 bytes per lane); int8 uses two 16x16x64 MFMAs
// (bytes 0..15, then 16..31 of each lane's 32).
//
// Weight stream.  Each weight lane load covers 32 contiguous bytes; the 4
// lanes of a row cover the row's whole 128-byte block, so a wave-wide load
// reads 16 full 128-byte lines.  A wave keeps PF blocks of loads in flight
// in PF register slots, consumed and refilled in batches.
//
// Activations.  The workgroup's token rows for its K range are staged once
// in LDS, only the rows that exist (R = min(TM, M - m0)), row by row: row r
// of the phase's K range starts at 16-byte slot r * RS, RS = 8 P + 1 for at
// most P K blocks per phase.  The odd row stride puts the 16 rows that the
// 16 lanes of a quarter read at 16 different bank groups, so the two
// ds_read_b128 per block are free of bank conflicts, and a row's K range is
// contiguous, as in memory.  Lanes
// whose row is past R use zeros.  When R x RS slots do not fit the LDS
// budget the range is processed in phases.
//
// Order of the memory requests.  The vector memory counter a wave waits on
// counts requests in issue order, so a wait for one load is a wait for every
// older one.  Each phase therefore first requests its activations (codes,
// or bf16 values to quantize), then the epilogue's scales, then the first PF
// weight blocks; the activations arrive first (they are few and
// L2-resident) and are staged in LDS while the weights are still in flight.
// Codes are copied by the memory system itself into LDS (loads with the LDS
// bit, no registers); bf16 values come through registers and are quantized
// on the way.  Every weight slot is requested on every path (a slot past
// the wave's last block uses an out-of-range offset, which returns zeros
// without touching memory), so the waits count exactly.
//
// Standard: A = activations (tokens are the MFMA rows), B = weights.  The
// 16x16 result lane l holds column l % 16 = channel and rows 4(l/16)+i =
// tokens.  Swap-AB: A = weights, B = activations, so the result is the
// transpose: lane l holds token l % 16 and channels 4(l/16)+i, which makes
// the output stores 4 channels wide and needs one activation scale per lane.
//
// In-kernel quantization (XC > 0, per-token formats and the block format):
// each wave owns whole token rows (rows w, w + waves, ...) and holds up to
// XC 8-value chunks of them per lane in registers, so the activations are
// read once: per-token formats take the row's amax over all of K by a wave
// reduction (the rows are small and shared by every workgroup, so they come
// from L2), the block format the 1x128 group amax over the 16 lanes that
// hold a group.  The codes of the workgroup's K range are written to the
// LDS staging layout directly.

template <int FMT>
struct AccT;
template <>
struct AccT<FMT_I8> {
    typedef v4i type;
    typedef int scalar;
};
template <>
struct AccT<FMT_FP8> {
    typedef v4f type;
    typedef float scalar;
};
template <>
struct AccT<FMT_BLOCK> {
    typedef v4f type;
    typedef float scalar;
};

__device__ __forceinline__ v8i join(uint4 lo, uint4 hi) {
    v8i r;
    r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
    return r;
}
__device__ __forceinline__ v4i lo4(v8i v) { return v4i{v[0], v[1], v[2], v[3]}; }
__device__ __forceinline__ v4i hi4(v8i v) { return v4i{v[4], v[5], v[6], v[7]}; }

// acc (+)= A . B for one 128-wide K block
template <int FMT>
__device__ __forceinline__ typename AccT<FMT>::type block_mma(v8i a, v8i b,
                                                              typename AccT<FMT>::type c) {
    if constexpr (FMT == FMT_I8) {
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(lo4(a), lo4(b), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(hi4(a), hi4(b), c, 0, 0, 0);
        return c;
    } else {
        // operand formats 0/0 = fp8 E4M3 for A and B; zero scale operands
        // select the unscaled instruction
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
    }
}

__device__ __forceinline__ uint4 select4(bool keep, uint4 v) {
    return keep ? v : make_uint4(0, 0, 0, 0);
}

// Buffer resources: base address and size in bytes; the hardware checks
// every access against the size, and an offset at or past it returns zeros
// and makes no memory access.
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kBufferFormat = 0x00020000;   // descriptor word 3 for gfx9-family targets

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kBufferFormat);
}

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    const v4i v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// Cache policy of the weight stream when every weight tile is read by one
// token tile only (a launch with one tile of tokens, or a grouped launch):
// non-temporal (the buffer instructions' nt bit).  The weights then pass
// through once, while the activation codes are read by every workgroup of
// an XCD; marked non-temporal, the weights no longer push the codes out of
// the caches.  Measured on the three workload steps: 8 % faster (BlockFP8),
// 5 % (W8A8INT8 and FP8Dynamic GEMM launches); the sc0 bit alone changed
// nothing.  With more token tiles the later tiles re-read each weight tile
// from the caches, and non-temporal weights made those launches 4-6 % slower
// (crossover sweep, 256 and 512 tokens), so they keep the default policy.
constexpr int kStreamCpol = 2;

// 32 bytes of the lane's weight row in K block kb: bytes 32 quarter ..
// 32 quarter + 31 of the block, as two 16-byte halves.  Row-major codes:
// lane_off = row * K + 32 * quarter in a resource that covers the sub-tile's
// rows, halves 16 bytes apart, blocks 128 bytes apart; a half at or past K
// (in a partial last block) is read out of range.  Packed codes: lane_off =
// 16 (16 quarter + row) in a resource that covers the sub-tile's 16-row
// group, halves 1 KiB apart, blocks 2 KiB apart, the tail of K already
// zero.  The block's offset is a scalar operand, so a slot costs no address
// registers; a dead slot uses an out-of-range lane offset, so every lane
// issues the same two loads per block and nothing has to be masked after
// the data arrives.  CPOL: the loads' cache policy (kStreamCpol for
// weights, 0 for activation fragments, which other waves read too).
template <int CPOL>
__device__ __forceinline__ v8i load_w(__amdgpu_buffer_rsrc_t rs, uint32_t lane_off, int kb, int k,
                                      int K, bool live, bool packed) {
    const int boff = __builtin_amdgcn_readfirstlane(kb * (packed ? kPackBlock : kGroup));
    const int hoff = packed ? kPackBlock / 2 : 16;
    const uint32_t lo_off = live && (packed || k < K) ? lane_off : kOutOfRange;
    const uint32_t hi_off = live && (packed || k + 16 < K) ? lane_off : kOutOfRange;
    const v4i lo = __builtin_amdgcn_raw_buffer_load_b128(rs, lo_off, boff, CPOL);
    const v4i hi = __builtin_amdgcn_raw_buffer_load_b128(rs, hi_off, boff + hoff, CPOL);
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Orders this thread's earlier global atomics before what follows: wait for
// every outstanding memory operation to be acknowledged.  (Device-scope
// atomics are coherent across the chip's L2 slices; what the arrival counter
// needs is only that a partition's additions are performed before its
// arrival is counted.  A device-scope release fence would also write back
// the whole L2, which costs far more than the kernel.)
__device__ __forceinline__ void wait_memory_idle() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// byte offset in the LDS staging layout (row stride RS 16-byte slots) of
// 8-byte chunk cl (0, 1, ... along the K range) of row `row`
__device__ __forceinline__ int stage_offset8(int cl, int row, int RS) { return row * RS * 16 + cl * 8; }

// The last partition of a split-K tile adds the nsplit slices of its
// rows x cols outputs at (m0, n0) (slice z at part + z * slice, row stride
// N; cols a multiple of 4) in partition order, hands every group of 4
// consecutive outputs to emit(m, n, v[4]), and leaves the slices zero.  The
// slices were written by other workgroups, possibly on other XCDs, with
// device-coherent stores, so they are read with device-coherent loads
// (8 bytes each); a batch of 4 groups x 4 partitions is requested before
// any of it is used, so the reduction takes one memory round trip per
// batch rather than one per output.
template <typename acc_s, typename Emit>
__device__ __forceinline__ void reduce_slices(acc_s *part, int64_t slice, int N, int m0, int n0, int rows,
                                              int cols, int nsplit, int tid, int nthreads, Emit emit) {
    constexpr int GB = 4;   // groups of 4 outputs per thread and batch
    constexpr int ZB = 4;   // partitions per batch
    typedef unsigned long long u64;
    const int cols4 = cols >> 2;
    const int groups = rows * cols4;
    for (int g0 = tid; g0 < groups; g0 += nthreads * GB) {
        int64_t idx[GB];
        bool ok[GB];
#pragma unroll
        for (int b = 0; b < GB; ++b) {
            const int gi = g0 + b * nthreads;
            ok[b] = gi < groups;
            const int r = ok[b] ? gi / cols4 : 0, c = ok[b] ? gi - r * cols4 : 0;
            idx[b] = (int64_t)(m0 + r) * N + n0 + 4 * c;
        }
        acc_s v[GB][4];
#pragma unroll
        for (int b = 0; b < GB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) v[b][i] = 0;
        for (int z0 = 0; z0 < nsplit; z0 += ZB) {
            u64 w[ZB][GB][2];
#pragma unroll
            for (int zz = 0; zz < ZB; ++zz)
#pragma unroll
                for (int b = 0; b < GB; ++b) {
                    const bool live = ok[b] && z0 + zz < nsplit;
                    const u64 *p = reinterpret_cast<const u64 *>(part + (int64_t)(z0 + zz) * slice + idx[b]);
                    w[zz][b][0] = live ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
                    w[zz][b][1] = live ? __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
                }
#pragma unroll
            for (int zz = 0; zz < ZB; ++zz) {
                if (z0 + zz >= nsplit) break;
#pragma unroll
                for (int b = 0; b < GB; ++b)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const uint32_t lo = (uint32_t)w[zz][b][h], hi = (uint32_t)(w[zz][b][h] >> 32);
                        acc_s a0, a1;
                        __builtin_memcpy(&a0, &lo, 4);
                        __builtin_memcpy(&a1, &hi, 4);
                        v[b][2 * h] += a0;
                        v[b][2 * h + 1] += a1;
                    }
            }
        }
#pragma unroll
        for (int b = 0; b < GB; ++b) {
            if (!ok[b]) continue;
            const int gi = g0 + b * nthreads, r = gi / cols4, c = gi - r * cols4;
            emit(m0 + r, n0 + 4 * c, v[b]);
            for (int z = 0; z < nsplit; ++z) {   // leave the workspace zero
                u64 *p = reinterpret_cast<u64 *>(part + (int64_t)z * slice + idx[b]);
                __hip_atomic_store(p, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(p + 1, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

// Inclusive prefix sum / maximum over the wave's 64 lanes through DPP (no
// LDS traffic): shifts by 1, 2, 4 and 8 lanes within each row of 16 (lanes
// with no source combine with 0), then row_bcast:15 combines row r's last
// value into row r + 1 (rows 1 and 3) and row_bcast:31 lane 31's into rows 2
// and 3.  (The maximum is meant for non-negative values.)
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int add_dpp(int v) {
    return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int max_dpp_i(int v) {
    return max(v, __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false));
}
__device__ __forceinline__ int wave_inclusive_sum(int v) {
    v = add_dpp<0x111>(v);
    v = add_dpp<0x112>(v);
    v = add_dpp<0x114>(v);
    v = add_dpp<0x118>(v);
    v = add_dpp<0x142, 0xA>(v);
    return add_dpp<0x143, 0xC>(v);
}
__device__ __forceinline__ int wave_inclusive_max(int v) {
    v = max_dpp_i<0x111>(v);
    v = max_dpp_i<0x112>(v);
    v = max_dpp_i<0x114>(v);
    v = max_dpp_i<0x118>(v);
    v = max_dpp_i<0x142, 0xA>(v);
    return max_dpp_i<0x143, 0xC>(v);
}

// Grouped launches: finds the j-th (group, token tile) pair in the list of
// such pairs over the groups that have rows, in group order.  Group e holds
// rows [P(e), P(e + 1)) of `total`, where P(x) is the largest of off[0..x]
// clamped into [0, total]: for non-decreasing offsets that is off[e] ..
// off[e + 1], and whatever the offsets, the groups' rows never overlap (so
// two groups never share outputs or split-K sums).  A group has
// ceil(rows / tm) tiles of tm rows.  Each wave scans 64 groups at a time
// (one group per lane: running maxima of the offsets and an inclusive prefix
// sum of the tile counts across the wave); every wave of a workgroup gets the
// same, wave-uniform answer.  Returns false when j is past the end of the list.
__device__ __forceinline__ bool group_tile(const int *off, int groups, int total, int tm, int j, int lane,
                                           int &e_out, int &tile_out, int &lo_out, int &hi_out) {
    int base = 0, carry = 0;   // tiles and P(c) of the groups before this chunk
    for (int c = 0; c < groups; c += 64) {
        const int e = c + lane;
        int a = 0, b = 0;
        if (e < groups) {
            a = min(max(off[e], 0), total);
            b = min(max(off[e + 1], 0), total);
        }
        const int lo = max(carry, wave_inclusive_max(a));    // P(e)
        const int hi = max(lo, wave_inclusive_max(b));       // P(e + 1)
        const int tiles = e < groups ? (hi - lo + tm - 1) / tm : 0;
        const int incl = wave_inclusive_sum(tiles);
        const int sum = __builtin_amdgcn_readlane(incl, 63);
        if (j < base + sum) {
            const int l = __builtin_amdgcn_readfirstlane(__builtin_ctzll(__ballot(base + incl > j)));
            e_out = c + l;
            tile_out = j - base - (__builtin_amdgcn_readlane(incl, l) - __builtin_amdgcn_readlane(tiles, l));
            lo_out = __builtin_amdgcn_readlane(lo, l);
            hi_out = __builtin_amdgcn_readlane(hi, l);
            return true;
        }
        base += sum;
        carry = __builtin_amdgcn_readlane(hi, 63);
    }
    return false;
}

// s_waitcnt operand that waits until at most n vector memory requests are
// outstanding and leaves the other counters alone (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// NT: weight loads with the non-temporal cache policy (kStreamCpol)
template <int FMT, bool SWAP, int MT, int NR, int PF, int XC, bool NT>
__global__ __launch_bounds__(64 * kMaxWaves) void gemm_kernel(GemmLaunch g) {
    typedef typename AccT<FMT>::type acc_t;
    typedef typename AccT<FMT>::scalar acc_s;
    constexpr bool FUSE = XC > 0;
    // direct activations: codes quantized beforehand, each wave loads its
    // own fragments with the weight slot they multiply (no LDS staging)
    constexpr bool DIRECT = XC < 0;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ int s_last;
    __shared__ float s_rowscale[16 * MT];
    __shared__ float s_rowrecip[16 * MT];
    __shared__ float s_seg[FUSE ? XC * kMaxWaves : 1];   // per-token amax of 64-chunk segments

    const int lane = threadIdx.x & 63;
    // wave-level values are made explicitly uniform (scalar registers), so
    // the block loop below branches on scalars
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nthreads = blockDim.x;
    const int nwaves = nthreads >> 6;
    const int nw = wave % g.nw, kw = wave / g.nw;
    // weight rows per sub-tile: 16, or 8 (then the other 8 rows of the
    // matrix core's 16 read zeros, and their outputs are never stored)
    const int SR = g.sub_rows;
    const int TN = SR * NR * g.nw;
    const int n_tile0 = blockIdx.x * TN;
    // grouped launch: blockIdx.y is the index of a (group, token tile) pair
    // in the list of such pairs over the groups that have rows; the group's
    // rows, weights, scales, output rows and split-K sums take the place of
    // the call's (workgroups past the end of the list read nothing)
    int mtile = blockIdx.y, tile_rows = 16 * MT;
    // (grouped launches take quantized codes: the fused variants leave this out)
    if (!FUSE && g.group_off) {
        int e, lo, hi;
        tile_rows = g.group_rows;   // <= 16 * MT: the rows the LDS staging was sized for
        if (!group_tile(g.group_off, g.groups, g.M, tile_rows, (int)blockIdx.y, lane, e, mtile, lo, hi)) return;
        const int Gk = (g.K + kGroup - 1) / kGroup;
        g.xq += (int64_t)lo * g.K;
        g.xs += (int64_t)lo * (FMT == FMT_BLOCK ? Gk : 1);
        g.y = static_cast<uint8_t *>(g.y) + (int64_t)lo * g.N * (g.out_type == QLIN_OUT_BF16 ? 2 : 4);
        g.wq += (int64_t)e * g.w_group_stride;
        g.wsc += (int64_t)e * (FMT == FMT_BLOCK ? (int64_t)(g.N / kGroup) * Gk : g.N);
        if (g.acc_ws) g.acc_ws = static_cast<uint8_t *>(g.acc_ws) + (int64_t)lo * g.N * (g.packed ? 8 : 4);
        g.M = hi - lo;
    }
    const int m0 = mtile * tile_rows;
    const int kb_begin = blockIdx.z * g.kb_per_split;
    const int kb_end = min(g.nkb, kb_begin + g.kb_per_split);
    const int R = min(tile_rows, g.M - m0);   // token rows that exist in this tile
    // every row guard below is against the tile's own end (in a grouped
    // launch the next rows may belong to the next tile)
    const int M = m0 + R, N = g.N, K = g.K;
    const int r16 = lane & 15, quarter = lane >> 4;
    // whether this lane's output channels are real rows of its sub-tiles
    const bool col_ok = SWAP ? 4 * quarter < SR : r16 < SR;
    const int G = (K + kGroup - 1) / kGroup;
    const int RS = 8 * g.phase_blocks + 1;   // LDS staging row stride in 16-byte slots (odd)
    // fused path: the first column of workgroups also stores the codes and
    // scales it produces (every workgroup of a row of tiles produces the same)
    const bool writer = FUSE && blockIdx.x == 0;

    int nsub[NR];
    __amdgpu_buffer_rsrc_t wrs[NR];
    const bool wpk = g.w_packed != 0;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        nsub[r] = n_tile0 + (nw * NR + r) * SR;
        // sub-tiles past N get an empty resource: their loads return zeros
        const int base = min(nsub[r], N - SR);
        if (wpk) {
            // packed: the 16-row group's 2 KiB blocks; an 8-row sub-tile that
            // is the group's second half starts 128 bytes into each 1 KiB
            // half-block (its rows are lanes 8 .. 15 of every quarter)
            const int half = (base >> 3) & 1;
            wrs[r] = buffer_rsrc(g.wq + (int64_t)(base >> 4) * g.nkb * kPackBlock + half * 128,
                                 nsub[r] < N ? (uint32_t)(g.nkb * kPackBlock - half * 128) : 0u);
        } else {
            // row-major: rows SR .. 15 of the sub-tile lie past the resource's end
            wrs[r] = buffer_rsrc(g.wq + (int64_t)base * K, nsub[r] < N ? (uint32_t)SR * K : 0u);
        }
    }
    // packed: lanes of rows SR .. 15 read out of range (zeros)
    const uint32_t lane_off = wpk ? (r16 < SR ? (uint32_t)(quarter * 256 + r16 * 16) : kOutOfRange)
                                  : (uint32_t)(r16 * K + quarter * 32);
    // the lane's activation fragment in a staged block: [half 0][quarter][row]
    // (rows past R read an existing row, and their data is replaced by zeros)
    int lds_lo[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) lds_lo[mt] = ((mt * 16 + r16 < R ? mt * 16 + r16 : 0) * RS + 2 * quarter) * 16;
    // direct activations: lane (r16, quarter) of fragment mt holds 32 bytes of
    // the tile's token row 16 mt + r16 (codes row-major [M][K]; rows past R
    // read out of range, i.e. zeros), and for the block format that row's
    // scale of the block
    const __amdgpu_buffer_rsrc_t ars = buffer_rsrc(g.xq + (int64_t)m0 * K, DIRECT ? (uint32_t)(R * K) : 0u);
    const __amdgpu_buffer_rsrc_t asr =
        buffer_rsrc(g.xs + (int64_t)m0 * G, DIRECT && FMT == FMT_BLOCK ? (uint32_t)(R * G * 4) : 0u);
    uint32_t a_off[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) a_off[mt] = (uint32_t)((mt * 16 + r16) * K + quarter * 32);

    acc_t acc[NR][MT];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[r][mt] = acc_t{0, 0, 0, 0};

    // Per-channel formats: the epilogue's channel (and, unfused, token)
    // scales, requested after the first weight blocks so that their latency
    // hides behind the weight stream.  Swap-AB lanes need one token scale and
    // 4 channel scales per sub-tile, Standard lanes 4 token scales and one
    // channel scale.
    float pre_sa[MT][SWAP ? 1 : 4], pre_sw[NR][SWAP ? 4 : 1];
    auto token_of = [&](int mt, int i) { return SWAP ? m0 + mt * 16 + r16 : m0 + mt * 16 + 4 * quarter + i; };
    // (buffer loads: 32-bit offsets, and positions past N or M read zeros)
    auto prefetch_scales = [&]() {
        if constexpr (FMT != FMT_BLOCK) {
            const __amdgpu_buffer_rsrc_t wsr = buffer_rsrc(g.wsc, (uint32_t)N * 4);
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int i = 0; i < (SWAP ? 4 : 1); ++i) {
                    const int n = SWAP ? nsub[r] + 4 * quarter + i : nsub[r] + r16;
                    pre_sw[r][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(wsr, n * 4, 0, 0));
                }
            if constexpr (!FUSE) {
                const __amdgpu_buffer_rsrc_t xsr = buffer_rsrc(g.xs + m0, (uint32_t)R * 4);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < (SWAP ? 1 : 4); ++i)
                        pre_sa[mt][i] = __uint_as_float(
                            __builtin_amdgcn_raw_buffer_load_b32(xsr, (token_of(mt, i) - m0) * 4, 0, 0));
            }
        }
    };

    // request K block kb into a register slot (the block format also fetches
    // each sub-tile's 128x128 weight-block scale); a dead slot (live false)
    // is requested with out-of-range offsets
    // (the block scales come by buffer loads too, so that they count in the
    // same vector memory counter as the weights)
    const __amdgpu_buffer_rsrc_t bsr = buffer_rsrc(g.wsc, FMT == FMT_BLOCK ? (uint32_t)(N / kGroup * G * 4) : 0u);
    v8i wbuf[PF][NR];
    float wsbuf[PF][NR];
    v8i abuf[DIRECT ? PF : 1][MT];      // direct activations: fragments of slot p
    float asbuf[DIRECT ? PF : 1][MT];   // ... and (block format) their token scales
    auto issue = [&](int p, int kb, bool live) {
        const int k = kb * kGroup;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            wbuf[p][r] = load_w<NT ? kStreamCpol : 0>(wrs[r], lane_off, kb, k + quarter * 32, K, live, wpk);
            if constexpr (FMT == FMT_BLOCK) {
                const int soff = __builtin_amdgcn_readfirstlane(
                    ((min(nsub[r], N - 1) / kGroup) * G + min(kb, G - 1)) * 4);
                wsbuf[p][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bsr, 0, soff, 0));
            }
        }
        if constexpr (DIRECT) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                abuf[p][mt] = load_w<0>(ars, a_off[mt], kb, k + quarter * 32, K, live, false);
                if constexpr (FMT == FMT_BLOCK)
                    asbuf[p][mt] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                        asr, live ? (uint32_t)(((mt * 16 + r16) * G + kb) * 4) : kOutOfRange, 0, 0));
            }
        }
    };

    const int kstep = g.kw;

    for (int pb0 = kb_begin; pb0 < kb_end; pb0 += g.phase_blocks) {
        const int nblk = min(kb_end - pb0, g.phase_blocks);
        // this wave's blocks of the phase are kw, kw + kstep, ... (a uniform count)
        const int nmine = kw < nblk ? (nblk - kw + kstep - 1) / kstep : 0;
        float *s_scale = reinterpret_cast<float *>(smem + (size_t)R * RS * 16);

        // ---- 1. activation requests
        // fused: the tile's R rows x cn chunk positions of 8 values (per-token
        // formats: all of K, for the amax, padded to a multiple of 64; block
        // format: the K range) in a flat order, chunk slots i of thread t =
        // t + i * nthreads (the fused path has a single phase: its range
        // fits the LDS)
        const int nchunk = K >> 3;
        const int c_lo = FMT == FMT_BLOCK ? kb_begin * 16 : 0;
        const int cn = FMT == FMT_BLOCK ? (kb_end - kb_begin) * 16 : (nchunk + 63) & ~63;
        const int row0 = threadIdx.x / cn, c0 = threadIdx.x - row0 * cn;
        const int t_rows = nthreads / cn, t_chunks = nthreads - t_rows * cn;
        auto next_slot = [&](int &row, int &c) {
            c += t_chunks;
            row += t_rows;
            if (c >= cn) { c -= cn; ++row; }
        };
        uint4 xr[FUSE ? XC : 1];
        if (pb0 != kb_begin) __syncthreads();   // the previous phase's readers are done
        // nothing is in flight here (the previous phase's dead weight slots
        // are done by now; this tells the compiler so)
        __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
        if constexpr (FUSE) {
            const __amdgpu_buffer_rsrc_t xrs =
                buffer_rsrc(g.x + (int64_t)m0 * g.ldx, (uint32_t)(((R - 1) * g.ldx + K) * 2));
            int row = row0, c = c0;
#pragma unroll
            for (int i = 0; i < XC; ++i) {
                const bool ok = row < R && c_lo + c < nchunk;
                xr[i] = load16(xrs, ok ? (uint32_t)((row * g.ldx + (c_lo + c) * 8) * 2) : kOutOfRange);
                next_slot(row, c);
            }
        } else if constexpr (!DIRECT) {
            // the codes go from memory straight into the LDS staging layout:
            // a 16-byte buffer load with the LDS bit writes lane l's data 16 l
            // bytes past the wave's LDS address, so one request copies 64
            // consecutive 16-byte chunks of a row (8 K blocks): the lane
            // offset is 16 l and the row and chunk group are scalars.  The
            // waves take the R x ceil(nblk / 8) requests in turn; lanes past
            // the phase's blocks are masked off, chunks past K are read out of
            // range, which stores zeros.
            const __amdgpu_buffer_rsrc_t qrs = buffer_rsrc(g.xq + (int64_t)m0 * K, (uint32_t)(R * K));
            const int ngrp = (nblk + 7) >> 3;        // 64-chunk groups per row
            const int nreq = R * ngrp;
            const int dr = nwaves / ngrp, di = nwaves - dr * ngrp;
            int r = wave / ngrp, i = wave - r * ngrp;   // this wave's first request
            for (int t = wave; t < nreq; t += nwaves) {
                const int c0 = pb0 * 8 + i * 64;                    // first chunk (absolute)
                const int live = min(64, nblk * 8 - i * 64);        // chunks of the phase
                const int inK = (K >> 4) - c0;                      // chunks before K
                if (lane < live)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        qrs, (__attribute__((address_space(3))) void *)(smem + (r * RS + i * 64) * 16), 16,
                        lane < inK ? (uint32_t)lane * 16 : kOutOfRange,
                        __builtin_amdgcn_readfirstlane(r * K + c0 * 16), 0, 0);
                r += dr;
                i += di;
                if (i >= ngrp) { i -= ngrp; ++r; }
            }
            if constexpr (FMT == FMT_BLOCK) {
                // the activation scales of the phase, [block][row] after the
                // codes, the same way with 4-byte loads (lane l writes 4 l
                // bytes past the wave's address)
                const __amdgpu_buffer_rsrc_t srs = buffer_rsrc(g.xs + (int64_t)m0 * G, (uint32_t)(R * G * 4));
                const int nsc = nblk * R;
                const int sl0 = wave * 64 + lane;
                int sb = sl0 / R, sr = sl0 - sb * R;
                const int dsb = nthreads / R, dsr = nthreads - dsb * R;
                for (int s0 = wave * 64; s0 < nsc; s0 += nthreads) {
                    if (s0 + lane < nsc)
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            srs, (__attribute__((address_space(3))) void *)(s_scale + s0), 4,
                            (uint32_t)((sr * G + pb0 + sb) * 4), 0, 0, 0);
                    sr += dsr;
                    sb += dsb;
                    if (sr >= R) { sr -= R; ++sb; }
                }
            }
        }

        // ---- 2. the epilogue's scales, then the first batch of weight blocks
        // (the weight loads are always the youngest requests in flight; the
        // scheduling barriers keep the compiler from sinking the earlier
        // requests below them)
        prefetch_scales();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < PF; ++p) issue(p, pb0 + kw + p * kstep, p < nmine);
        __builtin_amdgcn_sched_barrier(0);

        // ---- 3. activations into LDS
        if constexpr (FUSE) {
            const int kc0 = kb_begin * 16, kc1 = kb_end * 16;   // chunks staged (absolute)
            auto stage8 = [&](int row, int c, uint2 codes) {   // c absolute
                *reinterpret_cast<uint2 *>(smem + stage_offset8(c - kc0, row, RS)) = codes;
                if (writer && c < nchunk)
                    *reinterpret_cast<uint2 *>(g.xq_out + (int64_t)(m0 + row) * K + c * 8) = codes;
            };
            if constexpr (FMT == FMT_BLOCK) {
                // one 1x128 group = 16 chunks = 16 neighbouring lanes (cn and
                // nthreads are multiples of 16)
                int row = row0, c = c0;
#pragma unroll
                for (int i = 0; i < XC; ++i) {
                    const float amax = row16_max(absmax8(xr[i]));
                    const float sc = amax == 0.0f ? 0.0f : amax / 448.0f;
                    if (row < R) {
                        stage8(row, c_lo + c, quant8<FMT>(xr[i], sc, recip_scale(sc)));
                        if ((c & 15) == 0) {
                            s_scale[(c >> 4) * R + row] = sc;
                            if (writer) g.xs_out[(int64_t)(m0 + row) * G + kb_begin + (c >> 4)] = sc;
                        }
                    }
                    next_slot(row, c);
                }
            } else {
                // per-token amax: cn and nthreads are multiples of 64, so the
                // 64 chunks of one wave and slot lie in one row; their
                // maximum is segment (t + i * nthreads) / 64 of the flat
                // order, and a row's amax is the maximum of its cn / 64
                // segments.  Positions past K hold zeros; those in the last
                // (partial) K block are staged as zero codes.
                const int segs = cn >> 6;
                {
                    int row = row0, c = c0;
#pragma unroll
                    for (int i = 0; i < XC; ++i) {
                        const float a = wave_max(absmax8(xr[i]));
                        if (row < R && lane == 0) s_seg[(row * cn + c) >> 6] = a;
                        next_slot(row, c);
                    }
                }
                __syncthreads();
                // one thread per row: the row's amax, scale and reciprocal
                if ((int)threadIdx.x < R) {
                    const int row = threadIdx.x;
                    float amax = 0.0f;
                    for (int sg = 0; sg < segs; ++sg) amax = fmaxf(amax, s_seg[row * segs + sg]);
                    const float sc = amax == 0.0f ? 0.0f : amax / qmax_of<FMT>();
                    s_rowscale[row] = sc;
                    s_rowrecip[row] = recip_scale(sc);
                    if (writer && blockIdx.z == 0) g.xs_out[m0 + row] = sc;
                }
                __syncthreads();
                int row = row0, c = c0;
#pragma unroll
                for (int i = 0; i < XC; ++i) {
                    if (row < R && c >= kc0 && c < kc1)
                        stage8(row, c, quant8<FMT>(xr[i], s_rowscale[row], s_rowrecip[row]));
                    next_slot(row, c);
                }
            }
        } else if constexpr (!DIRECT) {
            // this thread's staging loads are done once at most the younger
            // requests (the first batch of weight slots: two loads per
            // sub-tile and slot, and the block format's block scale) are
            // outstanding; the barrier below then makes every wave's slots
            // visible
            constexpr int younger = PF * NR * (FMT == FMT_BLOCK ? 3 : 2);
            static_assert(younger < 64, "vmcnt holds at most 63");
            __builtin_amdgcn_s_waitcnt(vmcnt_only(younger));
        }
        if constexpr (!DIRECT) __syncthreads();

        // ---- 4. the weight stream
        // one block: MFMAs of the weights in slot p against this wave's block
        // jb of the phase
        auto compute = [&](int p, int jb) {
            const int b = kw + jb * kstep;
            // activation fragments of this block (zeros past row R; the read
            // address is clamped to an existing row)
            const int boff = b * kGroup;   // uniform
            v8i xf[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if constexpr (DIRECT) {
                    xf[mt] = abuf[p][mt];
                } else {
                    const bool live = mt * 16 + r16 < R;
                    const uint4 lo = *reinterpret_cast<const uint4 *>(smem + lds_lo[mt] + boff);
                    const uint4 hi = *reinterpret_cast<const uint4 *>(smem + lds_lo[mt] + 16 + boff);
                    xf[mt] = join(select4(live, lo), select4(live, hi));
                }
            }
            if constexpr (FMT == FMT_BLOCK) {
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    const float swv = wsbuf[p][r];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const v4f t = SWAP ? block_mma<FMT>(wbuf[p][r], xf[mt], v4f{0, 0, 0, 0})
                                           : block_mma<FMT>(xf[mt], wbuf[p][r], v4f{0, 0, 0, 0});
                        const float *sc = s_scale + b * R;
                        if (SWAP) {
                            const int row = mt * 16 + r16;
                            float sa;
                            if constexpr (DIRECT) sa = asbuf[p][mt];   // 0 past R (read out of range)
                            else sa = row < R ? sc[row] : 0.0f;
                            const float c = sa * swv;
#pragma unroll
                            for (int i = 0; i < 4; ++i) acc[r][mt][i] += t[i] * c;
                        } else {
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int row = mt * 16 + 4 * quarter + i;
                                acc[r][mt][i] += t[i] * ((row < R ? sc[row] : 0.0f) * swv);
                            }
                        }
                    }
                }
            } else {
#pragma unroll
                for (int r = 0; r < NR; ++r)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        acc[r][mt] = SWAP ? block_mma<FMT>(wbuf[p][r], xf[mt], acc[r][mt])
                                          : block_mma<FMT>(xf[mt], wbuf[p][r], acc[r][mt]);
            }
        };

        // Rolling refill: as soon as slot p's block has been multiplied, the
        // slot is requested again for the block PF places later, so PF - 1
        // to PF blocks stay in flight the whole time (consuming a whole batch
        // before requesting the next one would let the stream run dry once
        // per batch).  In the steady-state loop every slot is requested on
        // every pass (past the wave's blocks with out-of-range offsets), so
        // each wait counts exactly PF - 1 younger blocks; the last partial
        // batch is computed after the loop without new requests.  The loop
        // body is unrolled by PF, so the slots live in fixed registers.
        int j = 0;
        for (; j + PF < nmine; j += PF) {
#pragma unroll
            for (int p = 0; p < PF; ++p) {
                compute(p, j + p);
                issue(p, pb0 + kw + (j + PF + p) * kstep, j + PF + p < nmine);
            }
        }
#pragma unroll
        for (int p = 0; p < PF; ++p)
            if (j + p < nmine) compute(p, j + p);
    }

    if constexpr (FUSE && FMT != FMT_BLOCK) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < (SWAP ? 1 : 4); ++i) {
                const int row = token_of(mt, i) - m0;
                pre_sa[mt][i] = row < R ? s_rowscale[row] : 0.0f;
            }
    }

    // add the partial sums of the kw waves of each column through LDS
    if (g.kw > 1) {
        __syncthreads();
        acc_t *red = reinterpret_cast<acc_t *>(smem);
        if (kw > 0) {
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    red[((((kw - 1) * g.nw + nw) * NR + r) * MT + mt) * 64 + lane] = acc[r][mt];
        }
        __syncthreads();
        if (kw == 0) {
            for (int jw = 1; jw < g.kw; ++jw)
#pragma unroll
                for (int r = 0; r < NR; ++r)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        acc[r][mt] += red[((((jw - 1) * g.nw + nw) * NR + r) * MT + mt) * 64 + lane];
        }
    }

    // output value from a total t (scaled sum for the block format, raw sum
    // otherwise) for accumulator element (r, mt, i) of this lane
    auto scaled = [&](float t, int r, int mt, int i) -> float {
        if constexpr (FMT == FMT_BLOCK) return t;
        else return (t * pre_sa[mt][SWAP ? 0 : i]) * pre_sw[r][SWAP ? i : 0];
    };
    auto store1 = [&](int64_t idx, float o, int raw) {
        if (g.out_type == QLIN_OUT_I32_ACC) static_cast<int *>(g.y)[idx] = raw;
        else if (g.out_type == QLIN_OUT_F32_ACC) static_cast<float *>(g.y)[idx] = o;
        else static_cast<uint16_t *>(g.y)[idx] = (uint16_t)bf16_bits(o);
    };

    if (g.nsplit == 1) {
        if (kw != 0) return;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            if (nsub[r] >= N) continue;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if (SWAP) {
                    const int m = m0 + mt * 16 + r16;
                    const int n = nsub[r] + 4 * quarter;
                    if (m >= M || !col_ok) continue;
                    if (g.out_type == QLIN_OUT_I32_ACC) {
                        *reinterpret_cast<int4 *>(static_cast<int *>(g.y) + (int64_t)m * N + n) =
                            make_int4((int)acc[r][mt][0], (int)acc[r][mt][1], (int)acc[r][mt][2],
                                      (int)acc[r][mt][3]);
                    } else {
                        float o[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) o[i] = scaled((float)acc[r][mt][i], r, mt, i);
                        if (g.out_type == QLIN_OUT_F32_ACC) {
                            *reinterpret_cast<float4 *>(static_cast<float *>(g.y) + (int64_t)m * N + n) =
                                make_float4(o[0], o[1], o[2], o[3]);
                        } else {
                            *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(g.y) + (int64_t)m * N + n) =
                                make_uint2(bf16_bits(o[0]) | (bf16_bits(o[1]) << 16),
                                           bf16_bits(o[2]) | (bf16_bits(o[3]) << 16));
                        }
                    }
                } else {
                    const int n = nsub[r] + r16;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m = m0 + mt * 16 + 4 * quarter + i;
                        if (m >= M || !col_ok) continue;
                        store1((int64_t)m * N + n, scaled((float)acc[r][mt][i], r, mt, i), (int)acc[r][mt][i]);
                    }
                }
            }
        }
        return;
    }

    // Split-K: the partitions' partial sums are combined in one of two ways.
    //
    // Packed (exact formats: int8, and fp8 with per-channel scales): one
    // returning 64-bit atomic per output.  A partition's sum is an integer:
    // int8 sums are int32, and fp8 products are whole multiples of 2^-18, so
    // every fp32 partial sum of them is too and p * 2^18 converts exactly.
    // Each partition adds p + 2^52 to a zeroed element; while |sum| < 2^51
    // the value returned, old = S + c * 2^52, gives the number c of
    // partitions that came before and their exact sum S.  The partition that
    // sees c = nsplit - 1 holds the total, writes the output and zeroes the
    // element.  One round trip, and the result does not depend on the order.
    if constexpr (FMT != FMT_BLOCK) {
        if (g.packed) {
            if (kw != 0) return;
            unsigned long long *ws64 = static_cast<unsigned long long *>(g.acc_ws);
            const unsigned long long kUnit = 1ull << 52, kHalf = 1ull << 51;
            // per 16-token fragment: all of the lane's atomics first (one
            // round trip: the addends and addresses are all formed before the
            // first atomic, so that none waits for another; elements past M
            // or N are masked off), then the outputs of the elements this
            // partition completes
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                unsigned long long old[NR][4], add[NR][4];
                long long val[NR][4];
                unsigned long long *dst[NR][4];
                bool live[NR][4];
#pragma unroll
                for (int r = 0; r < NR; ++r)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m = token_of(mt, i);
                        const int n = SWAP ? nsub[r] + 4 * quarter + i : nsub[r] + r16;
                        if constexpr (FMT == FMT_I8) val[r][i] = (long long)acc[r][mt][i];
                        else val[r][i] = (long long)(acc[r][mt][i] * 262144.0f);
                        live[r][i] = m < M && nsub[r] < N && col_ok;
                        add[r][i] = (unsigned long long)(val[r][i] + (long long)kUnit);
                        // (kept in a register of its own: formed inside the
                        // masked branch, every addend would reuse one
                        // register and each atomic would wait for the last)
                        asm volatile("" : "+v"(add[r][i]));
                        dst[r][i] = &ws64[(int64_t)m * N + n];
                        old[r][i] = 0;
                    }
#pragma unroll
                for (int r = 0; r < NR; ++r)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (live[r][i])
                            old[r][i] = __hip_atomic_fetch_add(dst[r][i], add[r][i], __ATOMIC_RELAXED,
                                                               __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    if (nsub[r] >= N) continue;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m = token_of(mt, i);
                        const int n = SWAP ? nsub[r] + 4 * quarter + i : nsub[r] + r16;
                        if (m >= M || !col_ok) continue;
                        const int64_t idx = (int64_t)m * N + n;
                        const unsigned long long before = (old[r][i] + kHalf) >> 52;
                        if (before != (unsigned long long)(g.nsplit - 1)) continue;
                        const long long total = (long long)(old[r][i] - before * kUnit) + val[r][i];
                        float t;
                        if constexpr (FMT == FMT_I8) t = (float)total;
                        else t = (float)((double)total * (1.0 / 262144.0));
                        store1(idx, scaled(t, r, mt, i), (int)total);
                        __hip_atomic_store(&ws64[idx], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
            }
            return;
        }
    }

    // Slices (any format): each partition stores its partial sums into its
    // own slice of the workspace with device-coherent stores, waits until
    // they are acknowledged, and counts its arrival for the tile.  The last
    // partition to arrive adds the slices in partition order (so the result
    // is deterministic), writes the output, and zeroes the slices and the
    // counter.
    acc_s *part = static_cast<acc_s *>(g.acc_ws);
    const int64_t slice = g.slice;
    if (kw == 0) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            if (nsub[r] >= N) continue;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = token_of(mt, i);
                    const int n = SWAP ? nsub[r] + 4 * quarter + i : nsub[r] + r16;
                    if (m < M && col_ok)
                        __hip_atomic_store(&part[blockIdx.z * slice + (int64_t)m * N + n],
                                           (acc_s)acc[r][mt][i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
        }
    }
    wait_memory_idle();
    __syncthreads();
    const int tile = blockIdx.y * gridDim.x + blockIdx.x;
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(&g.counters[tile], 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (uint32_t)(g.nsplit - 1);
    }
    __syncthreads();
    if (!s_last) return;
    const int tn = min(TN, N - n_tile0);   // a multiple of 8
    reduce_slices(part, slice, N, m0, n_tile0, R, tn, g.nsplit, (int)threadIdx.x, nthreads,
                  [&](int m, int n, const acc_s (&v)[4]) {
#pragma unroll
                      for (int i = 0; i < 4; ++i) {
                          float o;
                          if constexpr (FMT == FMT_BLOCK) o = v[i];
                          else if constexpr (FUSE) o = ((float)v[i] * s_rowscale[m - m0]) * g.wsc[n + i];
                          else o = ((float)v[i] * g.xs[m]) * g.wsc[n + i];
                          store1((int64_t)m * N + n + i, o, (int)v[i]);
                      }
                  });
    if (threadIdx.x == 0)
        __hip_atomic_store(&g.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// prefetch depth: 8 blocks of 16 weight rows in flight per wave (2 for NR = 4)
#define QLIN_PF(NR_, XC_) (NR_ >= 4 ? 2 : 8 / NR_)
// the block format's variants: 4 blocks (2 for NR = 2, 1 for NR = 4).  Each
// of its slots also waits for a block scale, and every block is scaled on
// the vector ALU; on its workload 4 measured ~3 % faster than 8, 6 in
// between, 2 slower.  The other formats measured 3 % slower at 6.
#define QLIN_PF_BLOCK(NR_, XC_) (NR_ >= 4 ? 1 : 4 / NR_)
// direct activations hold a slot's activation fragments too: half the depth
// at 32-token tiles
#define QLIN_PF_DIRECT(PF_, MT_) ((PF_) / (MT_) > 0 ? (PF_) / (MT_) : 1)

typedef void (*gemm_fn)(GemmLaunch);

// The kernel for a (format, schedule, tile) choice, or null; defined by the
// per-format source files.  xc: register chunks of the in-kernel
// quantization (0 = codes come quantized); nt: the skinny kernel's weights
// with the non-temporal cache policy.
gemm_fn gemm_pick_fp8(bool swap, int tile_m, int nr, int xc, bool nt);
gemm_fn gemm_pick_i8(bool swap, int tile_m, int nr, int xc, bool nt);
gemm_fn gemm_pick_block(bool swap, int tile_m, int nr, int xc, bool nt);

}  // namespace qlin
