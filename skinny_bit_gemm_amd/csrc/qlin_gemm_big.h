// qlin_gemm_big.h -- the large-M side of the crossover: a tiled quantized
// GEMM for token counts past the skinny range (M = 64 .. 512 and beyond),
// where the product turns matrix-core-bound.  Same formats, layouts,
// numerics and split-K slice reduction as the skinny kernel; included by the
// per-format source files.
//
// Product: "Building a High-Performance and Portable vLLM Linear Backend
// with Helion", sections "Scope" and "Kernel Implementation"; the pages hand
// num_tokens > 32 to a general kernel (section "Hybrid Dispatch"), which
// here is this one.
//
// Work decomposition.  A workgroup of 4 waves owns a BM x 128 tile of the
// output (tokens x channels) and a range of 128-wide K blocks, with
// 16x16x128 fp8 (or 16x16x64 int8) matrix-core instructions on the same
// lane -> (row, k) fragment assignment as the skinny kernel.  Two variants:
//   - staged weights: the waves form a 2 x 2 grid, each computing
//     (BM/2) x 64, and both operand tiles go through the LDS;
//   - direct weights (BD): each wave computes all BM tokens x 32 channels
//     and loads its own weight fragments straight into registers (a ring of
//     STAGES blocks, refilled in place); only the token tile goes through
//     the LDS.  A CU's LDS then carries the token fragments only: per
//     matrix-core instruction, 1.25 KiB of reads and copies instead of 1.5.
//
// Operand staging.  The LDS tiles of a K block are copied by the memory
// system straight into LDS (buffer loads with the LDS bit: lane l's 16
// bytes land 16 l bytes past the wave's LDS address), through a ring of
// STAGES buffers, STAGES - 1 blocks ahead of the computation, with one
// barrier per block.
// A tile is stored row by row, 128 bytes per row, 16-byte chunk c of row r
// at position c ^ (r & 7): one request copies 8 whole rows (1 KB) with a
// per-lane offset that never changes, and the fragment reads (8 lanes of a
// pass on 8 consecutive rows, same chunk) hit 8 different bank groups.  No
// register holds staged data.  Every request is issued on every path
// (past-the-end ones out of range, which store zeros), so each wave has the
// same number of requests per block and an explicit wait counts exactly.
//
// Tile order.  The grid is one-dimensional and the hardware deals workgroups
// to the 8 XCDs round robin; tiles are numbered so that the M tiles sharing
// one 128-channel weight slab land on the same XCD back to back, and its L2
// serves the slab to all of them.

#pragma once

#include "qlin_gemm.h"

namespace qlin {

constexpr int kBigN = 128;         // channels per tile
constexpr int kBigThreads = 256;   // 4 waves

// BD (direct weights): the waves split the tile's channels only (each wave
// all BM tokens x 32 channels) and load their weight fragments straight
// into registers, a ring of STAGES blocks like the LDS ring; only the
// token tile goes through the LDS.  Otherwise the waves form a 2 x 2 grid
// of (BM/2) x 64 and both operand tiles go through the LDS.
template <int FMT, int BM, bool BD>
struct BigTile {
    static constexpr int WM = BD ? BM : BM / 2;   // rows per wave
    static constexpr int FM = WM / 16;            // 16-row fragments per wave
    static constexpr int FN = BD ? 2 : 4;         // 16-channel fragments per wave
    static constexpr int WN = 16 * FN;            // channels per wave
    // LDS buffers (blocks in flight: STAGES - 1), sized so that two
    // workgroups share a compute unit: one computes while the other waits
    // (BD: 4, or 2 for the block format's 128-token tiles, whose per-block
    // scaling leaves registers for two weight slots only)
    static constexpr int STAGES = BD ? (FMT == FMT_BLOCK && BM == 128 ? 2 : 4) : BM == 64 ? 3 : 2;
    static constexpr int WG_PER_CU = 2;
    static constexpr int A_BYTES = BM * kGroup;
    static constexpr int B_BYTES = BD ? 0 : kBigN * kGroup;
    // block format: token scales of the block (one 64-entry group per wave,
    // entries past BM zero) and the weight block's scale
    static constexpr int S_BYTES = FMT == FMT_BLOCK ? 4 * 64 * 4 + 16 : 0;
    static constexpr int BUF_BYTES = A_BYTES + B_BYTES + S_BYTES;
    static constexpr int REQ_A = BM / 8 / 4;   // 8-row requests per wave and block
    // weight requests per wave and block: 8-row copies, or (BD) two 16-byte
    // halves per fragment
    static constexpr int REQ_B = BD ? 2 * FN : kBigN / 8 / 4;
    static constexpr int REQ = REQ_A + REQ_B + (FMT == FMT_BLOCK ? 2 : 0);
    // requests younger than block j's token tile when block j is due: the
    // younger blocks' (and, BD, one more block of weights, whose ring runs
    // one block further ahead)
    static constexpr int WAIT = (STAGES - 2) * REQ + (BD ? REQ_B : 0);
    static_assert(WAIT < 64, "vmcnt holds at most 63");
    static_assert(STAGES * BUF_BYTES * WG_PER_CU <= 160 * 1024, "LDS of a compute unit");
};

// Fragment reads from LDS, as inline-assembly blocks that end with their
// own wait.  (Written as plain loads, the compiler would make every LDS
// read wait for all the LDS copies in flight, the later blocks' included,
// which would drain the ring every block.)  A fragment is two 16-byte
// halves at the lane's lo / hi chunk addresses; the 4 channel fragments of
// a wave are 2048 bytes (16 rows) apart.
#define QLIN_RD(d, a, off) "ds_read_b128 %[" #d "], %[" #a "] offset:" #off "\n"
#define QLIN_RD_B                                                                              \
    QLIN_RD(b0l, bl, 0) QLIN_RD(b0h, bh, 0) QLIN_RD(b1l, bl, 2048) QLIN_RD(b1h, bh, 2048)      \
        QLIN_RD(b2l, bl, 4096) QLIN_RD(b2h, bh, 4096) QLIN_RD(b3l, bl, 6144) QLIN_RD(b3h, bh, 6144)
#define QLIN_OUT_B                                                                                \
    [b0l] "=&v"(b[0][0]), [b0h] "=&v"(b[0][1]), [b1l] "=&v"(b[1][0]), [b1h] "=&v"(b[1][1]),      \
        [b2l] "=&v"(b[2][0]), [b2h] "=&v"(b[2][1]), [b3l] "=&v"(b[3][0]), [b3h] "=&v"(b[3][1])

// the wave's 4 channel fragments and its first token fragment
__device__ __forceinline__ void lds_frags_first(v4i (&a)[2], v4i (&b)[4][2], uint32_t al, uint32_t ah,
                                                uint32_t bl, uint32_t bh) {
    asm volatile(QLIN_RD_B QLIN_RD(a0l, al, 0) QLIN_RD(a0h, ah, 0) "s_waitcnt lgkmcnt(0)"
                 : QLIN_OUT_B, [a0l] "=&v"(a[0]), [a0h] "=&v"(a[1])
                 : [bl] "v"(bl), [bh] "v"(bh), [al] "v"(al), [ah] "v"(ah)
                 : "memory");
}

// block format: the same, plus the lane's 4 token scales of each of FM
// token fragments (64 bytes, 16 rows, apart) and the weight block's scale
template <int FM>
__device__ __forceinline__ void lds_frags_first_scaled(v4i (&a)[2], v4i (&b)[4][2], v4i (&sa)[FM], float &sw,
                                                       uint32_t al, uint32_t ah, uint32_t bl, uint32_t bh,
                                                       uint32_t sl, uint32_t sb) {
    static_assert(FM == 2 || FM == 4, "2 or 4 token fragments");
    if constexpr (FM == 2)
        asm volatile(QLIN_RD_B QLIN_RD(a0l, al, 0) QLIN_RD(a0h, ah, 0) QLIN_RD(s0, sl, 0) QLIN_RD(s1, sl, 64)
                     "ds_read_b32 %[sw], %[sb]\n"
                     "s_waitcnt lgkmcnt(0)"
                     : QLIN_OUT_B, [a0l] "=&v"(a[0]), [a0h] "=&v"(a[1]), [s0] "=&v"(sa[0]), [s1] "=&v"(sa[1]),
                       [sw] "=&v"(sw)
                     : [bl] "v"(bl), [bh] "v"(bh), [al] "v"(al), [ah] "v"(ah), [sl] "v"(sl), [sb] "v"(sb)
                     : "memory");
    else
        asm volatile(QLIN_RD_B QLIN_RD(a0l, al, 0) QLIN_RD(a0h, ah, 0) QLIN_RD(s0, sl, 0) QLIN_RD(s1, sl, 64)
                         QLIN_RD(s2, sl, 128) QLIN_RD(s3, sl, 192) "ds_read_b32 %[sw], %[sb]\n"
                     "s_waitcnt lgkmcnt(0)"
                     : QLIN_OUT_B, [a0l] "=&v"(a[0]), [a0h] "=&v"(a[1]), [s0] "=&v"(sa[0]), [s1] "=&v"(sa[1]),
                       [s2] "=&v"(sa[2]), [s3] "=&v"(sa[3]), [sw] "=&v"(sw)
                     : [bl] "v"(bl), [bh] "v"(bh), [al] "v"(al), [ah] "v"(ah), [sl] "v"(sl), [sb] "v"(sb)
                     : "memory");
}

// a token fragment, the lane's 4 token scales of it and the weight block's
// scale (block format, direct weights)
__device__ __forceinline__ void lds_frag_scaled(v4i (&a)[2], v4i &sa, float &sw, uint32_t al, uint32_t ah,
                                                uint32_t sl, uint32_t sb) {
    asm volatile("ds_read_b128 %[a0l], %[al]\n"
                 "ds_read_b128 %[a0h], %[ah]\n"
                 "ds_read_b128 %[s0], %[sl]\n"
                 "ds_read_b32 %[sw], %[sb]\n"
                 "s_waitcnt lgkmcnt(0)"
                 : [a0l] "=&v"(a[0]), [a0h] "=&v"(a[1]), [s0] "=&v"(sa), [sw] "=&v"(sw)
                 : [al] "v"(al), [ah] "v"(ah), [sl] "v"(sl), [sb] "v"(sb)
                 : "memory");
}

// one more token fragment
__device__ __forceinline__ void lds_frag(v4i (&a)[2], uint32_t al, uint32_t ah) {
    asm volatile(QLIN_RD(a0l, al, 0) QLIN_RD(a0h, ah, 0) "s_waitcnt lgkmcnt(0)"
                 : [a0l] "=&v"(a[0]), [a0h] "=&v"(a[1])
                 : [al] "v"(al), [ah] "v"(ah)
                 : "memory");
}
#undef QLIN_RD
#undef QLIN_RD_B
#undef QLIN_OUT_B

__device__ __forceinline__ v8i join4(v4i lo, v4i hi) {
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <int FMT, int BM, bool BD>
__global__ __launch_bounds__(kBigThreads, 2) void gemm_big_kernel(GemmLaunch g) {   // two per compute unit
    typedef BigTile<FMT, BM, BD> T;
    typedef typename AccT<FMT>::type acc_t;
    typedef typename AccT<FMT>::scalar acc_s;
    __shared__ __attribute__((aligned(16))) uint8_t lds[T::STAGES * T::BUF_BYTES];
    __shared__ int s_last;

    const int M = g.M, N = g.N, K = g.K;
    const int G = (K + kGroup - 1) / kGroup;

    // tile of this workgroup (XCD-aware order, see above)
    const int n8 = (g.n_tiles + 7) & ~7;
    const int per_split = g.m_tiles * n8;
    const int L = blockIdx.x % per_split;
    const int z = blockIdx.x / per_split;
    const int r = L >> 3;
    const int n_tile = (L & 7) + 8 * (r / g.m_tiles);
    const int m_tile = r % g.m_tiles;
    if (n_tile >= g.n_tiles) return;
    const int m0 = m_tile * BM, n0 = n_tile * kBigN;
    const int kb_begin = z * g.kb_per_split;
    const int kb_end = min(g.nkb, kb_begin + g.kb_per_split);
    const int nsteps = kb_end - kb_begin;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = BD ? 0 : wave & 1, wn = BD ? wave : wave >> 1;
    const int r16 = lane & 15, quarter = lane >> 4;
    const int rows_a = min(BM, M - m0), rows_b = min(kBigN, N - n0);

    // operand tiles through buffer resources (rows past M or N read zeros)
    const __amdgpu_buffer_rsrc_t ars = buffer_rsrc(g.xq + (int64_t)m0 * K, (uint32_t)(rows_a * K));
    // weights: row-major rows n0 .., or the packed 16-row groups n0 / 16 ..
    // (2 KiB per group and K block; N is a multiple of 16)
    const bool wpk = g.w_packed != 0;
    const __amdgpu_buffer_rsrc_t brs =
        wpk ? buffer_rsrc(g.wq + (int64_t)(n0 / kPackRows) * g.nkb * kPackBlock,
                          (uint32_t)(rows_b / kPackRows * g.nkb * kPackBlock))
            : buffer_rsrc(g.wq + (int64_t)n0 * K, (uint32_t)(rows_b * K));
    const __amdgpu_buffer_rsrc_t srs =
        buffer_rsrc(FMT == FMT_BLOCK ? (const void *)(g.xs + (int64_t)m0 * G) : (const void *)g.xs,
                    FMT == FMT_BLOCK ? (uint32_t)(rows_a * G * 4) : 0u);
    const __amdgpu_buffer_rsrc_t wrs =
        buffer_rsrc(g.wsc + (FMT == FMT_BLOCK ? (int64_t)(n0 / kGroup) * G : 0), FMT == FMT_BLOCK ? (uint32_t)(G * 4) : 0u);

    // lane l of an 8-row request: row l / 8 of the request, LDS chunk
    // position l % 8, which holds source chunk (l % 8) ^ (l / 8)
    const int lrow = lane >> 3, lchunk = (lane & 7) ^ lrow;
    const uint32_t lane_off = (uint32_t)(lrow * K + lchunk * 16);
    // Packed weights keep their own order in LDS: the tile's 16-row groups,
    // 2 KiB apart (as 16 row-major rows would be), each the packed block
    // itself, so one request copies 1 KiB of consecutive bytes (half a
    // group) to consecutive LDS, and a lane's fragment halves are at 16 lane
    // and 16 lane + 1 KiB of its group.
    typedef __attribute__((address_space(3))) void *lds_ptr;

    // requests of block j of the range into LDS buffer `base` (the token
    // tile, unless BD the weight tile, and the block format's scales;
    // buffers are addressed by their 32-bit LDS addresses)
    auto issue_a = [&](int j, uint32_t base) {
        const bool live = j < nsteps;
        const int kb = kb_begin + j;
        const int k0 = kb * kGroup;
        const bool kin = live && k0 + lchunk * 16 < K;
#pragma unroll
        for (int i = 0; i < T::REQ_A; ++i) {
            const int r0 = (wave * T::REQ_A + i) * 8;
            const bool ok = kin && r0 + lrow < rows_a;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, (lds_ptr)(uintptr_t)(base + r0 * kGroup), 16,
                                                     ok ? (uint32_t)(r0 * K) + lane_off : kOutOfRange,
                                                     __builtin_amdgcn_readfirstlane(k0), 0, 0);
        }
        if constexpr (!BD) {
#pragma unroll
            for (int i = 0; i < T::REQ_B; ++i) {
                const int r0 = (wave * T::REQ_B + i) * 8;
                if (wpk) {
                    // request j = r0 / 8 is half j % 2 of group j / 2 (the packed
                    // layout holds zeros past K)
                    const int j = r0 >> 3;
                    const bool ok = live && (j >> 1) * kPackRows < rows_b;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        brs, (lds_ptr)(uintptr_t)(base + T::A_BYTES + r0 * kGroup), 16,
                        ok ? (uint32_t)lane * 16 : kOutOfRange,
                        __builtin_amdgcn_readfirstlane(((j >> 1) * g.nkb + kb) * kPackBlock + (j & 1) * (kPackBlock / 2)),
                        0, 0);
                } else {
                    const bool ok = kin && r0 + lrow < rows_b;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(brs, (lds_ptr)(uintptr_t)(base + T::A_BYTES + r0 * kGroup), 16,
                                                             ok ? (uint32_t)(r0 * K) + lane_off : kOutOfRange,
                                                             __builtin_amdgcn_readfirstlane(k0), 0, 0);
                }
            }
        }
        if constexpr (FMT == FMT_BLOCK) {
            const uint32_t sbase = base + T::A_BYTES + T::B_BYTES;
            const int e = wave * 64 + lane;   // token row of this lane's scale
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                srs, (lds_ptr)(uintptr_t)(sbase + wave * 64 * 4), 4,
                live && e < rows_a ? (uint32_t)((e * G + kb) * 4) : kOutOfRange, 0, 0, 0);
            // the weight block's scale: lane 0 of every wave, to the same slot
            if (lane == 0)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (lds_ptr)(uintptr_t)(sbase + 4 * 64 * 4), 4,
                                                         live ? (uint32_t)(kb * 4) : kOutOfRange, 0, 0, 0);
        }
    };
    // direct weights: block j's fragments of the wave's channels into the
    // register slot `bdst`
    auto issue_b = [&](int j, v8i (&bdst)[T::FN]) {
        const bool live = j < nsteps;
        const int kb = kb_begin + j;
        const int k0 = kb * kGroup;
        // the wave's FN fragments of 16 channels straight into registers:
        // packed, the two 1 KiB halves of the group's block; row-major, the
        // lane's row, bytes 32 quarter .. + 31 of the block (zeros past K and
        // past the tile's rows).  One code path for both layouts (offsets
        // selected, not branched on), so the loads of every slot land in the
        // same registers.
#pragma unroll
        for (int fn = 0; fn < T::FN; ++fn) {
            const int c0 = wn * T::WN + fn * 16;   // the fragment's first channel in the tile
            const int kq = k0 + quarter * 32;
            const uint32_t voff = wpk ? (uint32_t)lane * 16 : (uint32_t)((c0 + r16) * K + quarter * 32);
            const int soff = __builtin_amdgcn_readfirstlane(wpk ? ((c0 / kPackRows) * g.nkb + kb) * kPackBlock : k0);
            const int hoff = wpk ? kPackBlock / 2 : 16;
            const bool lo_ok = live && (wpk ? c0 < rows_b : kq < K);
            const bool hi_ok = live && (wpk ? c0 < rows_b : kq + 16 < K);
            const v4i lo = __builtin_amdgcn_raw_buffer_load_b128(brs, lo_ok ? voff : kOutOfRange, soff, 0);
            const v4i hi = __builtin_amdgcn_raw_buffer_load_b128(brs, hi_ok ? voff : kOutOfRange, soff + hoff, 0);
            bdst[fn] = join4(lo, hi);
        }
    };

    acc_t acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j) acc[i][j] = acc_t{0, 0, 0, 0};

    // the lane's fragment: row (16-row group base + r16), chunks 2 quarter
    // and 2 quarter + 1, at positions chunk ^ (row & 7); LDS byte addresses
    const int a_row = wm * T::WM + r16, b_row = wn * T::WN + r16;
    const int sw = r16 & 7;   // row & 7 (group bases are multiples of 16)
    const uint32_t c_lo = ((2 * quarter) ^ sw) * 16, c_hi = ((2 * quarter + 1) ^ sw) * 16;
    // the lane's weight fragment halves within the B tile: row-major (the
    // swizzled rows), or packed (the wave's first 16-row group, 16 lane and
    // 16 lane + 1 KiB)
    const uint32_t b_lo = wpk ? (uint32_t)((wn * T::WN / kPackRows) * kPackBlock + lane * 16)
                              : (uint32_t)(b_row * kGroup) + c_lo;
    const uint32_t b_hi = wpk ? b_lo + kPackBlock / 2 : (uint32_t)(b_row * kGroup) + c_hi;
    // one block from the buffer at b0: the channel fragments and the first
    // token fragment, its products, then the requests of a later block
    // (`after`, so that they leave while the matrix core works), then the
    // other token fragments and their products
    // (direct weights: the channel fragments are the registers `bq`, and
    // each token fragment is read with its token scales)
    auto compute = [&](uint32_t b0, const v8i (&bq)[T::FN], auto after) {
        const uint32_t al = b0 + a_row * kGroup + c_lo, ah = b0 + a_row * kGroup + c_hi;
        const uint32_t bl = b0 + T::A_BYTES + b_lo, bh = b0 + T::A_BYTES + b_hi;
        v4i a[2], b[T::FN][2];
        v8i bf[T::FN];
        if constexpr (BD) {
            const uint32_t sbase = b0 + T::A_BYTES;
#pragma unroll
            for (int fm = 0; fm < T::FM; ++fm) {
                const uint32_t ao = fm * 16 * kGroup;
                v8i af;
                float c[4];
                if constexpr (FMT == FMT_BLOCK) {
                    // this block's token scales for the lane's 4 rows, times
                    // the weight block's scale
                    v4i sa;
                    float swt;
                    lds_frag_scaled(a, sa, swt, al + ao, ah + ao, sbase + (fm * 16 + 4 * quarter) * 4,
                                    sbase + 4 * 64 * 4);
#pragma unroll
                    for (int i = 0; i < 4; ++i) c[i] = __int_as_float(sa[i]) * swt;
                } else {
                    lds_frag(a, al + ao, ah + ao);
                }
                af = join4(a[0], a[1]);
#pragma unroll
                for (int fn = 0; fn < T::FN; ++fn) {
                    if constexpr (FMT == FMT_BLOCK) {
                        const v4f p4 = block_mma<FMT>(af, bq[fn], v4f{0, 0, 0, 0});
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[fm][fn][i] += p4[i] * c[i];
                    } else {
                        acc[fm][fn] = block_mma<FMT>(af, bq[fn], acc[fm][fn]);
                    }
                }
                if (fm == 0) {
                    __builtin_amdgcn_sched_barrier(0);
                    after();
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else if constexpr (FMT == FMT_BLOCK) {
            v4i sa[T::FM];
            float swt;
            const uint32_t sbase = b0 + T::A_BYTES + T::B_BYTES;
            lds_frags_first_scaled<T::FM>(a, b, sa, swt, al, ah, bl, bh, sbase + (wm * T::WM + 4 * quarter) * 4,
                                          sbase + 4 * 64 * 4);
#pragma unroll
            for (int fn = 0; fn < T::FN; ++fn) bf[fn] = join4(b[fn][0], b[fn][1]);
#pragma unroll
            for (int fm = 0; fm < T::FM; ++fm) {
                if (fm > 0) lds_frag(a, al + fm * 16 * kGroup, ah + fm * 16 * kGroup);
                // this block's token scales for the lane's 4 rows, times the
                // weight block's scale
                const v8i af = join4(a[0], a[1]);
                const float c0 = __int_as_float(sa[fm][0]) * swt, c1 = __int_as_float(sa[fm][1]) * swt;
                const float c2 = __int_as_float(sa[fm][2]) * swt, c3 = __int_as_float(sa[fm][3]) * swt;
#pragma unroll
                for (int fn = 0; fn < T::FN; ++fn) {
                    const v4f p4 = block_mma<FMT>(af, bf[fn], v4f{0, 0, 0, 0});
                    acc[fm][fn][0] += p4[0] * c0;
                    acc[fm][fn][1] += p4[1] * c1;
                    acc[fm][fn][2] += p4[2] * c2;
                    acc[fm][fn][3] += p4[3] * c3;
                }
                if (fm == 0) {
                    __builtin_amdgcn_sched_barrier(0);
                    after();
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else {
            lds_frags_first(a, b, al, ah, bl, bh);
#pragma unroll
            for (int fn = 0; fn < T::FN; ++fn) bf[fn] = join4(b[fn][0], b[fn][1]);
#pragma unroll
            for (int fm = 0; fm < T::FM; ++fm) {
                if (fm > 0) lds_frag(a, al + fm * 16 * kGroup, ah + fm * 16 * kGroup);
                const v8i af = join4(a[0], a[1]);
#pragma unroll
                for (int fn = 0; fn < T::FN; ++fn) acc[fm][fn] = block_mma<FMT>(af, bf[fn], acc[fm][fn]);
                if (fm == 0) {
                    __builtin_amdgcn_sched_barrier(0);
                    after();
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    };

    // ---- main loop.  At block j the requests of blocks j .. j + STAGES - 2
    // are in flight; wait until only the younger STAGES - 2 blocks' are, then
    // the barrier makes block j visible to every wave and tells that every
    // wave has finished block j - 1, whose buffer then takes block
    // j + STAGES - 1.  The barrier is a bare one (every wave has waited for
    // its own copies, and its reads of a buffer completed inside its
    // fragment-read blocks): a fence would wait for the copies in flight as
    // well.  Every pass issues its requests, past the range too (they are
    // out of range), so the waits count exactly; only the products are
    // skipped there.  Unrolled by STAGES, so the buffers' addresses are
    // constants.
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr)lds;   // LDS address of the ring
    // Direct weights: a register ring, slot u holding blocks j = u mod
    // STAGES, refilled in place (block j + STAGES) once block j's products
    // are issued, so each slot keeps its registers; the weights run one
    // block further ahead than the token tiles.  Issue order: B(0), then
    // A(0) B(1), A(1) B(2), ..., and in pass j A(j + STAGES - 1) then
    // B(j + STAGES), so that T::WAIT requests are younger than A(j) at
    // block j on every pass.
    v8i bq[BD ? T::STAGES : 1][T::FN];
    if constexpr (BD) issue_b(0, bq[0]);
#pragma unroll
    for (int st = 0; st < T::STAGES - 1; ++st) {
        issue_a(st, lds0 + st * T::BUF_BYTES);
        if constexpr (BD) issue_b(st + 1, bq[BD ? st + 1 : 0]);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int j0 = 0; j0 < nsteps; j0 += T::STAGES) {
#pragma unroll
        for (int u = 0; u < T::STAGES; ++u) {
            const int j = j0 + u;
            const uint32_t next = lds0 + ((u + T::STAGES - 1) % T::STAGES) * T::BUF_BYTES;
            __builtin_amdgcn_s_waitcnt(vmcnt_only(T::WAIT));
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            auto req = [&]() { issue_a(j + T::STAGES - 1, next); };
            if (j < nsteps) compute(lds0 + u * T::BUF_BYTES, bq[BD ? u : 0], req);
            else req();
            if constexpr (BD) {
                __builtin_amdgcn_sched_barrier(0);
                issue_b(j + T::STAGES, bq[BD ? u : 0]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // the past-the-end copies still in flight land in LDS before the
    // workgroup can end
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));

    // ---- epilogue.  Lane layout of a 16x16 result: channel r16, tokens
    // 4 * quarter + i.
    const int mrow0 = m0 + wm * T::WM + 4 * quarter;
    const int ncol0 = n0 + wn * T::WN + r16;
    auto out_value = [&](acc_s v, int m, int n) -> float {
        if constexpr (FMT == FMT_BLOCK) return (float)v;
        else return ((float)v * g.xs[m]) * g.wsc[n];
    };
    auto store1 = [&](int64_t idx, float o, int raw) {
        if (g.out_type == QLIN_OUT_I32_ACC) static_cast<int *>(g.y)[idx] = raw;
        else if (g.out_type == QLIN_OUT_F32_ACC) static_cast<float *>(g.y)[idx] = o;
        else static_cast<uint16_t *>(g.y)[idx] = (uint16_t)bf16_bits(o);
    };

    if (g.nsplit == 1) {
#pragma unroll
        for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < T::FN; ++fn) {
                const int n = ncol0 + fn * 16;
                if (n >= N) continue;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = mrow0 + fm * 16 + i;
                    if (m < M) store1((int64_t)m * N + n, out_value(acc[fm][fn][i], m, n), (int)acc[fm][fn][i]);
                }
            }
        return;
    }

    // Split-K through slices: each partition stores its partial sums into its
    // own slice with device-coherent stores, waits for them, counts its
    // arrival; the last one adds the slices in partition order, writes the
    // output and leaves slices and counter zero.
    acc_s *part = static_cast<acc_s *>(g.acc_ws);
    const int64_t slice = g.slice;
#pragma unroll
    for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < T::FN; ++fn) {
            const int n = ncol0 + fn * 16;
            if (n >= N) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = mrow0 + fm * 16 + i;
                if (m < M)
                    __hip_atomic_store(&part[z * slice + (int64_t)m * N + n], (acc_s)acc[fm][fn][i],
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    wait_memory_idle();
    __syncthreads();
    const int tile = m_tile * g.n_tiles + n_tile;
    if (t == 0) {
        const uint32_t prev =
            __hip_atomic_fetch_add(&g.counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (uint32_t)(g.nsplit - 1);
    }
    __syncthreads();
    if (!s_last) return;
    reduce_slices(part, slice, N, m0, n0, rows_a, rows_b, g.nsplit, t, kBigThreads,
                  [&](int m, int n, const acc_s (&v)[4]) {
#pragma unroll
                      for (int i = 0; i < 4; ++i) store1((int64_t)m * N + n + i, out_value(v[i], m, n + i), (int)v[i]);
                  });
    if (t == 0) __hip_atomic_store(&g.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace qlin
