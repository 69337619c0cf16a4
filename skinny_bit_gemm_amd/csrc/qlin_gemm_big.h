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
// output (tokens x channels) and a range of 128-wide K blocks; the waves
// form a 2 x 2 grid, each computing (BM/2) x 64 with 16x16x128 fp8 (or
// 16x16x64 int8) matrix-core instructions on the same lane -> (row, k)
// fragment assignment as the skinny kernel.  Both operand tiles of a K block
// go through LDS (double buffered, one barrier per block), each as
// [half][quarter][row][16 bytes] with an odd number of row slots per group:
// the fragment reads (16 lanes on 16 consecutive rows) and the staging writes
// (8 lanes on the 8 groups of one row) are free of bank conflicts.  The
// tiles are requested from memory STAGES blocks ahead into registers (every
// request issued on every path, past-the-end ones with out-of-range
// offsets, so the waits count exactly).
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

template <int FMT, int BM>
struct BigTile {
    static constexpr int WM = BM / 2;        // rows per wave
    static constexpr int FM = WM / 16;       // 16-row fragments per wave
    static constexpr int FN = 4;             // 16-channel fragments per wave (64 channels)
    static constexpr int PA = BM + 1;        // row slots per LDS group, odd
    static constexpr int PB = kBigN + 1;
    static constexpr int UA = BM * 8 / kBigThreads;      // 16-byte units per thread per block
    static constexpr int UB = kBigN * 8 / kBigThreads;
    static constexpr int STAGES = 3;                     // blocks requested ahead
    static constexpr int A_BYTES = 8 * PA * 16;
    static constexpr int B_BYTES = 8 * PB * 16;
    static constexpr int BUF_BYTES = A_BYTES + B_BYTES + (FMT == FMT_BLOCK ? BM * 4 : 0);
};

template <int FMT, int BM>
__global__ __launch_bounds__(kBigThreads) void gemm_big_kernel(GemmLaunch g) {
    typedef BigTile<FMT, BM> T;
    typedef typename AccT<FMT>::type acc_t;
    typedef typename AccT<FMT>::scalar acc_s;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * T::BUF_BYTES];
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
    const int wm = wave & 1, wn = wave >> 1;
    const int r16 = lane & 15, quarter = lane >> 4;
    const int rows_a = min(BM, M - m0), rows_b = min(kBigN, N - n0);

    // operand tiles through buffer resources (rows past M or N read zeros)
    const __amdgpu_buffer_rsrc_t ars = buffer_rsrc(g.xq + (int64_t)m0 * K, (uint32_t)(rows_a * K));
    const __amdgpu_buffer_rsrc_t brs = buffer_rsrc(g.wq + (int64_t)n0 * K, (uint32_t)(rows_b * K));
    const __amdgpu_buffer_rsrc_t srs =
        buffer_rsrc(FMT == FMT_BLOCK ? (const void *)(g.xs + (int64_t)m0 * G) : (const void *)g.xs,
                    FMT == FMT_BLOCK ? (uint32_t)(rows_a * G * 4) : 0u);

    // this thread's staging units: unit u = t + 256 i is (row u / 8, 16-byte
    // chunk u % 8) of the block; its LDS slot and its offset in the tile
    int a_lds[T::UA], b_lds[T::UB];
    uint32_t a_off[T::UA], b_off[T::UB];
    int a_k[T::UA], b_k[T::UB];
#pragma unroll
    for (int i = 0; i < T::UA; ++i) {
        const int u = t + kBigThreads * i, row = u >> 3, c = u & 7;
        a_lds[i] = (((c & 1) * 4 + (c >> 1)) * T::PA + row) * 16;
        a_off[i] = (uint32_t)(row * K + c * 16);
        a_k[i] = c * 16;
    }
#pragma unroll
    for (int i = 0; i < T::UB; ++i) {
        const int u = t + kBigThreads * i, row = u >> 3, c = u & 7;
        b_lds[i] = T::A_BYTES + (((c & 1) * 4 + (c >> 1)) * T::PB + row) * 16;
        b_off[i] = (uint32_t)(row * K + c * 16);
        b_k[i] = c * 16;
    }

    // register stages: the units of STAGES blocks in flight (block format:
    // also the token scales of the block and the weight block's scale)
    uint4 ra[T::STAGES][T::UA], rb[T::STAGES][T::UB];
    float rs[T::STAGES], rw[T::STAGES];
    const __amdgpu_buffer_rsrc_t wrs =
        buffer_rsrc(g.wsc + (FMT == FMT_BLOCK ? (int64_t)(n0 / kGroup) * G : 0), FMT == FMT_BLOCK ? (uint32_t)(G * 4) : 0u);
    auto request = [&](int st, int j) {   // block j of the range into stage st
        const bool live = j < nsteps;
        const int kb = kb_begin + j;
        const int k0 = kb * kGroup;
        const int boff = __builtin_amdgcn_readfirstlane(k0);
#pragma unroll
        for (int i = 0; i < T::UA; ++i) {
            const bool ok = live && k0 + a_k[i] < K;
            const v4i v = __builtin_amdgcn_raw_buffer_load_b128(ars, ok ? a_off[i] : kOutOfRange, boff, 0);
            ra[st][i] = make_uint4(v[0], v[1], v[2], v[3]);
        }
#pragma unroll
        for (int i = 0; i < T::UB; ++i) {
            const bool ok = live && k0 + b_k[i] < K;
            const v4i v = __builtin_amdgcn_raw_buffer_load_b128(brs, ok ? b_off[i] : kOutOfRange, boff, 0);
            rb[st][i] = make_uint4(v[0], v[1], v[2], v[3]);
        }
        if constexpr (FMT == FMT_BLOCK) {
            // token scales of the block (one per row, threads t < BM)
            const bool ok = live && t < BM;
            rs[st] = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(srs, ok ? (uint32_t)((t * G + kb) * 4) : kOutOfRange, 0, 0));
            rw[st] = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(wrs, live ? (uint32_t)(kb * 4) : kOutOfRange, 0, 0));
        }
    };
    float sw_now = 0.0f;                  // block format: weight block scale of the staged block
    auto stage = [&](int st, int buf) {   // stage st -> LDS buffer buf
        uint8_t *base = lds + buf * T::BUF_BYTES;
        if constexpr (FMT == FMT_BLOCK) sw_now = rw[st];
#pragma unroll
        for (int i = 0; i < T::UA; ++i) *reinterpret_cast<uint4 *>(base + a_lds[i]) = ra[st][i];
#pragma unroll
        for (int i = 0; i < T::UB; ++i) *reinterpret_cast<uint4 *>(base + b_lds[i]) = rb[st][i];
        if constexpr (FMT == FMT_BLOCK) {
            if (t < BM) reinterpret_cast<float *>(base + T::A_BYTES + T::B_BYTES)[t] = rs[st];
        }
    };

    acc_t acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j) acc[i][j] = acc_t{0, 0, 0, 0};

    // the lane's fragment slots: row r16 of 16-row group f, quarter `quarter`
    const int a_frag = (quarter * T::PA + wm * T::WM + r16) * 16;
    const int b_frag = T::A_BYTES + (quarter * T::PB + wn * 64 + r16) * 16;
    auto compute = [&](int buf) {
        const uint8_t *base = lds + buf * T::BUF_BYTES;
        v8i bf[T::FN];
#pragma unroll
        for (int fn = 0; fn < T::FN; ++fn) {
            const uint8_t *p = base + b_frag + fn * 16 * 16;
            bf[fn] = join(*reinterpret_cast<const uint4 *>(p),
                          *reinterpret_cast<const uint4 *>(p + 4 * T::PB * 16));
        }
        const float sw = sw_now;
#pragma unroll
        for (int fm = 0; fm < T::FM; ++fm) {
            const uint8_t *p = base + a_frag + fm * 16 * 16;
            const v8i af = join(*reinterpret_cast<const uint4 *>(p),
                                *reinterpret_cast<const uint4 *>(p + 4 * T::PA * 16));
            if constexpr (FMT == FMT_BLOCK) {
                // this block's token scales for the lane's 4 rows, times the
                // weight block's scale
                const float4 sa = *reinterpret_cast<const float4 *>(
                    base + T::A_BYTES + T::B_BYTES + (wm * T::WM + fm * 16 + 4 * quarter) * 4);
                const float c0 = sa.x * sw, c1 = sa.y * sw, c2 = sa.z * sw, c3 = sa.w * sw;
#pragma unroll
                for (int fn = 0; fn < T::FN; ++fn) {
                    const v4f p4 = block_mma<FMT>(af, bf[fn], v4f{0, 0, 0, 0});
                    acc[fm][fn][0] += p4[0] * c0;
                    acc[fm][fn][1] += p4[1] * c1;
                    acc[fm][fn][2] += p4[2] * c2;
                    acc[fm][fn][3] += p4[3] * c3;
                }
            } else {
#pragma unroll
                for (int fn = 0; fn < T::FN; ++fn) acc[fm][fn] = block_mma<FMT>(af, bf[fn], acc[fm][fn]);
            }
        }
    };

    // ---- main loop: STAGES blocks in flight, two LDS buffers, one barrier
    // per block.  Buffer j & 1 is rewritten at block j only after every wave
    // has passed the barrier of block j - 1, i.e. finished computing block
    // j - 2 from it.  Staging, the barrier and the requests run on every
    // pass (past the range they move zeros), so the waits count exactly;
    // only the computation is skipped there.
    // (the scheduling barriers keep the stages' requests in issue order)
#pragma unroll
    for (int st = 0; st < T::STAGES; ++st) {
        request(st, st);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int j0 = 0; j0 < nsteps; j0 += T::STAGES) {
#pragma unroll
        for (int st = 0; st < T::STAGES; ++st) {
            const int j = j0 + st;
            stage(st, j & 1);
            __syncthreads();
            request(st, j + T::STAGES);
            if (j < nsteps) compute(j & 1);
        }
    }

    // ---- epilogue.  Lane layout of a 16x16 result: channel r16, tokens
    // 4 * quarter + i.
    const int mrow0 = m0 + wm * T::WM + 4 * quarter;
    const int ncol0 = n0 + wn * 64 + r16;
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
    const int64_t slice = (int64_t)M * N;
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
    for (int e = t; e < rows_a * rows_b; e += kBigThreads) {
        const int m = m0 + e / rows_b;
        const int n = n0 + e % rows_b;
        const int64_t idx = (int64_t)m * N + n;
        acc_s v = 0;
        for (int zz = 0; zz < g.nsplit; ++zz)
            v += __hip_atomic_load(&part[zz * slice + idx], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int zz = 0; zz < g.nsplit; ++zz)
            __hip_atomic_store(&part[zz * slice + idx], (acc_s)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        store1(idx, out_value(v, m, n), (int)v);
    }
    if (t == 0) __hip_atomic_store(&g.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace qlin
