// qlin_kernels.hip -- gfx950 (CDNA4) kernels of the quantized skinny linear
// layer: activation and weight quantization, and the skinny GEMM with its
// Standard / Split-K / Swap-AB schedules.
//
// Formats and product: "Building a High-Performance and Portable vLLM Linear
// Backend with Helion", section "Scope" (FP8_Dynamic, W8A8_INT8, Block_FP8
// scale granularities) and section "Kernel Implementation" (one contraction,
// float32 accumulator, split_k / swap_ab as schedule choices, Split-K
// partials added into a zeroed output).
//
// Data layout (all row-major): activations x bf16 [M][ldx], codes xq [M][K],
// weights wq [N][K] (K contiguous, as a torch Linear weight), output y [M][N].
#include <hip/hip_runtime.h>

#include "qlin_internal.h"

namespace qlin {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

enum { FMT_FP8 = QLIN_FP8_DYNAMIC, FMT_I8 = QLIN_W8A8_INT8, FMT_BLOCK = QLIN_BLOCK_FP8 };

// ------------------------------------------------------------ conversions

// fp32 -> fp8 E4M3FN code.  Magnitudes at or above 448 saturate to 448
// (0x7E); normal results round the 23-bit mantissa to 3 bits, nearest with
// ties to even, carrying into the exponent; below 2^-6 the value is a whole
// multiple of 2^-9, so |v| * 512 (exact) is rounded to an integer 0..8 (8 is
// the code of 2^-6).  The sign bit is copied, so -0 and tiny negatives give
// 0x80.  Inputs are finite.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a >= 0x43E00000u) return sign | 0x7Eu;            // |v| >= 448
    if (a >= 0x3C800000u) {                               // |v| >= 2^-6
        const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
        return sign | (r - (120u << 3));                   // rebias 127 -> 7
    }
    const float t = __uint_as_float(a) * 512.0f;
    return sign | (uint32_t)__builtin_rintf(t);
}

// code of one value given its row/group scale (scale 0: the run was zero)
template <int FMT>
__device__ __forceinline__ uint32_t quant_code(float x, float s) {
    if (s == 0.0f) return 0u;
    const float t = x / s;   // IEEE division, correctly rounded
    if (FMT == FMT_I8) {
        float r = __builtin_rintf(t);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        return (uint32_t)(int32_t)r & 0xFFu;
    }
    return e4m3_code(t);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, nearest with ties to even (finite inputs)
__device__ __forceinline__ uint32_t bf16_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int FMT>
__device__ __forceinline__ float qmax_of() { return FMT == FMT_I8 ? 127.0f : 448.0f; }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// --------------------------------------------------- activation quantization

// bf16 x 8 (one 16-byte chunk) -> max |value|
__device__ __forceinline__ float absmax8(uint4 v) {
    return fmaxf(fmaxf(fmaxf(fabsf(bf16_lo(v.x)), fabsf(bf16_hi(v.x))),
                       fmaxf(fabsf(bf16_lo(v.y)), fabsf(bf16_hi(v.y)))),
                 fmaxf(fmaxf(fabsf(bf16_lo(v.z)), fabsf(bf16_hi(v.z))),
                       fmaxf(fabsf(bf16_lo(v.w)), fabsf(bf16_hi(v.w)))));
}

// bf16 x 8 -> 8 codes packed little-endian into two words
template <int FMT>
__device__ __forceinline__ uint2 quant8(uint4 v, float s) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        lo |= quant_code<FMT>(bf16_lo(w[j]), s) << (16 * j);
        lo |= quant_code<FMT>(bf16_hi(w[j]), s) << (16 * j + 8);
        hi |= quant_code<FMT>(bf16_lo(w[j + 2]), s) << (16 * j);
        hi |= quant_code<FMT>(bf16_hi(w[j + 2]), s) << (16 * j + 8);
    }
    return make_uint2(lo, hi);
}

constexpr int kQuantThreads = 512;

// One workgroup per token.  With CPT > 0 every thread keeps its (at most
// CPT) 16-byte chunks of the row in registers: one read of the row, the
// row's amax by a wave reduction and one across waves, then the codes.
// CPT == 0 is the fallback for very long rows: the row is read twice.
template <int FMT, int CPT>
__global__ __launch_bounds__(kQuantThreads) void quant_token_kernel(const uint16_t *__restrict__ x,
                                                                    int64_t ldx, int K,
                                                                    uint8_t *__restrict__ xq,
                                                                    float *__restrict__ xs) {
    __shared__ float red[kQuantThreads / 64];
    const int m = blockIdx.x;
    const uint16_t *row = x + (int64_t)m * ldx;
    uint8_t *qrow = xq + (int64_t)m * K;
    const int nch = K >> 3;
    float amax = 0.0f;
    uint4 v[CPT > 0 ? CPT : 1];
    if constexpr (CPT > 0) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int c = threadIdx.x + j * kQuantThreads;
            v[j] = c < nch ? *reinterpret_cast<const uint4 *>(row + c * 8) : make_uint4(0, 0, 0, 0);
            amax = fmaxf(amax, absmax8(v[j]));
        }
    } else {
        for (int c = threadIdx.x; c < nch; c += kQuantThreads)
            amax = fmaxf(amax, absmax8(*reinterpret_cast<const uint4 *>(row + c * 8)));
    }
    amax = wave_max(amax);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = red[0];
#pragma unroll
    for (int w = 1; w < kQuantThreads / 64; ++w) amax = fmaxf(amax, red[w]);
    const float s = amax == 0.0f ? 0.0f : amax / qmax_of<FMT>();
    if (threadIdx.x == 0) xs[m] = s;
    if constexpr (CPT > 0) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int c = threadIdx.x + j * kQuantThreads;
            if (c < nch) *reinterpret_cast<uint2 *>(qrow + c * 8) = quant8<FMT>(v[j], s);
        }
    } else {
        for (int c = threadIdx.x; c < nch; c += kQuantThreads)
            *reinterpret_cast<uint2 *>(qrow + c * 8) =
                quant8<FMT>(*reinterpret_cast<const uint4 *>(row + c * 8), s);
    }
}

// Per (token, 128-wide K group): 16 lanes own one group, 8 values each; a
// 256-thread workgroup covers 16 groups.
__global__ __launch_bounds__(256) void quant_group_kernel(const uint16_t *__restrict__ x,
                                                          int64_t ldx, int M, int K,
                                                          uint8_t *__restrict__ xq,
                                                          float *__restrict__ xs) {
    const int G = K / kGroup;
    const int gi = blockIdx.x * 16 + (threadIdx.x >> 4);
    const int j = threadIdx.x & 15;
    const bool live = gi < M * G;
    const int m = live ? gi / G : 0;
    const int g = live ? gi - m * G : 0;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (live) v = *reinterpret_cast<const uint4 *>(x + (int64_t)m * ldx + g * kGroup + j * 8);
    float amax = absmax8(v);
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
    const float s = amax == 0.0f ? 0.0f : amax / 448.0f;
    if (!live) return;
    if (j == 0) xs[(int64_t)m * G + g] = s;
    *reinterpret_cast<uint2 *>(xq + (int64_t)m * K + g * kGroup + j * 8) = quant8<FMT_BLOCK>(v, s);
}

// ------------------------------------------------------- weight quantization

__device__ __forceinline__ float block_max256(float v, float *red) {
    v = wave_max(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ uint32_t pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    return a | (b << 8) | (c << 16) | (d << 24);
}

// One workgroup per output channel n (row of W), 4 floats per step.
template <int FMT>
__global__ __launch_bounds__(256) void quant_channel_kernel(const float *__restrict__ w, int K,
                                                            uint8_t *__restrict__ wq,
                                                            float *__restrict__ ws) {
    __shared__ float red[4];
    const int n = blockIdx.x;
    const float *row = w + (int64_t)n * K;
    float amax = 0.0f;
    for (int c = threadIdx.x; c < K / 4; c += 256) {
        const float4 v = *reinterpret_cast<const float4 *>(row + c * 4);
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    amax = block_max256(amax, red);
    const float s = amax == 0.0f ? 0.0f : amax / qmax_of<FMT>();
    if (threadIdx.x == 0) ws[n] = s;
    for (int c = threadIdx.x; c < K / 4; c += 256) {
        const float4 v = *reinterpret_cast<const float4 *>(row + c * 4);
        *reinterpret_cast<uint32_t *>(wq + (int64_t)n * K + c * 4) =
            pack4(quant_code<FMT>(v.x, s), quant_code<FMT>(v.y, s), quant_code<FMT>(v.z, s),
                  quant_code<FMT>(v.w, s));
    }
}

// One workgroup per 128x128 block: thread t covers 4 floats of each of the
// block's rows 2*(t/64)... in turn (row r, columns 4*(t%32)..+4 for r = t/32 + 8*i).
__global__ __launch_bounds__(256) void quant_block_weight_kernel(const float *__restrict__ w,
                                                                 int K, uint8_t *__restrict__ wq,
                                                                 float *__restrict__ ws) {
    __shared__ float red[4];
    const int kb = blockIdx.x, nb = blockIdx.y;
    const int col = (threadIdx.x & 31) * 4;
    const int r0 = threadIdx.x >> 5;
    const float *base = w + (int64_t)nb * kGroup * K + kb * kGroup + col;
    float amax = 0.0f;
    for (int r = r0; r < kGroup; r += 8) {
        const float4 v = *reinterpret_cast<const float4 *>(base + (int64_t)r * K);
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    amax = block_max256(amax, red);
    const float s = amax == 0.0f ? 0.0f : amax / 448.0f;
    if (threadIdx.x == 0) ws[(int64_t)nb * (K / kGroup) + kb] = s;
    uint8_t *qbase = wq + (int64_t)nb * kGroup * K + kb * kGroup + col;
    for (int r = r0; r < kGroup; r += 8) {
        const float4 v = *reinterpret_cast<const float4 *>(base + (int64_t)r * K);
        *reinterpret_cast<uint32_t *>(qbase + (int64_t)r * K) =
            pack4(quant_code<FMT_BLOCK>(v.x, s), quant_code<FMT_BLOCK>(v.y, s),
                  quant_code<FMT_BLOCK>(v.z, s), quant_code<FMT_BLOCK>(v.w, s));
    }
}

// ------------------------------------------------------------------- GEMM
//
// Work decomposition.  A workgroup owns a tile of up to TM = 16*MT tokens by
// TN = 16*NR*nw output channels and a range of 128-wide K blocks (all of K,
// or one Split-K partition).  Its waves form an nw x kw grid: a wave owns NR
// sub-tiles of 16 channels and every kw-th K block of the range, so the kw
// waves of a column stream neighbouring K blocks of the same weight rows at
// the same time; their partial sums are added through LDS at the end.
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
// (a ring of PF register slots), and its first PF blocks are requested
// before the activations are staged, so the two latencies overlap.
//
// Activations.  The workgroup's token rows for its K range are staged once
// in LDS, only the rows that exist (R = min(TM, M - m0)), laid out as
// [K block][half][quarter][row][16 bytes]: the 16 lanes of a quarter read 16
// consecutive 16-byte chunks, so the two ds_read_b128 per block are free of
// bank conflicts.  Lanes whose row is past R use zeros.  When R x (K range)
// does not fit the LDS budget the range is processed in phases.
//
// Standard: A = activations (tokens are the MFMA rows), B = weights.  The
// 16x16 result lane l holds column l % 16 = channel and rows 4(l/16)+i =
// tokens.  Swap-AB: A = weights, B = activations, so the result is the
// transpose: lane l holds token l % 16 and channels 4(l/16)+i, which makes
// the output stores 4 channels wide and needs one activation scale per lane.

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

// 32 bytes of one weight row starting at byte k of the row (p points there);
// 16-byte halves at or beyond K read as zero
__device__ __forceinline__ v8i load_w(const uint8_t *p, int k, int K, bool full) {
    if (full) {
        const uint4 lo = *reinterpret_cast<const uint4 *>(p);
        const uint4 hi = *reinterpret_cast<const uint4 *>(p + 16);
        return join(lo, hi);
    }
    uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
    if (k < K) lo = *reinterpret_cast<const uint4 *>(p);
    if (k + 16 < K) hi = *reinterpret_cast<const uint4 *>(p + 16);
    return join(lo, hi);
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

// Activation staging of the fused path: 16 consecutive bf16 values of one
// token row become 16 codes (one uint4).  For the block format the 8 lanes
// that share a 128-wide group (lanes 8j .. 8j+7 of a wave) first reduce the
// group's amax.  Returns the codes; *gscale receives the group scale.
template <int FMT>
__device__ __forceinline__ uint4 quant16(const uint16_t *src, float row_scale, float *gscale) {
    const uint4 a = *reinterpret_cast<const uint4 *>(src);
    const uint4 b = *reinterpret_cast<const uint4 *>(src + 8);
    float s = row_scale;
    if constexpr (FMT == FMT_BLOCK) {
        float amax = fmaxf(absmax8(a), absmax8(b));
#pragma unroll
        for (int o = 4; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 8));
        s = amax == 0.0f ? 0.0f : amax / 448.0f;
        *gscale = s;
    }
    const uint2 lo = quant8<FMT>(a, s);
    const uint2 hi = quant8<FMT>(b, s);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

template <int FMT, bool SWAP, int MT, int NR, int PF, bool FUSE>
__global__ __launch_bounds__(64 * kMaxWaves) void gemm_kernel(GemmLaunch g) {
    typedef typename AccT<FMT>::type acc_t;
    typedef typename AccT<FMT>::scalar acc_s;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ int s_last;
    __shared__ float s_rowscale[16 * MT];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nthreads = blockDim.x;
    const int nwaves = nthreads >> 6;
    const int nw = wave % g.nw, kw = wave / g.nw;
    const int TN = 16 * NR * g.nw;
    const int n_tile0 = blockIdx.x * TN;
    const int m0 = blockIdx.y * 16 * MT;
    const int kb_begin = blockIdx.z * g.kb_per_split;
    const int kb_end = min(g.nkb, kb_begin + g.kb_per_split);
    const int M = g.M, N = g.N, K = g.K;
    const int r16 = lane & 15, quarter = lane >> 4;
    const int G = (K + kGroup - 1) / kGroup;
    const int R = min(16 * MT, M - m0);   // token rows that exist in this tile
    // fused path: the first column of workgroups also stores the codes and
    // scales it produces (every workgroup of a row of tiles produces the same)
    const bool writer = FUSE && blockIdx.x == 0;

    int nsub[NR];
    const uint8_t *wrow[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        nsub[r] = n_tile0 + (nw * NR + r) * 16;
        const int n = min(nsub[r] + r16, N - 1);
        wrow[r] = g.wq + (int64_t)n * K + quarter * 32;
    }

    acc_t acc[NR][MT];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[r][mt] = acc_t{0, 0, 0, 0};

    // Per-channel formats: the epilogue's channel scales are requested now,
    // so their latency hides behind the weight stream (token scales too,
    // unless the fused path computes them below).  Swap-AB lanes need one
    // token scale and 4 channel scales per sub-tile, Standard lanes 4 token
    // scales and one channel scale.
    float pre_sa[MT][SWAP ? 1 : 4], pre_sw[NR][SWAP ? 4 : 1];
    auto token_of = [&](int mt, int i) { return SWAP ? m0 + mt * 16 + r16 : m0 + mt * 16 + 4 * quarter + i; };
    if constexpr (FMT != FMT_BLOCK) {
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int i = 0; i < (SWAP ? 4 : 1); ++i) {
                const int n = SWAP ? nsub[r] + 4 * quarter + i : nsub[r] + r16;
                pre_sw[r][i] = g.wsc[min(n, N - 1)];
            }
        if constexpr (!FUSE) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < (SWAP ? 1 : 4); ++i) pre_sa[mt][i] = g.xs[min(token_of(mt, i), M - 1)];
        }
    }

    // issue the loads of absolute K block kb into a register slot (the block
    // format also fetches each sub-tile's 128x128 weight-block scale)
    auto issue = [&](v8i(&slot)[NR], float(&sws)[NR], int kb) {
        const int k = kb * kGroup;
        const bool full = k + kGroup <= K;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            slot[r] = load_w(wrow[r] + k, k + quarter * 32, K, full);
            if constexpr (FMT == FMT_BLOCK)
                sws[r] = g.wsc[(int64_t)(min(nsub[r], N - 1) / kGroup) * G + kb];
        }
    };

    v8i wbuf[PF][NR];
    float wsbuf[PF][NR];
    const int kstep = g.kw;

    for (int pb0 = kb_begin; pb0 < kb_end; pb0 += g.phase_blocks) {
        const int nblk = min(kb_end - pb0, g.phase_blocks);
        // weight requests for the first PF blocks of this phase go out first
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int b = kw + p * kstep;
            if (b < nblk) issue(wbuf[p], wsbuf[p], pb0 + b);
        }
        if (pb0 != kb_begin) __syncthreads();
        float *s_scale = reinterpret_cast<float *>(smem + (size_t)g.phase_blocks * kGroup * R);

        if constexpr (FUSE && FMT != FMT_BLOCK) {
            // per-token scales need the whole row: one wave per token row
            // finds its amax over all of K (the rows are small and shared by
            // every workgroup, so they come from L2)
            if (pb0 == kb_begin) {
                for (int row = wave; row < R; row += nwaves) {
                    const uint16_t *xr = g.x + (int64_t)(m0 + row) * g.ldx;
                    float amax = 0.0f;
                    for (int c = lane; c < K / 8; c += 64)
                        amax = fmaxf(amax, absmax8(*reinterpret_cast<const uint4 *>(xr + c * 8)));
                    amax = wave_max(amax);
                    if (lane == 0) {
                        const float sc = amax == 0.0f ? 0.0f : amax / qmax_of<FMT>();
                        s_rowscale[row] = sc;
                        if (writer && blockIdx.z == 0) g.xs_out[m0 + row] = sc;
                    }
                }
                __syncthreads();
            }
        }

        // stage the activation codes of this phase: [block][half][quarter][row][16B]
        const int items = R * nblk * 8;
        for (int it = threadIdx.x; it < items; it += nthreads) {
            const int c = it & 7;
            const int rest = it >> 3;
            const int b = rest % nblk;
            const int row = rest / nblk;
            const int k = (pb0 + b) * kGroup + c * 16;
            uint4 v = make_uint4(0, 0, 0, 0);
            if constexpr (FUSE) {
                float gs = 0.0f;
                if (k < K) {
                    v = quant16<FMT>(g.x + (int64_t)(m0 + row) * g.ldx + k,
                                     FMT == FMT_BLOCK ? 0.0f : s_rowscale[row], &gs);
                    if (writer) *reinterpret_cast<uint4 *>(g.xq_out + (int64_t)(m0 + row) * K + k) = v;
                }
                if constexpr (FMT == FMT_BLOCK) {
                    if (c == 0) {
                        s_scale[b * R + row] = gs;
                        if (writer) g.xs_out[(int64_t)(m0 + row) * G + pb0 + b] = gs;
                    }
                }
            } else {
                if (k < K) v = *reinterpret_cast<const uint4 *>(g.xq + (int64_t)(m0 + row) * K + k);
            }
            *reinterpret_cast<uint4 *>(smem + (((b * 2 + (c & 1)) * 4 + (c >> 1)) * R + row) * 16) = v;
        }
        if constexpr (FMT == FMT_BLOCK && !FUSE) {
            for (int it = threadIdx.x; it < nblk * R; it += nthreads) {
                const int row = it % R, b = it / R;
                s_scale[b * R + row] = g.xs[(int64_t)(m0 + row) * G + pb0 + b];
            }
        }
        __syncthreads();

        bool more = kw < nblk;
        for (int j = 0; more; j += PF) {
#pragma unroll
            for (int p = 0; p < PF; ++p) {
                const int b = kw + (j + p) * kstep;
                if (b >= nblk) {
                    more = false;
                    break;
                }
                // activation fragments of this block (zeros past row R)
                v8i xf[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const int row = mt * 16 + r16;
                    uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
                    if (row < R) {
                        const uint8_t *base = smem + (((b * 2) * 4 + quarter) * R + row) * 16;
                        lo = *reinterpret_cast<const uint4 *>(base);
                        hi = *reinterpret_cast<const uint4 *>(base + 4 * R * 16);
                    }
                    xf[mt] = join(lo, hi);
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
                                const float c = (row < R ? sc[row] : 0.0f) * swv;
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
                const int bn = b + PF * kstep;
                if (bn < nblk) issue(wbuf[p], wsbuf[p], pb0 + bn);
            }
        }
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
            for (int j = 1; j < g.kw; ++j)
#pragma unroll
                for (int r = 0; r < NR; ++r)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        acc[r][mt] += red[((((j - 1) * g.nw + nw) * NR + r) * MT + mt) * 64 + lane];
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
                    if (m >= M) continue;
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
                        if (m >= M) continue;
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
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                if (nsub[r] >= N) continue;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m = token_of(mt, i);
                        const int n = SWAP ? nsub[r] + 4 * quarter + i : nsub[r] + r16;
                        if (m >= M) continue;
                        const int64_t idx = (int64_t)m * N + n;
                        long long v;
                        if constexpr (FMT == FMT_I8) v = (long long)acc[r][mt][i];
                        else v = (long long)(acc[r][mt][i] * 262144.0f);
                        const unsigned long long old = __hip_atomic_fetch_add(
                            &ws64[idx], (unsigned long long)(v + (long long)kUnit), __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_AGENT);
                        const unsigned long long before = (old + kHalf) >> 52;
                        if (before != (unsigned long long)(g.nsplit - 1)) continue;
                        const long long total = (long long)(old - before * kUnit) + v;
                        float t;
                        if constexpr (FMT == FMT_I8) t = (float)total;
                        else t = (float)((double)total * (1.0 / 262144.0));
                        store1(idx, scaled(t, r, mt, i), (int)total);
                        __hip_atomic_store(&ws64[idx], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
    const int64_t slice = (int64_t)M * N;
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
                    if (m < M)
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
    const int tn = min(TN, N - n_tile0);
    for (int e = threadIdx.x; e < R * tn; e += nthreads) {
        const int m = m0 + e / tn;
        const int n = n_tile0 + e % tn;
        const int64_t idx = (int64_t)m * N + n;
        acc_s v = 0;
        for (int z = 0; z < g.nsplit; ++z)
            v += __hip_atomic_load(&part[z * slice + idx], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int z = 0; z < g.nsplit; ++z)   // leave the workspace zero
            __hip_atomic_store(&part[z * slice + idx], (acc_s)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        float o;
        if constexpr (FMT == FMT_BLOCK) o = v;
        else if constexpr (FUSE) o = ((float)v * s_rowscale[m - m0]) * g.wsc[n];
        else o = ((float)v * g.xs[m]) * g.wsc[n];
        store1(idx, o, (int)v);
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(&g.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// --------------------------------------------------------------- launchers

hipError_t launch_quant_act(int fmt, int M, int K, const void *x, int64_t ldx, void *xq,
                            float *xs, hipStream_t s) {
    const uint16_t *xb = static_cast<const uint16_t *>(x);
    uint8_t *q = static_cast<uint8_t *>(xq);
    if (fmt == FMT_BLOCK) {
        const int groups = M * (K / kGroup);
        hipLaunchKernelGGL(quant_group_kernel, dim3((groups + 15) / 16), dim3(256), 0, s, xb, ldx,
                           M, K, q, xs);
    } else {
        const int nch = K / 8;
        const int cpt = (nch + kQuantThreads - 1) / kQuantThreads;
#define QLIN_QT(F, C) \
    hipLaunchKernelGGL((quant_token_kernel<F, C>), dim3(M), dim3(kQuantThreads), 0, s, xb, ldx, K, q, xs)
#define QLIN_QT_ALL(F)                  \
    if (cpt <= 1) QLIN_QT(F, 1);        \
    else if (cpt <= 2) QLIN_QT(F, 2);   \
    else if (cpt <= 4) QLIN_QT(F, 4);   \
    else if (cpt <= 8) QLIN_QT(F, 8);   \
    else QLIN_QT(F, 0);
        if (fmt == FMT_I8) {
            QLIN_QT_ALL(FMT_I8)
        } else {
            QLIN_QT_ALL(FMT_FP8)
        }
#undef QLIN_QT_ALL
#undef QLIN_QT
    }
    return hipGetLastError();
}

hipError_t launch_quant_weight(int fmt, int N, int K, const float *w, void *wq, float *ws,
                               hipStream_t s) {
    uint8_t *q = static_cast<uint8_t *>(wq);
    if (fmt == FMT_BLOCK) {
        hipLaunchKernelGGL(quant_block_weight_kernel, dim3(K / kGroup, N / kGroup), dim3(256), 0, s,
                           w, K, q, ws);
    } else if (fmt == FMT_I8) {
        hipLaunchKernelGGL(quant_channel_kernel<FMT_I8>, dim3(N), dim3(256), 0, s, w, K, q, ws);
    } else {
        hipLaunchKernelGGL(quant_channel_kernel<FMT_FP8>, dim3(N), dim3(256), 0, s, w, K, q, ws);
    }
    return hipGetLastError();
}

typedef void (*gemm_fn)(GemmLaunch);

// prefetch depth: 8 blocks of 16 weight rows in flight per wave (4 for NR = 4)
#define QLIN_PF(NR_) (NR_ >= 4 ? 2 : 8 / NR_)

template <int FMT, bool SWAP>
static gemm_fn pick(int tile_m, int nr, bool fuse) {
#define QLIN_PICK(MT_, NR_, FUSE_)                                 \
    if (tile_m == 16 * MT_ && nr == NR_ && fuse == FUSE_)          \
        return gemm_kernel<FMT, SWAP, MT_, NR_, QLIN_PF(NR_), FUSE_>;
    QLIN_PICK(1, 1, false) QLIN_PICK(1, 2, false) QLIN_PICK(1, 4, false)
    QLIN_PICK(2, 1, false) QLIN_PICK(2, 2, false) QLIN_PICK(2, 4, false)
    QLIN_PICK(1, 1, true) QLIN_PICK(1, 2, true) QLIN_PICK(1, 4, true)
#undef QLIN_PICK
    return nullptr;
}

static gemm_fn pick_any(int fmt, bool swap, int tile_m, int nr, bool fuse) {
    switch (fmt) {
    case FMT_FP8: return swap ? pick<FMT_FP8, true>(tile_m, nr, fuse) : pick<FMT_FP8, false>(tile_m, nr, fuse);
    case FMT_I8: return swap ? pick<FMT_I8, true>(tile_m, nr, fuse) : pick<FMT_I8, false>(tile_m, nr, fuse);
    case FMT_BLOCK:
        return swap ? pick<FMT_BLOCK, true>(tile_m, nr, fuse) : pick<FMT_BLOCK, false>(tile_m, nr, fuse);
    }
    return nullptr;
}

bool gemm_variant_exists(int fmt, int tile_m, int nr, bool fuse) {
    return pick_any(fmt, false, tile_m, nr, fuse) != nullptr;
}

hipError_t launch_gemm(int fmt, bool swap, int tile_m, int nr, bool fuse, const GemmLaunch &g,
                       size_t lds_bytes, hipStream_t s) {
    gemm_fn f = pick_any(fmt, swap, tile_m, nr, fuse);
    if (!f) return hipErrorInvalidValue;
    const dim3 grid(g.n_tiles, g.m_tiles, g.nsplit);
    const dim3 block(64 * g.nw * g.kw);
    hipLaunchKernelGGL(f, grid, block, lds_bytes, s, g);
    return hipGetLastError();
}

}  // namespace qlin
