// qlin_kernels.hip -- gfx950 (CDNA4) activation and weight quantization
// kernels of the quantized skinny linear layer, and the kernel launchers
// (the GEMM variants themselves live in qlin_gemm_<format>.hip).
//
// Formats: "Building a High-Performance and Portable vLLM Linear Backend
// with Helion", section "Scope" (FP8_Dynamic, W8A8_INT8, Block_FP8 scale
// granularities).
//
// Data layout (all row-major): activations x bf16 [M][ldx], codes xq [M][K],
// weights wq [N][K] (K contiguous, as a torch Linear weight), output y [M][N].
#include "qlin_gemm.h"

namespace qlin {

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
    const float y = recip_scale(s);
    if (threadIdx.x == 0) xs[m] = s;
    if constexpr (CPT > 0) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int c = threadIdx.x + j * kQuantThreads;
            if (c < nch) *reinterpret_cast<uint2 *>(qrow + c * 8) = quant8<FMT>(v[j], s, y);
        }
    } else {
        for (int c = threadIdx.x; c < nch; c += kQuantThreads)
            *reinterpret_cast<uint2 *>(qrow + c * 8) =
                quant8<FMT>(*reinterpret_cast<const uint4 *>(row + c * 8), s, y);
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
    const float amax = row16_max(absmax8(v));
    const float s = amax == 0.0f ? 0.0f : amax / 448.0f;
    if (!live) return;
    if (j == 0) xs[(int64_t)m * G + g] = s;
    *reinterpret_cast<uint2 *>(xq + (int64_t)m * K + g * kGroup + j * 8) = quant8<FMT_BLOCK>(v, s, recip_scale(s));
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

bool gemm_variant_exists(int fmt, int tile_m, int nr, int xc) {
    switch (fmt) {
    case FMT_FP8: return gemm_pick_fp8(false, tile_m, nr, xc) != nullptr;
    case FMT_I8: return gemm_pick_i8(false, tile_m, nr, xc) != nullptr;
    case FMT_BLOCK: return gemm_pick_block(false, tile_m, nr, xc) != nullptr;
    }
    return false;
}

hipError_t launch_gemm(int fmt, bool swap, int tile_m, int nr, int xc, const GemmLaunch &g,
                       size_t lds_bytes, hipStream_t s) {
    gemm_fn f = nullptr;
    switch (fmt) {
    case FMT_FP8: f = gemm_pick_fp8(swap, tile_m, nr, xc); break;
    case FMT_I8: f = gemm_pick_i8(swap, tile_m, nr, xc); break;
    case FMT_BLOCK: f = gemm_pick_block(swap, tile_m, nr, xc); break;
    }
    if (!f) return hipErrorInvalidValue;
    if (tile_m >= 64) {
        // large-M kernel: one-dimensional grid in its XCD-aware tile order
        // (N tiles padded to a multiple of 8), static LDS
        const unsigned n8 = (unsigned)((g.n_tiles + 7) & ~7);
        hipLaunchKernelGGL(f, dim3(n8 * g.m_tiles * g.nsplit), dim3(256), 0, s, g);
        return hipGetLastError();
    }
    const dim3 grid(g.n_tiles, g.m_tiles, g.nsplit);
    const dim3 block(64 * g.nw * g.kw);
    hipLaunchKernelGGL(f, grid, block, lds_bytes, s, g);
    return hipGetLastError();
}

}  // namespace qlin

