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
#include <mutex>

#include "qlin_gemm.h"

namespace qlin {

// One token row per TPR threads (TPR / 64 waves), max(1, 256 / TPR) rows per
// workgroup.  With CPT > 0 every thread keeps its (at most CPT) 16-byte
// chunks of the row in registers: one read of the row, the row's amax by a
// wave reduction (and, for more than one wave per row, one across the row's
// waves through LDS), then the codes.  CPT == 0 is the fallback for rows
// longer than CPT chunks per thread allow: the row is read twice.  One wave
// per row needs no LDS and no barrier; more waves per row cut each thread's
// share of the row (fewer chunks to convert one after another).
template <int FMT, int TPR, int CPT>
__global__ __launch_bounds__(TPR >= 256 ? TPR : 256) void quant_token_kernel(const uint16_t *__restrict__ x,
                                                                            int64_t ldx, int M, int K,
                                                                            uint8_t *__restrict__ xq,
                                                                            float *__restrict__ xs) {
    constexpr int RPW = TPR >= 256 ? 1 : 256 / TPR;   // rows per workgroup
    constexpr int WPR = TPR / 64;                      // waves per row
    __shared__ float red[RPW * WPR];
    const int t = threadIdx.x % TPR, rsub = threadIdx.x / TPR;
    const int m = blockIdx.x * RPW + rsub;
    const bool live = m < M;
    const uint16_t *row = x + (int64_t)(live ? m : 0) * ldx;
    uint8_t *qrow = xq + (int64_t)(live ? m : 0) * K;
    const int nch = live ? K >> 3 : 0;
    float amax = 0.0f;
    uint4 v[CPT > 0 ? CPT : 1];
    if constexpr (CPT > 0) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int c = t + j * TPR;
            v[j] = c < nch ? *reinterpret_cast<const uint4 *>(row + c * 8) : make_uint4(0, 0, 0, 0);
            amax = fmaxf(amax, absmax8(v[j]));
        }
    } else {
        for (int c = t; c < nch; c += TPR)
            amax = fmaxf(amax, absmax8(*reinterpret_cast<const uint4 *>(row + c * 8)));
    }
    amax = wave_max(amax);
    if constexpr (WPR > 1) {
        if ((t & 63) == 0) red[rsub * WPR + (t >> 6)] = amax;
        __syncthreads();
        amax = red[rsub * WPR];
#pragma unroll
        for (int w = 1; w < WPR; ++w) amax = fmaxf(amax, red[rsub * WPR + w]);
    }
    if (!live) return;
    const float s = amax == 0.0f ? 0.0f : amax / qmax_of<FMT>();
    const float y = recip_scale(s);
    if (t == 0) xs[m] = s;
    if constexpr (CPT > 0) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int c = t + j * TPR;
            if (c < nch) *reinterpret_cast<uint2 *>(qrow + c * 8) = quant8<FMT>(v[j], s, y);
        }
    } else {
        for (int c = t; c < nch; c += TPR)
            *reinterpret_cast<uint2 *>(qrow + c * 8) =
                quant8<FMT>(*reinterpret_cast<const uint4 *>(row + c * 8), s, y);
    }
}

// Per (token, 128-wide K group): 16 lanes own one group, 8 values each; a
// workgroup of 16 GPW threads covers GPW groups.
template <int GPW>
__global__ __launch_bounds__(16 * GPW) void quant_group_kernel(const uint16_t *__restrict__ x, int64_t ldx,
                                                               int M, int K, uint8_t *__restrict__ xq,
                                                               float *__restrict__ xs) {
    const int G = K / kGroup;
    const int gi = blockIdx.x * GPW + (threadIdx.x >> 4);
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
// ----------------------------------------------------------- weight packing

// Row-major codes [batch][N][K] -> the packed layout: for 16-row group s,
// K block kb, half h and lane l, the 16 bytes at byte
// 1024 ((s * nkb + kb) * 2 + h) + 16 l hold row 16 s + l % 16, bytes
// 128 kb + 32 (l / 16) + 16 h .. + 15 (zeros past K).  That is the GEMM
// kernels' per-lane fragment of a 16-row x 128-K block, so a wave's weight
// load reads 1 KiB of consecutive bytes.  One thread per 16-byte chunk:
// coalesced stores, 16-byte gathers.
__global__ __launch_bounds__(256) void pack_weight_kernel(const uint8_t *__restrict__ w, int N, int K,
                                                          int nkb, uint8_t *__restrict__ out) {
    const int64_t per = (int64_t)(N / kPackRows) * nkb * (kPackBlock / 16);   // chunks per matrix
    const uint8_t *src = w + (int64_t)blockIdx.y * N * K;
    uint8_t *dst = out + (int64_t)blockIdx.y * per * 16;
    for (int64_t c = blockIdx.x * (int64_t)256 + threadIdx.x; c < per; c += (int64_t)gridDim.x * 256) {
        const int t = (int)(c & 127);
        const int64_t blk = c >> 7;               // s * nkb + kb
        const int kb = (int)(blk % nkb);
        const int64_t row = (blk / nkb) * kPackRows + (t & 15);
        const int k0 = kb * kGroup + 32 * ((t & 63) >> 4) + 16 * (t >> 6);
        uint4 v = make_uint4(0, 0, 0, 0);
        if (k0 < K) v = *reinterpret_cast<const uint4 *>(src + row * K + k0);
        *reinterpret_cast<uint4 *>(dst + c * 16) = v;
    }
}

// --------------------------------------------------------------- launchers

hipError_t launch_pack_weight(int batch, int N, int K, const void *wq, void *out, hipStream_t s) {
    const int nkb = (K + kGroup - 1) / kGroup;
    const int64_t chunks = (int64_t)(N / kPackRows) * nkb * (kPackBlock / 16);
    const int64_t blocks = (chunks + 255) / 256;
    hipLaunchKernelGGL(pack_weight_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096), (unsigned)batch),
                       dim3(256), 0, s, static_cast<const uint8_t *>(wq), N, K, nkb, static_cast<uint8_t *>(out));
    return hipGetLastError();
}

// Threads per token row (per-token formats) or per workgroup (1x128
// groups) of the quantize kernels when the caller does not choose.
int quant_threads_rule(int fmt, int M, int K) {
    (void)M;
    (void)K;
    return fmt == FMT_BLOCK ? 256 : 512;
}

bool quant_threads_valid(int fmt, int threads) {
    if (fmt == FMT_BLOCK) return threads == 64 || threads == 256;
    return threads == 64 || threads == 128 || threads == 256 || threads == 512;
}

template <int F, int TPR>
static void launch_token(int M, int K, const uint16_t *xb, int64_t ldx, uint8_t *q, float *xs, hipStream_t s) {
    constexpr int RPW = TPR >= 256 ? 1 : 256 / TPR;
    const dim3 grid((M + RPW - 1) / RPW), block(TPR >= 256 ? TPR : 256);
    const int cpt = (K / 8 + TPR - 1) / TPR;
#define QLIN_QT(C) hipLaunchKernelGGL((quant_token_kernel<F, TPR, C>), grid, block, 0, s, xb, ldx, M, K, q, xs)
    if (cpt <= 1) QLIN_QT(1);
    else if (cpt <= 2) QLIN_QT(2);
    else if (cpt <= 4) QLIN_QT(4);
    else if (cpt <= 8) QLIN_QT(8);
    else if (cpt <= 16 && TPR <= 128) QLIN_QT(16);
    else QLIN_QT(0);
#undef QLIN_QT
}

template <int F>
static void launch_token_any(int threads, int M, int K, const uint16_t *xb, int64_t ldx, uint8_t *q, float *xs,
                             hipStream_t s) {
    switch (threads) {
    case 64: launch_token<F, 64>(M, K, xb, ldx, q, xs, s); break;
    case 128: launch_token<F, 128>(M, K, xb, ldx, q, xs, s); break;
    case 256: launch_token<F, 256>(M, K, xb, ldx, q, xs, s); break;
    default: launch_token<F, 512>(M, K, xb, ldx, q, xs, s); break;
    }
}

hipError_t launch_quant_act(int fmt, int M, int K, const void *x, int64_t ldx, void *xq,
                            float *xs, hipStream_t s, int threads) {
    const uint16_t *xb = static_cast<const uint16_t *>(x);
    uint8_t *q = static_cast<uint8_t *>(xq);
    if (threads == 0) threads = quant_threads_rule(fmt, M, K);
    if (fmt == FMT_BLOCK) {
        const int groups = M * (K / kGroup);
        if (threads == 64)
            hipLaunchKernelGGL(quant_group_kernel<4>, dim3((groups + 3) / 4), dim3(64), 0, s, xb, ldx, M, K, q, xs);
        else
            hipLaunchKernelGGL(quant_group_kernel<16>, dim3((groups + 15) / 16), dim3(256), 0, s, xb, ldx, M, K, q,
                               xs);
    } else if (fmt == FMT_I8) {
        launch_token_any<FMT_I8>(threads, M, K, xb, ldx, q, xs, s);
    } else {
        launch_token_any<FMT_FP8>(threads, M, K, xb, ldx, q, xs, s);
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

// ------------------------------------------------------ static scratch space

// The split-K workspace of qlin_linear_scratch: a file-scope device array
// that each GPU holds for the life of the process (every call on a GPU
// shares it).  In host code its name is only a stand-in for the symbol; the
// device address comes from hipGetSymbolAddress, once per device, and only
// that address is passed to kernels.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

struct ScratchSlot {
    std::once_flag once;
    hipError_t status = hipSuccess;
    void *ptr = nullptr;        // this device's address of `scratch`
    bool zeroed = false;        // a zero fill ran eagerly (outside capture)
};
ScratchSlot g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

__global__ __launch_bounds__(256) void zero_fill_kernel(uint4 *p, size_t n16) {
    for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
        p[i] = make_uint4(0, 0, 0, 0);
}

}  // namespace

// Device address of this device's scratch array, and makes sure it holds
// zeros before the first kernel that uses it: a fill kernel on `s` (not a
// memset node, which graph replays have been seen to mishandle).  A call
// made while `s` is being captured records the fill in the graph (so every
// replay starts from zeros) and leaves it to the next eager call to fill it
// once outside the graph.  After that the kernels keep it zero.
hipError_t static_scratch(hipStream_t s, void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    ScratchSlot &slot = g_scratch[dev];
    std::call_once(slot.once, [&slot]() {
        slot.status = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch));
        if (slot.status == hipSuccess && slot.ptr == nullptr) slot.status = hipErrorInvalidSymbol;
    });
    if (slot.status != hipSuccess) return slot.status;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!slot.zeroed) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        e = hipStreamIsCapturing(s, &cs);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(zero_fill_kernel, dim3(512), dim3(256), 0, s, static_cast<uint4 *>(slot.ptr),
                           kScratchBytes / 16);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (cs == hipStreamCaptureStatusNone) slot.zeroed = true;
    }
    *out = slot.ptr;
    return hipSuccess;
}

bool gemm_variant_exists(int fmt, bool swap, int tile_m, int nr, int xc) {
    switch (fmt) {
    case FMT_FP8: return gemm_pick_fp8(swap, tile_m, nr, xc, false) != nullptr;
    case FMT_I8: return gemm_pick_i8(swap, tile_m, nr, xc, false) != nullptr;
    case FMT_BLOCK: return gemm_pick_block(swap, tile_m, nr, xc, false) != nullptr;
    }
    return false;
}

hipError_t launch_gemm(int fmt, bool swap, int tile_m, int nr, int xc, const GemmLaunch &g,
                       size_t lds_bytes, hipStream_t s) {
    // the skinny kernel streams its weights with the non-temporal policy when
    // each weight tile is read by one token tile: one tile of tokens, or a
    // grouped launch (each expert's rows are normally one tile)
    const bool nt = g.group_off != nullptr || g.m_tiles == 1;
    gemm_fn f = nullptr;
    switch (fmt) {
    case FMT_FP8: f = gemm_pick_fp8(swap, tile_m, nr, xc, nt); break;
    case FMT_I8: f = gemm_pick_i8(swap, tile_m, nr, xc, nt); break;
    case FMT_BLOCK: f = gemm_pick_block(swap, tile_m, nr, xc, nt); break;
    }
    if (!f) return hipErrorInvalidValue;
    if (tile_m >= 64 && nr == 0) {
        // large-M kernel (nr 0; a 64-token tile with weight sub-tiles is the
        // skinny kernel's): one-dimensional grid in its XCD-aware tile order
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

