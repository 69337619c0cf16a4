/*
 * qlin_oracle.h -- plain, slow CPU reference for the quantized skinny linear
 * layer.  TEST INFRASTRUCTURE ONLY: the parity tests, the smoke check and the
 * benchmark's CPU-baseline leg call it; the GPU library never includes,
 * links or calls it, and it shares no code with the GPU library.
 *
 * What it computes follows "Building a High-Performance and Portable vLLM
 * Linear Backend with Helion":
 *   - section "Scope": the three 8-bit formats
 *       FP8_Dynamic  fp8 activations scaled per token, weights per channel,
 *       W8A8_INT8    int8 activations scaled per token, weights per channel,
 *       Block_FP8    fp8, one activation scale per 1x128 K-group of a token,
 *                    one weight scale per 128x128 block;
 *   - section "Kernel Implementation": out[M,N] = a[M,K] @ b[K,N] with a
 *     float32 accumulator, every schedule (Standard, Split-K, Swap-AB)
 *     computing the same product.
 * The pages leave the number formats, rounding and scale rules open; the
 * readings used here are: OCP E4M3FN fp8 (max 448), symmetric int8 in
 * [-127, 127], scale = amax / qmax as one fp32 division (0 when amax is 0),
 * codes = round-to-nearest-even of the fp32 quotient x / scale with
 * saturation, int8 products summed exactly in integers, fp8 products summed
 * exactly in fp64, the dequantized result formed in fp64.
 *
 * All functions return 0 on success and a negative value on bad arguments or
 * non-finite inputs.  Arrays are dense row-major, caller-owned host memory.
 */
#ifndef QLIN_ORACLE_H
#define QLIN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_FP8_DYNAMIC = 0, ORC_W8A8_INT8 = 1, ORC_BLOCK_FP8 = 2 };

/* fp8 E4M3FN code -> exact value (NaN codes 0x7F/0xFF give NaN). */
double orc_e4m3_decode(uint8_t code);
/* fp32 -> E4M3FN: clamp to [-448, 448], round to nearest (ties to even
 * mantissa), subnormals kept, sign kept (-tiny -> 0x80). -1 if not finite. */
int orc_e4m3_encode(float v, uint8_t *code);
/* Element-wise encode; returns the number of non-finite inputs (their code
 * is left 0xFF). */
int64_t orc_e4m3_encode_array(const float *v, uint8_t *out, int64_t n);

/* Activation quantization.  x: bf16 bit patterns [M][K].
 *   FP8_DYNAMIC / W8A8_INT8: s[M]      (one scale per token)
 *   BLOCK_FP8:               s[M][K/128] (one scale per 1x128 group)
 * q: [M][K] codes (int8 two's complement or e4m3). */
int orc_quant_act(int fmt, int M, int K, const uint16_t *x, uint8_t *q, float *s);

/* Weight quantization.  w: fp32 [N][K].
 *   FP8_DYNAMIC / W8A8_INT8: s[N]                 (one scale per channel)
 *   BLOCK_FP8:               s[N/128][K/128]      (one per 128x128 block) */
int orc_quant_weight(int fmt, int N, int K, const float *w, uint8_t *q, float *s);

/* Exact accumulators.  int8: acc[M][N] = sum_k qa*qw (int32 result, the sum
 * is checked to fit).  fp8: acc[M][N] = sum_k dec(qa)*dec(qw) in fp64 (exact
 * for K < 171196).  fp8 grouped: accg[M][N][K/128], one exact sum per group. */
int orc_acc_int8(int M, int N, int K, const uint8_t *qa, const uint8_t *qw, int32_t *acc);
int orc_acc_fp8(int M, int N, int K, const uint8_t *qa, const uint8_t *qw, double *acc);
int orc_acc_fp8_groups(int M, int N, int K, const uint8_t *qa, const uint8_t *qw, double *accg);

/* Dequantized result in fp64, ref[M][N]:
 *   per-channel formats: acc * sa[m] * sw[n]
 *   BLOCK_FP8:           sum over groups g (ascending) of
 *                        accg * sa[m][g] * sw[n/128][g]
 * acc_i32 (optional, int8 only) receives the int32 accumulators. */
int orc_gemm(int fmt, int M, int N, int K, const uint8_t *qa, const float *sa,
             const uint8_t *qw, const float *sw, double *ref, int32_t *acc_i32);

/* Same result for selected outputs only: ref[i] = ref(ms[i], ns[i]). */
int orc_gemm_sampled(int fmt, int M, int N, int K, const uint8_t *qa, const float *sa,
                     const uint8_t *qw, const float *sw, int64_t count, const int32_t *ms,
                     const int32_t *ns, double *ref, int32_t *acc_i32);

/* Whole linear layer: quantize x, then orc_gemm.  qa/sa receive the codes. */
int orc_linear(int fmt, int M, int N, int K, const uint16_t *x, const uint8_t *qw,
               const float *sw, uint8_t *qa, float *sa, double *ref, int32_t *acc_i32);

/* Round fp64 values to bfloat16 bit patterns (nearest, ties to even). */
void orc_round_bf16(const double *v, uint16_t *out, int64_t n);

/* Threads the parallel loops use (OpenMP), for reporting. */
int orc_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
