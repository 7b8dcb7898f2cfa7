/* Per-channel W8A8 int8 matmul on MI355X (gfx950).
 *
 * The scheme of "Experiment - int8 W8A8 path (the practical default)"
 * (Hypothesis, Implementation): int8 weights with one F32 scale per output
 * channel, int8 activations with one F32 scale per row, an int32 product and
 * the dequantization d[m][n] = aScale[m] * bScale[n] * C[m][n], multiplied
 * left to right.  The quantizers follow that page's arithmetic exactly:
 *   weights, per output channel n of w[OC][K] (done once, offline):
 *     mx = max(1e-9, max_k |w|); s = mx / 127; q = lrintf(w / s) (ties to
 *     even) clamped to [-127, 127];
 *   activations, per row m of x[M][K]:
 *     mx = max(1e-9, max_k |x|); aScale = mx / 127; inv = 127 / mx;
 *     v = x * inv; q = (int)(v + copysign(0.5, v)) (the sum rounded to F32,
 *     then truncated) clamped to [-127, 127].
 * Weights are stored wq[OC][K] (K contiguous, like the I2_S and I8_S
 * weights); the page transposes them for its NPU, which changes no value.
 * The contraction is the int8-MFMA tile kernel of the I8_S path with an F32
 * epilogue (an activation-resident kernel from 128 rows); at one to four
 * rows the whole op is one launch that quantizes and runs an int8 GEMV.
 *
 * Conventions as in i2s.h: device pointers, a hipStream_t or NULL, host-side
 * validation, no synchronization or allocation, I2S_* status codes.
 */
#ifndef W8A8_H
#define W8A8_H

#include <stddef.h>
#include <stdint.h>

#include "i2s.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Workspace of w8a8_mul_mat: the quantized activations q[M][K] then the M
 * row scales, each part 256-byte aligned (0 for a negative size). */
size_t w8a8_act_workspace_bytes(int64_t M, int64_t K);

/* Per-channel weight quantization: F32 w[OC][K] -> int8 wq[OC][K] and F32
 * wscale[OC].  One workgroup per channel.  Errors: I2S_EINVAL (null pointer,
 * negative size), I2S_ERANGE (OC*K >= 2^31), I2S_EHIP. */
int w8a8_quantize_weight(const float *w, int64_t OC, int64_t K,
                         int8_t *wq, float *wscale, void *stream);

/* Per-row activation quantization: F32 x[M][K] -> int8 q[M][K] and F32
 * ascale[M].  One workgroup per row.  Errors as w8a8_quantize_weight. */
int w8a8_quantize_act(const float *x, int64_t M, int64_t K,
                      int8_t *q, float *ascale, void *stream);

/* The contraction on quantized operands: y[M][OC] (F32) with
 * y[m][n] = aScale[m] * wscale[n] * (float)C[m][n]; dot_out (NULL or int32
 * [M][OC]) receives C.  K % 16 == 0 and K > 0; wq, aq, y and dot_out 16-byte
 * aligned, the scales 4-byte aligned; OC*K and M*K below 2^31 - 2^16, M*OC
 * below 2^29 - 2^14.  variant 0 = automatic, else an MFMA tile configuration
 * 2..i8s_variants() of the I8_S contraction, or 10: the activation-resident
 * kernel (64 activation rows in LDS, the int8 weights streamed; needs
 * K % 64 == 0 and K <= 2544).  Variant 11 quantizes F32 rows itself and is
 * refused here.  Errors: I2S_EINVAL, I2S_EALIGN (K), I2S_ERANGE, I2S_EKERNEL
 * (variant, or variant 10 with K it does not take), I2S_EHIP. */
int w8a8_matmul(const int8_t *wq, const float *wscale, int64_t OC, int64_t K,
                const int8_t *aq, const float *ascale, int64_t M,
                float *y, int32_t *dot_out, int variant, void *stream);

/* The whole op on F32 activations x[M][K] (16-byte aligned): quantize the
 * rows into `workspace` (>= w8a8_act_workspace_bytes(M, K), 256-byte
 * aligned, overwritten: the codes q[M][K], then at the next multiple of 256
 * bytes the scales, as w8a8_quantize_act writes them), then w8a8_matmul.
 * For 1 <= M <= 4 and K <= 9216 the automatic choice is variant 11, which
 * does both in one launch (every workgroup quantizes the rows itself, with
 * the same operations, then runs an int8 GEMV over its weight rows); the
 * results, and what the workspace holds afterwards, are those of the two
 * launches bit for bit.  Errors as above plus I2S_EWORKSPACE, and
 * I2S_EKERNEL for variant 11 outside 1 <= M <= 4, K <= 9216. */
int w8a8_mul_mat(const int8_t *wq, const float *wscale, int64_t OC, int64_t K,
                 const float *x, int64_t M, void *workspace, size_t workspace_bytes,
                 float *y, void *stream);

/* The same with dot_out and the tile variant. */
int w8a8_mul_mat_ex(const int8_t *wq, const float *wscale, int64_t OC, int64_t K,
                    const float *x, int64_t M, void *workspace, size_t workspace_bytes,
                    float *y, int32_t *dot_out, int variant, void *stream);

/* The variant the automatic choice of w8a8_mul_mat takes for this shape:
 * 11 (the fused decode launch) for 1 <= M <= 4 and K <= 9216 (K % 16 == 0),
 * else the contraction's choice. */
int w8a8_mul_mat_variant(int64_t OC, int64_t K, int64_t M);

/* The largest valid variant number (variant 1 and variants beyond it are
 * refused; w8a8_matmul also refuses 11). */
int w8a8_variants(void);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_H */
