/* I8_S per-tensor int8 type and its fused matmul on MI355X (gfx950).
 *
 * I8_S ("ggml: additive INT8/ternary types, fused CPU ops, and kernels for
 * VibeASR (1/2)", Two new types): a tensor of n int8 values stored as its n
 * payload bytes in row-major order, then one F32 scale in band: the
 * multiplier amax/127 (dequantize by multiplying), little-endian, in the four
 * bytes right after the payload, followed by 28 zero bytes -- a 32-byte slot,
 * i8s_bytes(n) = n + 32 bytes in all.  Carrying the scale in band makes every
 * tensor self-describing; the encoder requantizes between every stage.
 *
 * mul_mat_add / mul_mat_add_relu (same page, Five fused INT8 ops): I8_S x
 * I8_S -> I8_S with the bias added and the output requantized in the
 * epilogue; the relu form applies ReLU before requantizing.  For weights
 * w[OC][IC] (output channel o is row o) and activations x[N][IC]:
 *     acc[n][o] = sum_k w[o][k] * x[n][k]          int32, exact
 *     f[n][o]   = (float)acc * (ws * xs)           ws * xs formed first
 *     f[n][o]   = f[n][o] + bias[o]                one F32 add, if bias given
 *     f[n][o]   = max(f[n][o], 0)                  relu form only
 * and the output is the I8_S quantization of the whole f[N][OC] tensor:
 * amax = max|f| floored at 1e-5, s = amax/127, q = f/s rounded half away
 * from zero, clamped to [-127, 127] -- one scale for the tensor ("VibeASR in
 * audio.cpp", Architecture / Encoder: one scale per tensor, the 1e-5 floor).
 *
 * Conventions (as i2s.h): device pointers; `stream` is a hipStream_t or NULL
 * for the null stream; calls validate on the host, then enqueue kernels and
 * return without synchronizing; nothing allocates.  Status codes are the
 * I2S_* codes of i2s.h, explained by i2s_strerror.
 */
#ifndef I8S_H
#define I8S_H

#include <stddef.h>
#include <stdint.h>

#include "i2s.h"

#ifdef __cplusplus
extern "C" {
#endif

#define I8S_SCALE_SLOT 32
#define I8S_MAX_IC 133143 /* 127 * 127 * IC < 2^31: int32 accumulators stay exact */

/* Bytes of an I8_S tensor of n values: n + 32 (0 for n < 0). */
size_t i8s_bytes(int64_t n);

/* Workspace for i8s_quantize and i8s_mul_mat_add(_relu, _ex): per-workgroup
 * partial maxima of the requantization (at most 1024 floats).  Constant;
 * 256-byte aligned device memory owned by the caller, overwritten. */
size_t i8s_workspace_bytes(void);

/* F32 tensor x[n] (finite, 16-byte aligned) -> I8_S tensor `out`
 * (i8s_bytes(n) bytes, 16-byte aligned; payload and scale slot written):
 * amax over all n values floored at 1e-5, s = amax/127, q = x/s rounded half
 * away from zero, clamped to +-127.  Two launches (partial maxima, then
 * quantize).  n = 0 writes the scale slot only (s = 1e-5/127); x may then
 * be NULL.
 * Errors: I2S_EINVAL (null or misaligned pointer, n < 0), I2S_EWORKSPACE,
 * I2S_ERANGE (n >= 2^31), I2S_EHIP. */
int i8s_quantize(const float *x, int64_t n, uint8_t *out,
                 void *workspace, size_t workspace_bytes, void *stream);

/* I8_S tensor t of n values (16-byte aligned) -> F32 y[n] = q * s
 * (16-byte aligned; may be NULL for n = 0).  Errors: I2S_EINVAL, I2S_ERANGE,
 * I2S_EHIP. */
int i8s_dequantize(const uint8_t *t, int64_t n, float *y, void *stream);

/* mul_mat_add: w = I8_S [OC][IC], x = I8_S [N][IC], bias = NULL or F32
 * [OC] (4-byte aligned), out = I8_S [N][OC] (i8s_bytes(N*OC) bytes, payload
 * and scale slot overwritten; must not overlap the inputs).  w, x and out are
 * 16-byte aligned.  0 <= IC <= I8S_MAX_IC; OC*IC and N*IC below 2^31 - 2^16,
 * N*OC below 2^29 - 2^14.
 * Two passes of one int8-MFMA contraction (IC a multiple of 16; other IC take
 * a plain per-output kernel): the first reduces max|f| per workgroup into the
 * workspace, the second requantizes with the tensor's scale -- the F32 values
 * are never written to memory.  Errors: I2S_EINVAL, I2S_EWORKSPACE,
 * I2S_ERANGE, I2S_EHIP; nothing is launched on an error. */
int i8s_mul_mat_add(const uint8_t *w, int64_t OC, int64_t IC,
                    const uint8_t *x, int64_t N, const float *bias, uint8_t *out,
                    void *workspace, size_t workspace_bytes, void *stream);

/* mul_mat_add_relu: the same with ReLU applied before requantizing. */
int i8s_mul_mat_add_relu(const uint8_t *w, int64_t OC, int64_t IC,
                         const uint8_t *x, int64_t N, const float *bias, uint8_t *out,
                         void *workspace, size_t workspace_bytes, void *stream);

/* Either op with the contraction variant forced (0 = automatic, 1 = plain
 * per-output kernel for any IC, 2.. = MFMA tile configurations, which need
 * IC % 16 == 0; see i8s_variants) and an optional int32 dot_out[N][OC]
 * (4-byte aligned) receiving acc.  Errors as above, plus I2S_EKERNEL for an
 * unknown variant or an MFMA variant with IC % 16 != 0. */
int i8s_mul_mat_add_ex(const uint8_t *w, int64_t OC, int64_t IC,
                       const uint8_t *x, int64_t N, const float *bias, int relu,
                       uint8_t *out, int32_t *dot_out, int variant,
                       void *workspace, size_t workspace_bytes, void *stream);

/* The variant the automatic choice takes for this shape. */
int i8s_mul_mat_add_variant(int64_t OC, int64_t IC, int64_t N);

/* Number of variants (the largest valid variant number). */
int i8s_variants(void);

#ifdef __cplusplus
}
#endif

#endif /* I8S_H */
