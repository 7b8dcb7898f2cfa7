/*
 * CPU oracle for the I2_S ternary-weight x int8-activation matmul (W2A8),
 * for the I8_S per-tensor int8 type with its fused mul_mat_add(_relu), and
 * for the per-channel W8A8 matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * definition that the GPU library is checked against.  Only the tests, the
 * smoke check and the benchmark's CPU-baseline leg may load it; the product
 * path never calls it, and it shares no source with the GPU library.
 *
 * Every step is scalar C in the order the pages state it.  Floating point is
 * IEEE binary32 (the precision the pages fix for activations and scales),
 * compiled without fast-math and without FP contraction, so each float
 * operation written here is exactly one correctly rounded operation.
 *
 * Pages cited:
 *   [P1] "ggml: additive INT8/ternary types, fused CPU ops, and kernels for
 *        VibeASR (1/2)"
 *   [P2] "ggml-cpu: ternary I2_S matmul kernel (VibeASR, 3/4)"
 *   [P3] "VibeASR in audio.cpp"
 *   [P4] "Experiment - int8 W8A8 path (the practical default)"
 *
 * Parity pins (tests/test_oracle_pins.py): hand-decoded pack bytes, the
 * rounding vector, the headroom closed form, degenerate scales, sign
 * invariants, exact-rational quantization and Python-integer brute force with
 * signed weights; for the bias add, hand-derived binary32 values that tell
 * one add after the rounded epilogue from a fused multiply-add.  I8_S
 * (tests/test_oracle_i8s_pins.py): hand-worked mul_mat_add(_relu) bytes and
 * scale bits, an exact-rational model, numpy's integer matmul at full scale,
 * the per-row vectors on one-row tensors, round-trip bounds, equivariances,
 * and agreement with the I2_S op on ternary weights.  Per-channel W8A8
 * (tests/test_oracle_w8a8_pins.py): the hand-worked rounding row, exact-
 * rational models of both quantizers (near ties included) and of the
 * left-to-right dequantization, numpy's integer matmul, the 1e-9 start of the
 * running maximum.  The 28 padding bytes of
 * the in-band scale slot are "parity unpinned": nothing on the pages reads
 * them.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_GROUP_VALUES 128 /* values per packed group [P1 Two new types] */
#define ORACLE_GROUP_BYTES 32   /* bytes per packed group                    */
#define ORACLE_SCALE_SLOT 32    /* padded in-band F32 scale slot             */

/* Payload bytes (2 bits per weight) plus the padded in-band scale slot. */
size_t oracle_packed_bytes(int64_t rows, int64_t K)
{
    return (size_t)(rows * K / 4) + ORACLE_SCALE_SLOT;
}

/* Ternary value -> unsigned code: -1 -> 0, 0 -> 1, +1 -> 2
 * [P2 Arithmetic: the codes {0,1,2} stand for {-1,0,+1}].  Any other value
 * maps by its sign. */
static unsigned oracle_code(int8_t w)
{
    if (w > 0) return 2u;
    if (w < 0) return 0u;
    return 1u;
}

/* Where value number f of the flat tensor lives: a group holds 128 values in
 * 32 bytes, split into four slices of 32; the value at offset j of its group
 * goes to byte j mod 32 of the group, in the bit pair of slice j / 32, the
 * first slice in the top two bits and the last in the bottom two
 * [P1 Kernels; P2 Kernels; P3 Architecture/Decoder: packed over the whole
 * flat tensor]. */
static void oracle_locate(int64_t f, int64_t *byte, int *shift)
{
    int64_t group = f / ORACLE_GROUP_VALUES;
    int64_t j = f % ORACLE_GROUP_VALUES;   /* position inside the group      */
    int64_t slice = j / 32;                /* which 32-value slice (0..3)    */
    int64_t gp = j % 32;                   /* byte inside the group          */
    *byte = group * ORACLE_GROUP_BYTES + gp;
    *shift = 6 - 2 * (int)slice;
}

/* Pack a ternary matrix w[rows][K] and its weight scale ws into I2_S bytes:
 * the 2-bit codes of the whole flat tensor, then ws as a little-endian F32
 * followed by 28 zero bytes [P1 Two new types: scale carried in band, after
 * the payload].  Returns 0, or -1 if K is not a multiple of 128. */
int oracle_pack(const int8_t *w, float ws, int64_t rows, int64_t K, uint8_t *out)
{
    if (K <= 0 || K % ORACLE_GROUP_VALUES != 0 || rows < 0) return -1;
    int64_t total = rows * K;
    memset(out, 0, oracle_packed_bytes(rows, K));
    for (int64_t f = 0; f < total; ++f) {
        int64_t byte;
        int shift;
        oracle_locate(f, &byte, &shift);
        out[byte] |= (uint8_t)(oracle_code(w[f]) << shift);
    }
    memcpy(out + total / 4, &ws, sizeof(float));
    return 0;
}

/* Read the in-band weight scale that follows the payload. */
float oracle_weight_scale(const uint8_t *packed, int64_t rows, int64_t K)
{
    float ws;
    memcpy(&ws, packed + rows * K / 4, sizeof(float));
    return ws;
}

/* Per-row activation quantization.  For each row n of x[N][K]:
 *   amax = max_k |x|, floored at 1e-5 [P3 Architecture/Encoder];
 *   s = amax / 127, stored as a multiplier [P1 Two new types; P2 Arithmetic];
 *   q = x / s rounded half away from zero, clamped to [-127, 127];
 *   row_sum = sum_k q, kept for the epilogue [P2 Arithmetic].
 * The whole row is needed for amax, so a row is never split
 * [P2 Kernels, threading]. */
void oracle_quantize_act(const float *x, int64_t N, int64_t K,
                         int8_t *q, float *act_scale, int32_t *row_sum)
{
    for (int64_t n = 0; n < N; ++n) {
        const float *xr = x + n * K;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(xr[k]);
            if (a > amax) amax = a;
        }
        if (amax < 1e-5f) amax = 1e-5f;
        float s = amax / 127.0f;
        int32_t sum = 0;
        for (int64_t k = 0; k < K; ++k) {
            float v = xr[k] / s;
            float r = roundf(v); /* C roundf: halfway cases away from zero */
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            int8_t qi = (int8_t)r;
            q[n * K + k] = qi;
            sum += qi;
        }
        act_scale[n] = s;
        row_sum[n] = sum;
    }
}

/* Integer contraction: dot[n][o] = sum_k code[o][k] * q[n][k] in int32, with
 * the codes decoded from the packed bytes one value at a time
 * [P1 Arithmetic is exact where it can be; P2 Arithmetic: the kernel returns
 * sum(code*q)].  `packed` may start at any row boundary: groups never
 * straddle rows when K is a multiple of 128. */
void oracle_dot(const uint8_t *packed, int64_t rows, int64_t K,
                const int8_t *q, int64_t N, int32_t *dot)
{
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t o = 0; o < rows; ++o) {
            int32_t acc = 0;
            for (int64_t k = 0; k < K; ++k) {
                int64_t byte;
                int shift;
                oracle_locate(o * K + k, &byte, &shift);
                int32_t code = (packed[byte] >> shift) & 3;
                acc += code * (int32_t)q[n * K + k];
            }
            dot[n * rows + o] = acc;
        }
    }
}

/* Epilogue: y[n][o] = (float)(dot - row_sum) * (weight_scale * act_scale)
 * [P2 Arithmetic].  The bracketed product is formed first, then one multiply. */
void oracle_epilogue(const int32_t *dot, const int32_t *row_sum, const float *act_scale,
                     float ws, int64_t N, int64_t rows, float *y)
{
    for (int64_t n = 0; n < N; ++n) {
        float t = ws * act_scale[n];
        for (int64_t o = 0; o < rows; ++o) {
            float d = (float)(dot[n * rows + o] - row_sum[n]);
            y[n * rows + o] = d * t;
        }
    }
}

/* The whole op: F32 x[N][K] times the packed I2_S weight (scale read from
 * band), F32 y[N][rows] out [P2 Interface].  dot_out, if not NULL, receives
 * the raw int32 sum(code*q).  Returns 0, -1 on a bad K, -2 on allocation
 * failure. */
int oracle_mul_mat(const uint8_t *packed, int64_t rows, int64_t K,
                   const float *x, int64_t N, float *y, int32_t *dot_out)
{
    if (K <= 0 || K % ORACLE_GROUP_VALUES != 0 || rows < 0 || N < 0) return -1;
    if (rows == 0 || N == 0) return 0;
    int8_t *q = (int8_t *)malloc((size_t)(N * K));
    float *s = (float *)malloc((size_t)N * sizeof(float));
    int32_t *rs = (int32_t *)malloc((size_t)N * sizeof(int32_t));
    int32_t *dot = (int32_t *)malloc((size_t)(N * rows) * sizeof(int32_t));
    if (!q || !s || !rs || !dot) {
        free(q); free(s); free(rs); free(dot);
        return -2;
    }
    oracle_quantize_act(x, N, K, q, s, rs);
    oracle_dot(packed, rows, K, q, N, dot);
    oracle_epilogue(dot, rs, s, oracle_weight_scale(packed, rows, K), N, rows, y);
    if (dot_out) memcpy(dot_out, dot, (size_t)(N * rows) * sizeof(int32_t));
    free(q); free(s); free(rs); free(dot);
    return 0;
}

/* Bias of a projection: y[n][o] = y[n][o] + bias[o], one F32 add per output
 * after the epilogue.  The decoder's q/k/v projections carry F32 biases
 * [P3 Architecture/Decoder: norms and the q/k/v biases are F32 tensors]; the
 * plain reading is the usual separate F32 tensor add on the matmul's F32
 * output, so the epilogue value is rounded before the bias joins it. */
void oracle_add_bias(float *y, const float *bias, int64_t N, int64_t rows)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t o = 0; o < rows; ++o)
            y[n * rows + o] = y[n * rows + o] + bias[o];
}

/* ------------------------------------------------------------------------
 * I8_S: per-tensor int8 [P1 Two new types: nelements int8 bytes, then one
 * padded F32 scale, stored as the multiplier amax/127].  The scale occupies
 * the four bytes right after the payload, followed by 28 zero bytes (the same
 * 32-byte slot as I2_S; the padding is parity unpinned).
 */

size_t oracle_i8s_bytes(int64_t n)
{
    return (size_t)n + ORACLE_SCALE_SLOT;
}

float oracle_i8s_scale(const uint8_t *t, int64_t n)
{
    float s;
    memcpy(&s, t + n, sizeof(float));
    return s;
}

/* F32 tensor -> I8_S: one amax over the whole tensor, floored at 1e-5
 * [P3 Architecture/Encoder: the waveform's single scale], s = amax / 127,
 * q = x / s rounded half away from zero, clamped to [-127, 127]; the same
 * steps as the per-row activation quantization with the row taken to be the
 * whole tensor. */
void oracle_i8s_quantize(const float *x, int64_t n, uint8_t *out)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    if (amax < 1e-5f) amax = 1e-5f;
    float s = amax / 127.0f;
    for (int64_t i = 0; i < n; ++i) {
        float r = roundf(x[i] / s);
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        out[i] = (uint8_t)(int8_t)r;
    }
    memset(out + n, 0, ORACLE_SCALE_SLOT);
    memcpy(out + n, &s, sizeof(float));
}

/* I8_S -> F32: y = q * s (dequantize by multiplying [P1 Two new types]). */
void oracle_i8s_dequantize(const uint8_t *t, int64_t n, float *y)
{
    float s = oracle_i8s_scale(t, n);
    for (int64_t i = 0; i < n; ++i) y[i] = (float)(int8_t)t[i] * s;
}

/* mul_mat_add (relu = 0) and mul_mat_add_relu (relu = 1)
 * [P1 Five fused INT8 ops: I8_S x I8_S -> I8_S, the bias added and the
 * output requantized in the epilogue; the relu form applies ReLU before
 * requantizing].  w is I8_S [OC][IC] (output channel o is row o), x is I8_S
 * [N][IC]; per output:
 *   acc[n][o] = sum_k w[o][k] * x[n][k]                (int32, exact)
 *   f[n][o]   = (float)acc * (ws * xs)                 (ws * xs first)
 *   f[n][o]   = f[n][o] + bias[o]                      (if bias != NULL)
 *   f[n][o]   = f[n][o] > 0 ? f[n][o] : 0              (relu form)
 * then out = the I8_S quantization of the whole f[N][OC] tensor.  dot and f
 * (either may be NULL) receive acc and the pre-quantization values.  Returns
 * 0, or -2 on allocation failure. */
int oracle_i8s_mul_mat_add(const uint8_t *w, int64_t OC, int64_t IC,
                           const uint8_t *x, int64_t N, const float *bias, int relu,
                           uint8_t *out, int32_t *dot, float *f)
{
    float ws = oracle_i8s_scale(w, OC * IC);
    float xs = oracle_i8s_scale(x, N * IC);
    float t = ws * xs;
    float *v = (float *)malloc((size_t)(N * OC > 0 ? N * OC : 1) * sizeof(float));
    if (!v) return -2;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t o = 0; o < OC; ++o) {
            int32_t acc = 0;
            for (int64_t k = 0; k < IC; ++k)
                acc += (int32_t)(int8_t)w[o * IC + k] * (int32_t)(int8_t)x[n * IC + k];
            float r = (float)acc * t;
            if (bias) r = r + bias[o];
            if (relu && !(r > 0.0f)) r = 0.0f;
            v[n * OC + o] = r;
            if (dot) dot[n * OC + o] = acc;
        }
    }
    if (f) memcpy(f, v, (size_t)(N * OC) * sizeof(float));
    oracle_i8s_quantize(v, N * OC, out);
    free(v);
    return 0;
}

/* ------------------------------------------------------------------------
 * Per-channel W8A8 ["Experiment - int8 W8A8 path (the practical default)",
 * Hypothesis and Implementation]: int8 weights with one F32 scale per output
 * channel, int8 activations with one F32 scale per row, an int32 product,
 * and a dequantization that multiplies the activation row's scale, the
 * channel's scale and the converted int32 product, in that order.  Its
 * rounding differs from the I2_S activation quantizer in three places: the
 * maximum is never below 1e-9 (instead of a 1e-5 floor), weight codes round
 * ties to even, and activation codes multiply by the reciprocal of the
 * scale, step half a unit away from zero and drop the fraction.  Weights are kept as w[n][k] (K contiguous);
 * the page transposes them for its NPU, which changes no value.
 */

/* The largest magnitude of v[0..K), but never below the page's starting
 * value 1e-9 (so an all-zero row still has a finite, nonzero scale). */
static float w8a8_max_mag(const float *v, int64_t K)
{
    float m = 0.0f;
    for (int64_t k = 0; k < K; ++k)
        m = fmaxf(m, fabsf(v[k]));
    return m < 1e-9f ? 1e-9f : m;
}

static int8_t w8a8_clamp127(float r)
{
    return (int8_t)(r > 127.0f ? 127 : (r < -127.0f ? -127 : (int)r));
}

/* Weight code: the F32 quotient w / s rounded to the nearest integer, ties
 * to the even neighbour (the default rounding mode, as lrintf uses). */
static int8_t w8a8_weight_code(float w, float s)
{
    return w8a8_clamp127(rintf(w / s));
}

/* Activation code: the F32 product v = x * inv, moved half a unit away from
 * zero (that sum is itself rounded to F32), then the fraction dropped.  For
 * v = -0 the sign makes no difference: both +-0.5 truncate to 0. */
static int8_t w8a8_act_code(float x, float inv)
{
    float v = x * inv;
    float moved = v < 0.0f ? v - 0.5f : v + 0.5f;
    return w8a8_clamp127(truncf(moved));
}

/* Per output channel n of w[OC][K]: scale[n] = max / 127 and each weight's
 * code from w8a8_weight_code. */
void oracle_w8a8_quantize_weight(const float *w, int64_t OC, int64_t K, int8_t *q, float *scale)
{
    for (int64_t n = 0; n < OC; ++n) {
        const float *row = w + n * K;
        scale[n] = w8a8_max_mag(row, K) / 127.0f;
        for (int64_t k = 0; k < K; ++k)
            q[n * K + k] = w8a8_weight_code(row[k], scale[n]);
    }
}

/* Per activation row m of x[M][K]: scale[m] = max / 127, and the codes use
 * the reciprocal 127 / max (not the division by the stored scale). */
void oracle_w8a8_quantize_act(const float *x, int64_t M, int64_t K, int8_t *q, float *scale)
{
    for (int64_t m = 0; m < M; ++m) {
        const float *row = x + m * K;
        float mx = w8a8_max_mag(row, K);
        float inv = 127.0f / mx;
        scale[m] = mx / 127.0f;
        for (int64_t k = 0; k < K; ++k)
            q[m * K + k] = w8a8_act_code(row[k], inv);
    }
}

static int32_t w8a8_int_dot(const int8_t *u, const int8_t *v, int64_t K)
{
    int32_t s = 0;
    for (int64_t k = 0; k < K; ++k)
        s += (int32_t)u[k] * (int32_t)v[k];
    return s;
}

/* C[m][n] = the int32 dot of activation row m and weight row n; the
 * dequantized value multiplies the two scales first (activation scale on
 * the left) and then the converted C. */
void oracle_w8a8_matmul(const int8_t *a, const float *ascale, int64_t M,
                        const int8_t *w, const float *wscale, int64_t OC, int64_t K,
                        float *d, int32_t *c)
{
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < OC; ++n) {
            int32_t cv = w8a8_int_dot(a + m * K, w + n * K, K);
            float t = ascale[m] * wscale[n];
            if (c) c[m * OC + n] = cv;
            d[m * OC + n] = t * (float)cv;
        }
    }
}

/* The whole op on F32 activations x[M][K] and pre-quantized weights. */
int oracle_w8a8_mul_mat(const int8_t *w, const float *wscale, int64_t OC, int64_t K,
                        const float *x, int64_t M, float *d, int32_t *c)
{
    int8_t *a = (int8_t *)malloc((size_t)(M * K > 0 ? M * K : 1));
    float *as = (float *)malloc((size_t)(M > 0 ? M : 1) * sizeof(float));
    if (!a || !as) {
        free(a); free(as);
        return -2;
    }
    oracle_w8a8_quantize_act(x, M, K, a, as);
    oracle_w8a8_matmul(a, as, M, w, wscale, OC, K, d, c);
    free(a); free(as);
    return 0;
}
