/*
 * CPU oracle for the I2_S ternary-weight x int8-activation matmul (W2A8).
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
 *
 * Parity pins (tests/test_oracle_pins.py): hand-decoded pack bytes, the
 * rounding vector, the headroom closed form, degenerate scales, sign
 * invariants, exact-rational quantization and Python-integer brute force with
 * signed weights; for the bias add, hand-derived binary32 values that tell
 * one add after the rounded epilogue from a fused multiply-add.  The 28 padding bytes of the in-band scale slot are
 * "parity unpinned": nothing on the pages reads them.
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
 * 32 bytes; byte gp of a group holds the group-relative positions gp, 32+gp,
 * 64+gp and 96+gp in the bit pairs at shifts 6, 4, 2 and 0
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
