/*
 * i2s.h - C ABI of the gfx950 (MI355X) library for the I2_S ternary-weight x
 * int8-activation matmul (W2A8).
 *
 * The op, as the pages define it:
 *   "ggml-cpu: ternary I2_S matmul kernel (VibeASR, 3/4)", section Interface:
 *     a plain matmul of an I2_S weight (src0) with F32 activations (src1),
 *     giving F32 out;
 *   same page, section Arithmetic: the codes {0,1,2} stand for {-1,0,+1}; the
 *     kernel accumulates sum(code*q) in int32 and the epilogue computes
 *     dst = (float)(dot - row_sum) * (weight_scale * act_scale), with both
 *     scales multipliers (amax/127 for activations, the weight absmax for
 *     I2_S);
 *   "ggml: additive INT8/ternary types, fused CPU ops, and kernels for VibeASR
 *     (1/2)", section Two new types: I2_S holds 128 values per 32-byte group,
 *     then one padded F32 absmax in band, after the payload;
 *   same page, section Kernels: byte i of a group carries the codes of the
 *     group's positions i, i+32, i+64 and i+96, the first in the top bit pair
 *     (shift 6) and the last in the bottom one (shift 0);
 *   "VibeASR in audio.cpp", Architecture / Decoder: packed over the whole flat
 *     tensor; the kernel asserts K % 128 == 0;
 *   "VibeASR in audio.cpp", Architecture / Encoder: amax floored at 1e-5.
 * Activation rounding is half away from zero with a clamp to +-127.
 *
 * Conventions shared by every call:
 *   - Every data pointer is a DEVICE pointer (hipMalloc'd or a device tensor's
 *     storage) owned by the caller; the library never keeps, frees or
 *     allocates them.  Arrays are dense and row-major as stated per argument.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it and the call returns without synchronizing.
 *   - Arguments are checked on the host before anything is launched; a bad
 *     argument returns a nonzero status and launches nothing.  Faults inside
 *     a kernel surface at the caller's next synchronization on that stream.
 *   - N == 0 or rows == 0 is a successful no-op.
 *   - Calls are stateless and may be made from several host threads.
 *   - Results are bit-identical to the defining formulas above: integer steps
 *     are exact and the three F32 operations (x / s, ws * s, and the final
 *     multiply) are single IEEE round-to-nearest operations in a fixed order.
 */
#ifndef I2S_H
#define I2S_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define I2S_OK 0
#define I2S_EINVAL 1     /* null pointer where one is needed, or a negative size */
#define I2S_EALIGN 2     /* K is not a positive multiple of 128 */
#define I2S_EWORKSPACE 3 /* workspace NULL or smaller than i2s_act_workspace_bytes */
#define I2S_EHIP 4       /* the HIP runtime reported an error at launch */
#define I2S_ERANGE 5     /* a size beyond what this library addresses */
#define I2S_EKERNEL 6    /* i2s_mul_mat_ex/_ws: unknown kernel or variant, or
                            one that does not accept this N or K */
#define I2S_ESCRATCH 7   /* i2s_mul_mat_noalloc: the shape's workspace exceeds
                            I2S_NOALLOC_SCRATCH_BYTES */

/* Bytes of an I2_S tensor of `rows` x `K` weights: rows*K/4 bytes of 2-bit
 * codes, then a 32-byte slot whose first 4 bytes are the F32 weight scale
 * (little-endian) and whose other 28 bytes are zero.  0 if K is not a positive
 * multiple of 128 or rows < 0.
 * ("ggml: additive INT8/ternary types, ... (1/2)", Two new types.) */
size_t i2s_packed_bytes(int64_t rows, int64_t K);

/* Bytes of the activation workspace i2s_mul_mat needs for N rows of length K:
 * the int8 activations, then N F32 activation scales, then N int32 row sums
 * (the sidecar of "ggml-cpu: ternary I2_S matmul kernel (VibeASR, 3/4)",
 * Interface), then a second copy of the int8 activations in the skinny
 * MFMA kernel's operand order (ceil(N/16) * ceil(K/256) * 4096 bytes).  The
 * layout inside is private to the library.  0 if K is not a positive
 * multiple of 128 or N < 0. */
size_t i2s_act_workspace_bytes(int64_t N, int64_t K);

/* Pack ternary weights into I2_S.
 *   w            [rows][K] int8, values in {-1,0,+1}; any other value packs
 *                by its sign (code = sign(w) + 1).
 *   weight_scale F32 multiplier stored in band (the weight absmax; 0 allowed).
 *   packed       [i2s_packed_bytes(rows, K)] bytes, fully overwritten
 *                (payload, scale, and the 28 zero padding bytes).
 * Errors: I2S_EINVAL (null pointer, rows < 0), I2S_EALIGN, I2S_ERANGE,
 * I2S_EHIP.  ("ggml: additive INT8/ternary types, ... (1/2)", Two new types
 * and Kernels; "VibeASR in audio.cpp", Architecture / Decoder.) */
int i2s_pack(const int8_t *w, float weight_scale, int64_t rows, int64_t K,
             uint8_t *packed, void *stream);

/* Quantize F32 activation rows to int8, one scale and one int8 sum per row:
 *   amax = max_k |x[n][k]|, floored at 1e-5f;  act_scale[n] = amax / 127;
 *   q[n][k] = clamp(round_half_away(x[n][k] / act_scale[n]), -127, 127);
 *   row_sum[n] = sum_k q[n][k].
 *   x         [N][K] F32, finite values (NaN/Inf are not supported).
 *   q         [N][K] int8 (plain row-major order).
 *   act_scale [N] F32;  row_sum [N] int32.
 * Errors: I2S_EINVAL, I2S_EALIGN, I2S_ERANGE, I2S_EHIP.
 * ("ggml-cpu: ternary I2_S matmul kernel (VibeASR, 3/4)", Arithmetic and
 * Kernels/threading: a row is never split because its absmax is row-wide.) */
int i2s_quantize_act(const float *x, int64_t N, int64_t K,
                     int8_t *q, float *act_scale, int32_t *row_sum, void *stream);

/* The matmul: y[n][o] = (float)(dot[n][o] - row_sum[n]) * (ws * act_scale[n])
 * with dot[n][o] = sum_k code[o][k] * q[n][k] in int32 and ws read on the
 * device from the packed tensor's scale slot.  Quantizes x into `workspace`,
 * then runs the contraction with the epilogue fused: for N <= 3 (K <= 9216)
 * one fused quantize + v_dot4 GEMV launch; otherwise a weight-streaming v_dot4
 * GEMV for N = 1, a skinny int8-MFMA kernel up to N = 32 (N = 64 for at most
 * 4096 rows), an int8-MFMA GEMM above (i2s_mul_mat_kernel tells which).
 *   packed     I2_S tensor of rows x K (as written by i2s_pack).
 *   x          [N][K] F32 activations, finite.
 *   workspace  >= i2s_act_workspace_bytes(N, K) bytes, 256-byte aligned;
 *              overwritten.  Must not be shared by overlapping calls.
 *   y          [N][rows] F32 (rows contiguous), fully overwritten.
 *   dot_out    NULL, or [N][rows] int32 receiving sum(code*q).
 * Errors: I2S_EINVAL, I2S_EALIGN, I2S_EWORKSPACE, I2S_ERANGE, I2S_EHIP.
 * ("ggml-cpu: ternary I2_S matmul kernel (VibeASR, 3/4)", Interface,
 * Arithmetic, Kernels.) */
int i2s_mul_mat(const uint8_t *packed, int64_t rows, int64_t K,
                const float *x, int64_t N,
                void *workspace, size_t workspace_bytes,
                float *y, int32_t *dot_out, void *stream);

/* i2s_mul_mat with the contraction kernel chosen by the caller, for checking
 * that every launch geometry gives identical bits and for timing each kernel
 * on its own.  kernel: 0 = automatic (as i2s_mul_mat), 1 = GEMV (N <= 8),
 * 2 = MFMA GEMM (any N >= 1), 3 = fused quantize + GEMV in one launch
 * (N <= 4, K <= 9216; it does not use the workspace), 4 = skinny MFMA
 * (N <= 64).  variant: 0 =
 * automatic, else a 1-based index into the kernel's tile configurations
 * (i2s_kernel_variants).  Returns I2S_EKERNEL for an unknown pair or a kernel
 * that does not accept this N or K.  After any matmul call the workspace
 * contents are unspecified. */
int i2s_mul_mat_ex(const uint8_t *packed, int64_t rows, int64_t K,
                   const float *x, int64_t N,
                   void *workspace, size_t workspace_bytes,
                   float *y, int32_t *dot_out, int kernel, int variant, void *stream);

/* The two phases of i2s_mul_mat as separate calls, so that one quantized
 * activation can feed several weights (the sidecar of "ggml-cpu: ternary I2_S
 * matmul kernel (VibeASR, 3/4)", Interface; its Kernels/threading section
 * quantizes all rows first, then splits the output features).
 *
 * i2s_quantize_act_ws: quantize x[N][K] into `workspace` (private layout,
 * >= i2s_act_workspace_bytes(N, K) bytes, 256-byte aligned).
 * Errors: as i2s_mul_mat. */
int i2s_quantize_act_ws(const float *x, int64_t N, int64_t K,
                        void *workspace, size_t workspace_bytes, void *stream);

/* i2s_mul_mat_ws: contraction + epilogue of the packed weight against the
 * activations already quantized into `workspace` by i2s_quantize_act_ws with
 * the same N and K (stream-ordered after it).  kernel/variant as in
 * i2s_mul_mat_ex.  The workspace is only read. */
int i2s_mul_mat_ws(const uint8_t *packed, int64_t rows, int64_t K, int64_t N,
                   const void *workspace, size_t workspace_bytes,
                   float *y, int32_t *dot_out, int kernel, int variant, void *stream);

/* i2s_mul_mat_batched: the op on a 3-D activation ("ggml-cpu: ternary I2_S
 * matmul kernel (VibeASR, 3/4)", Tests: the batched case, whose activation
 * rows walk a batch stride and whose outputs walk theirs).  For b < B and
 * n < N, activation row (b, n) is the K floats at x + b*bsx + n*ldx and its
 * output row is the `rows` floats at y + b*bsy + n*ldy (dot_out, if not NULL,
 * uses y's strides); the 2-D weight is shared by every batch.  Strides are in
 * elements: ldx >= K with ldx and bsx multiples of 4 (activation rows start
 * 16-byte aligned), ldy >= rows, bsy >= 0, and outputs of different batches
 * must not overlap (bsy >= (N-1)*ldy + rows when B > 1).  x, y and dot_out
 * themselves are 16-byte aligned.  workspace >= i2s_act_workspace_bytes(N*B, K).
 * Dense strides run as one i2s_mul_mat of N*B rows; otherwise one quantize
 * launch (or, for N <= 3, one fused launch per batch) and one contraction per
 * batch.  Errors: as i2s_mul_mat, I2S_EINVAL for a bad stride, I2S_ERANGE for
 * ldx, ldy or N*B beyond 2^31 - 1. */
int i2s_mul_mat_batched(const uint8_t *packed, int64_t rows, int64_t K,
                        const float *x, int64_t N, int64_t B, int64_t ldx, int64_t bsx,
                        void *workspace, size_t workspace_bytes,
                        float *y, int64_t ldy, int64_t bsy, int32_t *dot_out, void *stream);

/* Grouped projections sharing one activation ("VibeASR in audio.cpp",
 * Architecture/Decoder: every decoder layer applies the ternary q, k and v
 * projections to one normed hidden state, and gate and up to another; the
 * q/k/v projections carry F32 biases).  Each projection is the whole op of
 * i2s_mul_mat on the same x -- quantized once, since quantization depends on
 * x alone -- followed, if it has a bias, by one F32 add per output
 * y[n][o] += bias[o] after the epilogue (the separate F32 bias tensor add).
 * All pointers in an i2s_proj are device pointers owned by the caller. */
#define I2S_GROUP_MAX 8
typedef struct i2s_proj {
    const uint8_t *packed;  /* I2_S tensor of rows x K (i2s_pack), 16-byte aligned     */
    int64_t rows;           /* output features (>= 0; 0 = skipped)                     */
    const float *bias;      /* NULL, or [rows] F32, 16-byte aligned                    */
    float *y;               /* [N][rows] F32, 16-byte aligned, fully overwritten       */
    int32_t *dot_out;       /* NULL, or [N][rows] int32 receiving sum(code*q)          */
} i2s_proj;

/* i2s_mul_mat_group: `count` (1..I2S_GROUP_MAX) projections of x[N][K] (F32,
 * finite, 16-byte aligned).  projs is a HOST array, read before the call
 * returns.  For N <= 3 and K <= 9216 the group runs as one fused
 * quantize + GEMV launch; otherwise x is quantized once into `workspace`
 * (>= i2s_act_workspace_bytes(N, K) bytes, 256-byte aligned, overwritten) and
 * each projection gets its own contraction launch.  Outputs of different
 * projections must not overlap.
 * Errors: I2S_EINVAL (count out of range, a null or misaligned pointer, a
 * negative size), I2S_EALIGN, I2S_EWORKSPACE, I2S_ERANGE, I2S_EHIP; nothing is
 * launched unless every projection passes. */
int i2s_mul_mat_group(const i2s_proj *projs, int count, int64_t K,
                      const float *x, int64_t N,
                      void *workspace, size_t workspace_bytes, void *stream);

/* i2s_mul_mat_group with the kernel and variant chosen by the caller, as in
 * i2s_mul_mat_ex (kernel 3 = the fused group launch). */
int i2s_mul_mat_group_ex(const i2s_proj *projs, int count, int64_t K,
                         const float *x, int64_t N,
                         void *workspace, size_t workspace_bytes,
                         int kernel, int variant, void *stream);

/* i2s_mul_mat without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The library calls no allocator in it.  The
 * activation workspace is instead a fixed array in the library's device
 * memory, I2S_NOALLOC_SCRATCH_BYTES (32 MiB) on every GPU the library runs on,
 * held until the process ends; the kernels and every result bit are those of
 * i2s_mul_mat.  Arguments as i2s_mul_mat's.
 * Shapes with i2s_act_workspace_bytes(N, K) > I2S_NOALLOC_SCRATCH_BYTES return
 * I2S_ESCRATCH before anything is launched (N * K up to about 16 million
 * fits: 512 x 1536 and 1024 x 8960 do).  All calls on one GPU share that
 * GPU's array, so calls that overlap on one GPU (other streams, other host
 * threads) race on it: order them on one stream, or use i2s_mul_mat with a
 * workspace each.  The array needs no clearing: every call writes the parts
 * it reads.  The first call on a device looks up the array's address there
 * (no allocation).
 * Errors: as i2s_mul_mat, and I2S_ESCRATCH. */
#define I2S_NOALLOC_SCRATCH_BYTES (32u << 20)
int i2s_mul_mat_noalloc(const uint8_t *packed, int64_t rows, int64_t K,
                        const float *x, int64_t N,
                        float *y, int32_t *dot_out, void *stream);

/* The size of that array: I2S_NOALLOC_SCRATCH_BYTES. */
size_t i2s_noalloc_scratch_bytes(void);

/* The contraction kernel i2s_mul_mat launches for this shape (1 = GEMV after
 * a separate quantize launch, 2 = MFMA GEMM after a separate quantize launch,
 * 3 = fused quantize + GEMV, one launch, 4 = skinny MFMA after a separate
 * quantize launch), or minus a status code.  i2s_mul_mat_ws with kernel 0
 * makes the same choice, except that it never fuses (x is not an argument):
 * where this returns 3 it runs kernel 1 for N = 1 and for N = 2 with
 * K <= 2048, kernel 4 otherwise. */
int i2s_mul_mat_kernel(int64_t rows, int64_t K, int64_t N);

/* The tile configuration (1-based variant) of that kernel which the automatic
 * choice uses for this shape, or minus a status code. */
int i2s_mul_mat_variant(int64_t rows, int64_t K, int64_t N);

/* Number of tile configurations kernel `kernel` (1 to 4) offers; 0 otherwise. */
int i2s_kernel_variants(int kernel);

/* A short static English description of a status code. */
const char *i2s_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* I2S_H */
