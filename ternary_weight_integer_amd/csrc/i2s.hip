// gfx950 (MI355X) kernels and C ABI for the I2_S ternary-weight x int8-activation
// matmul.  The ABI is declared, with its contract, in include/i2s.h.
//
// The op ("ggml-cpu: ternary I2_S matmul kernel (VibeASR, 3/4)", Interface and
// Arithmetic): weights are 2-bit codes {0,1,2} for {-1,0,+1}; activations are
// quantized per row to int8 with the multiplier scale amax/127; the
// contraction accumulates sum(code*q) in int32 and the epilogue computes
// (float)(dot - row_sum) * (weight_scale * act_scale).
//
// Packed layout ("ggml: additive INT8/ternary types, fused CPU ops, and kernels
// for VibeASR (1/2)", Two new types and Kernels): 128 values per 32-byte group;
// within a group, byte i carries the codes of positions i, i+32, i+64 and i+96
// (counted from the group's start), from the high bit pair down to the low
// one; the tensor's F32 scale follows the payload in band.
// A packed dword (bytes gp..gp+3 of a group) therefore yields, for slice s,
// (dword >> (6-2s)) & 0x03030303 = the codes of the four consecutive positions
// 32s+gp .. 32s+gp+3, one per byte, ready for a 4-way int8 dot.
//
// Private activation layout in the i2s_mul_mat workspace ("group-interleaved"):
// within each 128-value group, the 16 bytes that pair with packed dword c
// (bytes 4c..4c+3 of the group, c = 0..7) are stored together, slice by slice:
//     qp[g*128 + 16c + 4s + t] = q[g*128 + 32s + 4c + t]      (s, t in 0..3)
// so packed byte b of a row pairs with qp bytes 4b..4b+3, and a 16-byte
// chunk j of packed weights (row bytes 16j..16j+15) pairs with the 64
// contiguous qp bytes 64j..64j+63.  Integer sums do not depend on the order
// of their terms, so this permutation changes no result bit.
//
// The workspace also has room for an MFMA-tiled copy qt of qp, the operand
// order of the skinny int8-MFMA kernel, filled when a contraction has at most
// 64 rows: for each block b of 16 activation rows, each 256-position step st
// and each chunk d = 0..3, one KiB in which lane l = i + 16*kb (i, kb: 0..15,
// 0..3) holds at 16*l the 16 bytes qp[16b + i][256*st + 64*kb + 16*d ..], so
// one 16-byte load per lane reads a whole operand from contiguous memory.
// Slots of rows >= N and of positions >= K are never written (the kernel
// does not read them).

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <atomic>
#include <type_traits>

#include "i2s.h"

namespace {

constexpr int kGroupValues = 128;
constexpr int kScaleSlot = 32;
constexpr unsigned kCodeMask = 0x03030303u;
constexpr int64_t kMaxK = 8454528;  // 2*127*K stays below 2^31 (int32 accumulators)
constexpr int64_t kMaxDim = 0x7fffffff;
constexpr int64_t kTiledMaxN = 64;  // largest contraction N for which the quantizer fills the tiled copy

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct ActWorkspace {
  int8_t *q = nullptr;
  float *scale = nullptr;
  int32_t *row_sum = nullptr;
  int8_t *qt = nullptr;  // the MFMA-tiled copy of q, or nullptr where it is not filled
  int64_t qt_row0 = 0;   // tiled-copy row of q's row 0 (a batch's first row)
};

// Bytes of the MFMA-tiled copy: ceil(N/16) blocks x ceil(K/256) steps x 4 KiB.
inline size_t tiled_bytes(int64_t N, int64_t K) {
  if (N < 1) return 0;
  return static_cast<size_t>((N + 15) / 16) * static_cast<size_t>((K + 255) / 256) * 4096;
}

// The workspace of N activation rows of length K; the tiled copy is used
// (qt set) when the contractions that read it have at most kTiledMaxN rows
// (contraction_n: N, or a batch's rows).
inline ActWorkspace carve_workspace(void *base, int64_t N, int64_t K, int64_t contraction_n) {
  char *p = static_cast<char *>(base);
  size_t q_bytes = align_up(static_cast<size_t>(N) * static_cast<size_t>(K), 256);
  size_t s_bytes = align_up(static_cast<size_t>(N) * 4, 256);
  ActWorkspace ws;
  ws.q = reinterpret_cast<int8_t *>(p);
  ws.scale = reinterpret_cast<float *>(p + q_bytes);
  ws.row_sum = reinterpret_cast<int32_t *>(p + q_bytes + s_bytes);
  ws.qt = contraction_n <= kTiledMaxN && tiled_bytes(N, K) ? reinterpret_cast<int8_t *>(p + q_bytes + 2 * s_bytes)
                                                            : nullptr;
  ws.qt_row0 = 0;
  return ws;
}

// Offset in the tiled copy of byte p (group-interleaved order) of activation row n.
__device__ inline int64_t tiled_offset(int64_t n, int64_t p, int64_t steps) {
  return ((((n >> 4) * steps + (p >> 8)) * 4 + ((p >> 4) & 3)) << 10) + 16 * ((n & 15) + 16 * ((p >> 6) & 3)) + (p & 15);
}

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------------------
// Block-wide reductions (256 threads = 4 wave64s).

// Cross-lane steps as DPP moves (VALU, a few cycles each) instead of
// ds_bpermute (an LDS round trip each, which nothing hides at one wave per
// SIMD): within each quad, then each 8 and each 16 lanes by mirroring, then
// across the four rows of 16 by reading one lane of each.  Max and integer
// sums do not depend on the order of their terms.
template <int CTRL>
__device__ inline int dpp_move(int v) { return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false); }
constexpr int kDppXor1 = 0xB1;         // quad_perm(1,0,3,2)
constexpr int kDppXor2 = 0x4E;         // quad_perm(2,3,0,1)
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7-i within each 8
constexpr int kDppMirror = 0x140;      // lane i <- lane 15-i within each 16
constexpr int kDppRowRor8 = 0x128;     // lane i <- lane i ^ 8 within each 16 (rotation by 8)

__device__ inline float wave_max(float v) {
  v = fmaxf(v, __int_as_float(dpp_move<kDppXor1>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_move<kDppXor2>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_move<kDppHalfMirror>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_move<kDppMirror>(__float_as_int(v))));
  const int b = __float_as_int(v);
  return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 0)), __int_as_float(__builtin_amdgcn_readlane(b, 16))),
               fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 32)), __int_as_float(__builtin_amdgcn_readlane(b, 48))));
}

// Sum over each group of L consecutive lanes (L a power of two up to 64),
// the result in every lane of the group.
template <int L>
__device__ inline int lanes_sum(int v) {
  static_assert(L >= 1 && L <= 64 && (L & (L - 1)) == 0, "power-of-two lane group");
  if constexpr (L >= 2) v += dpp_move<kDppXor1>(v);
  if constexpr (L >= 4) v += dpp_move<kDppXor2>(v);
  if constexpr (L >= 8) v += dpp_move<kDppHalfMirror>(v);
  if constexpr (L >= 16) v += dpp_move<kDppMirror>(v);
  if constexpr (L == 32) {
    const int lo = __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16);
    const int hi = __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
    v = (threadIdx.x & 32) ? hi : lo;
  }
  if constexpr (L == 64)
    v = (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
        (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
  return v;
}

__device__ inline int wave_sum(int v) { return lanes_sum<64>(v); }

// Quantizes the 4*XPT activation values a thread holds with the row's scale
// s (an IEEE quotient amax/127): code = clamp(roundf(x / s), -127, 127) with
// x / s the IEEE quotient, four codes per dword (value t of float4 i in byte
// t of packed[i]).  Values past the row are 0 and give code 0.
//
// x / s is formed as x * rcp(s) with v_rcp_f32 (1 ulp): |x / s| <= 127.5,
// so the product is within 127.5 * 1.5 * 2^-23 < 2^-15 of the real quotient
// and within 2^-15 + 2^-18 < 2^-14 of the IEEE one.  A product farther than
// 2^-14 from every half-integer therefore lies strictly between the same two
// half-integers as the IEEE quotient, and rounding the product to nearest
// even gives roundf of that quotient.  A value nearer
// than that to a tie takes the exact division and roundf instead.  The
// branches are wave-uniform: one over the thread's values (no value of the
// wave near a tie: the common case, every value rounded from its product),
// and inside it one per float4 (only a float4 position where some lane is
// near a tie divides, so a long row that meets a tie somewhere divides a
// few values instead of all of them).  NaN and infinite inputs take the
// same values on both paths (rcp(inf) = 0).
template <int XPT>
__device__ inline void quantize_codes(const float4 (&v)[XPT], float s, uint32_t (&packed)[XPT]) {
  const float inv = __builtin_amdgcn_rcpf(s);
  float rq[XPT][4];
  float dm[XPT];  // per float4: nearest distance of a product to a half-integer
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const float e[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    dm[i] = 1.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      rq[i][t] = e[t] * inv;
      dm[i] = fminf(dm[i], fabsf(__builtin_amdgcn_fractf(fabsf(rq[i][t])) - 0.5f));
    }
  }
  float dmin = dm[0];
#pragma unroll
  for (int i = 1; i < XPT; ++i) dmin = fminf(dmin, dm[i]);
  // Near a tie a position's values are replaced by roundf of the quotient
  // (already integers); everywhere else they stay products, rounded below.
  if (__any(dmin <= 0x1p-14f)) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      if (__any(dm[i] <= 0x1p-14f)) {
        // The divisor passes through an empty asm statement, so that the
        // divisions cannot be hoisted out of this branch (speculated, they
        // would run for every value of every wave).
        float sd = s;
        __asm__ volatile("" : "+v"(sd));
        const float e[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) rq[i][t] = roundf(e[t] / sd);
      }
    }
  }
  // Clamp to [-127, 127], then round to nearest even and convert in one add:
  // for |r| <= 127, r + 1.5 * 2^23 lies in [2^23, 2^24), where the spacing
  // of floats is 1, so the sum is r rounded to nearest even (exact for the
  // integers of the near-tie path), and its low byte is that integer's
  // two's-complement byte (1.5 * 2^23 = 0x4B400000 has a zero low byte).
  // Clamping first gives the same codes as rounding first: any value beyond
  // +-127 (at most 127.5 here) rounds to +-127 or +-128 and is clamped to
  // +-127.  fmaxf/fminf map NaN to -127, as the conversion path did.
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    uint32_t b[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) b[t] = __float_as_uint(fminf(fmaxf(rq[i][t], -127.0f), 127.0f) + 0x1.8p23f);
    const uint32_t lo = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u);  // bytes: b0.0, b1.0, 0, 0
    const uint32_t hi = __builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u);  // bytes: b2.0, b3.0, 0, 0
    packed[i] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);             // lo.0, lo.1, hi.0, hi.1
  }
}

// Sum of the four signed bytes of a dword added to acc (one v_dot4).
__device__ inline int add_bytes(uint32_t p4, int acc) {
  return __builtin_amdgcn_sdot4(static_cast<int>(p4), 0x01010101, acc, false);
}

// ---------------------------------------------------------------------------
// Activation quantization + row sum: one workgroup per activation row (the
// row-wide absmax cannot be split).  Pass 1 reduces max|x| over the row;
// pass 2 quantizes 16 values per thread-step and accumulates the int8 sum.
//   amax = max(max|x|, 1e-5f); s = amax / 127 (IEEE division);
//   q = clamp(roundf(x / s), -127, 127)   (roundf: halfway away from zero).
// kInterleaved selects the workspace order above; otherwise q is row-major.
// Activation row n is read from x + (n / n_inner) * bsx + (n % n_inner) * ldx
// (batches of n_inner rows; contiguous rows have n_inner = N, ldx = K); q,
// the scales and the row sums are written densely, row n at n, and q also
// into the MFMA-tiled copy qt when it is given (interleaved order only).

constexpr int kQuantThreads = 256;

template <bool kInterleaved>
__global__ void __launch_bounds__(kQuantThreads)
quantize_rowsum_kernel(const float *__restrict__ x, int64_t K, int64_t n_inner, int64_t ldx, int64_t bsx,
                       int8_t *__restrict__ q, float *__restrict__ act_scale, int32_t *__restrict__ row_sum,
                       int8_t *__restrict__ qt) {
  __shared__ float red_f[kQuantThreads / 64];
  __shared__ int red_i[kQuantThreads / 64];
  const int64_t n = blockIdx.x;
  const float *xr = x + (n / n_inner) * bsx + (n % n_inner) * ldx;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;

  float amax = 0.0f;
  const float4 *x4 = reinterpret_cast<const float4 *>(xr);
  for (int64_t i = tid; i < K / 4; i += kQuantThreads) {
    float4 v = x4[i];
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  amax = wave_max(amax);
  if (lane == 0) red_f[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red_f[0], red_f[1]), fmaxf(red_f[2], red_f[3]));
  amax = fmaxf(amax, 1e-5f);
  const float s = amax / 127.0f;

  int sum = 0;
  int8_t *qr = q + n * K;
  for (int64_t u = tid; u < K / 16; u += kQuantThreads) {
    uint32_t out[4];
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      int64_t p = kInterleaved ? (u / 8) * 128 + 32 * sl + 4 * (u % 8) : 16 * u + 4 * sl;
      float4 v = *reinterpret_cast<const float4 *>(xr + p);
      float e[4] = {v.x, v.y, v.z, v.w};
      uint32_t packed = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float r = roundf(e[t] / s);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        int qi = static_cast<int>(r);
        sum += qi;
        packed |= (static_cast<uint32_t>(qi) & 0xffu) << (8 * t);
      }
      out[sl] = packed;
    }
    *reinterpret_cast<uint4 *>(qr + 16 * u) = make_uint4(out[0], out[1], out[2], out[3]);
    if (kInterleaved && qt)
      *reinterpret_cast<uint4 *>(qt + tiled_offset(n, 16 * u, (K + 255) / 256)) = make_uint4(out[0], out[1], out[2], out[3]);
  }
  sum = wave_sum(sum);
  if (lane == 0) red_i[wave] = sum;
  __syncthreads();
  if (tid == 0) {
    act_scale[n] = s;
    row_sum[n] = red_i[0] + red_i[1] + red_i[2] + red_i[3];
  }
}

// Block per row, single pass, for K <= 4*256*XPT: each of the 256 threads
// loads up to XPT float4 of the row into registers, the row's absmax and int8
// sum are block reductions, and each float4 becomes 4 bytes of q (4
// consecutive positions stay consecutive in the interleaved order).  The
// codes equal quantize_rowsum_kernel's bit for bit (quantize_codes: one
// reciprocal per thread, divisions only in a wave near a rounding tie).
template <bool kInterleaved, int XPT, int THREADS>
__global__ void __launch_bounds__(THREADS)
quantize_rowsum_reg_kernel(const float *__restrict__ x, int64_t K, int64_t n_inner, int64_t ldx, int64_t bsx,
                           int8_t *__restrict__ q, int8_t *__restrict__ qt, float *__restrict__ act_scale,
                           int32_t *__restrict__ row_sum) {
  // Argument order: everything up to qt is preloaded into scalar registers
  // at launch; the scale and row-sum pointers (written at the very end) are
  // fetched while the row loads are in flight (below).
  constexpr int kWaves = THREADS / 64;
  __shared__ float red_f[kWaves];
  __shared__ int red_i[kWaves];
  const int64_t n = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const float4 *xr = reinterpret_cast<const float4 *>(x + (n / n_inner) * bsx + (n % n_inner) * ldx);
  const int k4 = static_cast<int>(K / 4);
  float4 v[XPT];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int idx = tid + THREADS * i;
    v[i] = idx < k4 ? xr[idx] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }
  // The two pointers as operands of an empty asm: their scalar load (and its
  // wait) happens here, in the shadow of the row loads, instead of being
  // sunk to the final stores.
  __asm__ volatile("" ::"s"(act_scale), "s"(row_sum));
#pragma unroll
  for (int i = 0; i < XPT; ++i)
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
  amax = wave_max(amax);
  if (lane == 0) red_f[wave] = amax;
  __syncthreads();
  amax = red_f[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) amax = fmaxf(amax, red_f[w]);
  amax = fmaxf(amax, 1e-5f);
  const float s = amax / 127.0f;
  uint32_t codes[XPT];
  quantize_codes<XPT>(v, s, codes);
  int sum = 0;
  int8_t *qr = q + n * K;
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int idx = tid + THREADS * i;
    if (idx < k4) {
      sum = add_bytes(codes[i], sum);
      const int p = 4 * idx;
      const int jj = p & 127;
      const int off = kInterleaved ? (p & ~127) + 16 * ((jj & 31) >> 2) + 4 * (jj >> 5) : p;
      *reinterpret_cast<uint32_t *>(qr + off) = codes[i];
      if (kInterleaved && qt) *reinterpret_cast<uint32_t *>(qt + tiled_offset(n, off, (K + 255) / 256)) = codes[i];
    }
  }
  sum = wave_sum(sum);
  if (lane == 0) red_i[wave] = sum;
  __syncthreads();
  if (tid == 0) {
    int total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) total += red_i[w];
    act_scale[n] = s;
    row_sum[n] = total;
  }
}

// ---------------------------------------------------------------------------
// Pack: each thread writes 16 packed bytes (half a group) from the 4x16
// ternary values they hold; thread 0 also writes the scale slot.

constexpr int kPackThreads = 256;

__device__ inline uint32_t code_of(int8_t w) { return w > 0 ? 2u : (w < 0 ? 0u : 1u); }

__global__ void __launch_bounds__(kPackThreads)
pack_kernel(const int8_t *__restrict__ w, float weight_scale, int64_t units, int64_t payload,
            uint8_t *__restrict__ packed) {
  const int64_t u = static_cast<int64_t>(blockIdx.x) * kPackThreads + threadIdx.x;
  if (u == 0) {
    uint32_t slot[8] = {__float_as_uint(weight_scale), 0, 0, 0, 0, 0, 0, 0};
    uint4 *dst = reinterpret_cast<uint4 *>(packed + payload);
    dst[0] = make_uint4(slot[0], slot[1], slot[2], slot[3]);
    dst[1] = make_uint4(slot[4], slot[5], slot[6], slot[7]);
  }
  if (u >= units) return;
  const int64_t base = (u / 2) * kGroupValues + 16 * (u % 2);
  int8_t v[4][16];
#pragma unroll
  for (int sl = 0; sl < 4; ++sl) *reinterpret_cast<uint4 *>(v[sl]) = *reinterpret_cast<const uint4 *>(w + base + 32 * sl);
  uint32_t out[4] = {0, 0, 0, 0};
#pragma unroll
  for (int b = 0; b < 16; ++b) {
    uint32_t byte = (code_of(v[0][b]) << 6) | (code_of(v[1][b]) << 4) | (code_of(v[2][b]) << 2) | code_of(v[3][b]);
    out[b / 4] |= byte << (8 * (b % 4));
  }
  *reinterpret_cast<uint4 *>(packed + 16 * u) = make_uint4(out[0], out[1], out[2], out[3]);
}

// ---------------------------------------------------------------------------
// Epilogue shared by both contraction kernels: two IEEE multiplies in the
// stated order, t = ws * s first, then (float)(dot - row_sum) * t.

__device__ inline float epilogue(int32_t dot, int32_t rsum, float t) {
  return static_cast<float>(dot - rsum) * t;
}

// Optional F32 bias of a projection (the decoder's q/k/v projections carry
// one), added to the finished epilogue value as one more IEEE add: the
// bias tensor add that follows the matmul.  The library is built with FP
// contraction off, so the multiply above and this add are never fused.
__device__ inline float add_bias(float v, float b) { return v + b; }

// ---------------------------------------------------------------------------
// GEMV for N <= 8 columns: streams packed weights with 128-bit loads and
// accumulates with v_dot4 (4-way int8 dot into int32).
//
// A workgroup is 4 wave64s; in a wave, L consecutive lanes share a weight row
// and split its 16-byte chunks (chunk j goes to lane j mod L), 64/L rows per
// pass, RPL passes per wave, so a wave covers RPL*64/L rows.  Each lane loads
// its weight chunks for all RPL rows before touching activations; the 64
// group-interleaved activation bytes of a chunk are loaded once and reused for
// the RPL rows.  Partial sums are reduced across the L lanes of a row and the
// epilogue is applied in registers.

constexpr int kGemvThreads = 256;



// Raw buffer accesses: the descriptor bounds the tensor, out-of-range loads
// read 0 and out-of-range stores are dropped by the hardware.
typedef int v4i __attribute__((ext_vector_type(4)));
constexpr uint32_t kOutOfRange = 0x7ffffff0u;  // buffer offset beyond every descriptor's range
constexpr int kBufferFlags = 0x00020000;       // raw buffer, 32-bit data format

__device__ inline __amdgpu_buffer_rsrc_t buffer_of(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           kBufferFlags);
}

template <int NC, int L, int RPL, int CPL>
__global__ void __launch_bounds__(kGemvThreads)
gemv_kernel(const uint8_t *__restrict__ packed, const int8_t *__restrict__ qp, const float *__restrict__ act_scale,
            const int32_t *__restrict__ row_sum, const float *__restrict__ bias, int rows32, int K32, int ldy32,
            float *__restrict__ y, int32_t *__restrict__ dot_out) {
  // Argument order: the five pointers and three sizes that the first loads
  // need fill the 13 leading dwords, which are preloaded into scalar
  // registers at wave launch; only the output pointers, needed at the stores,
  // are loaded from the argument segment.  (With 64-bit sizes the bias
  // pointer came after the preloaded dwords, and every wave waited for its
  // scalar load before the first weight load.)
  const int64_t rows = rows32, K = K32, ldy = ldy32;
  constexpr int kSlots = 64 / L;
  constexpr int kRowsPerWave = kSlots * RPL;
  constexpr int kRowsPerBlock = kRowsPerWave * (kGemvThreads / 64);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int lam = lane % L, slot = lane / L;
  const int64_t C = K / 64;               // 16-byte chunks per packed row
  const int64_t row_bytes = K / 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + wave * kRowsPerWave + slot;

  // Epilogue constants first (buffer loads keep their place): the weight
  // scale from the in-band slot, the activation scales and row sums, and this
  // lane's biases.  Loaded at their use they would cost one more memory round
  // trip before the stores.
  const float ws = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(buffer_of(packed + rows * row_bytes, 4), 0, 0, 0));
  float asc[NC];
  int32_t rsum[NC];
  float bv[RPL];
  {
    const __amdgpu_buffer_rsrc_t sbuf = buffer_of(act_scale, 4 * NC);
    const __amdgpu_buffer_rsrc_t rbuf = buffer_of(row_sum, 4 * NC);
#pragma unroll
    for (int n = 0; n < NC; ++n) {
      asc[n] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(sbuf, 4 * n, 0, 0));
      rsum[n] = __builtin_amdgcn_raw_buffer_load_b32(rbuf, 4 * n, 0, 0);
    }
    const __amdgpu_buffer_rsrc_t bbuf = buffer_of(bias, bias ? static_cast<uint32_t>(rows * 4) : 0u);
#pragma unroll
    for (int m = 0; m < RPL; ++m) {
      const int64_t r = row0 + static_cast<int64_t>(m) * kSlots;
      bv[m] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          bbuf, r < rows ? static_cast<uint32_t>(4 * r) : kOutOfRange, 0, 0));
    }
  }

  int acc[RPL][NC];
#pragma unroll
  for (int m = 0; m < RPL; ++m)
#pragma unroll
    for (int n = 0; n < NC; ++n) acc[m][n] = 0;

  for (int64_t jb = 0; jb < C; jb += static_cast<int64_t>(L) * CPL) {
    uint4 wv[RPL][CPL];
#pragma unroll
    for (int m = 0; m < RPL; ++m) {
      const int64_t r = row0 + static_cast<int64_t>(m) * kSlots;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int64_t j = jb + lam + static_cast<int64_t>(L) * c;
        if (r < rows && j < C)
          wv[m][c] = *reinterpret_cast<const uint4 *>(packed + r * row_bytes + 16 * j);
        else
          wv[m][c] = make_uint4(0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u);
      }
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int64_t j = jb + lam + static_cast<int64_t>(L) * c;
      if (j >= C) continue;
#pragma unroll
      for (int n = 0; n < NC; ++n) {
        const uint4 *qv = reinterpret_cast<const uint4 *>(qp + static_cast<int64_t>(n) * K + 64 * j);
        uint4 qd[4] = {qv[0], qv[1], qv[2], qv[3]};
#pragma unroll
        for (int m = 0; m < RPL; ++m) {
          const uint32_t wd[4] = {wv[m][c].x, wv[m][c].y, wv[m][c].z, wv[m][c].w};
          int a = acc[m][n];
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const uint32_t w = wd[d];
            a = __builtin_amdgcn_sdot4(static_cast<int>((w >> 6) & kCodeMask), static_cast<int>(qd[d].x), a, false);
            a = __builtin_amdgcn_sdot4(static_cast<int>((w >> 4) & kCodeMask), static_cast<int>(qd[d].y), a, false);
            a = __builtin_amdgcn_sdot4(static_cast<int>((w >> 2) & kCodeMask), static_cast<int>(qd[d].z), a, false);
            a = __builtin_amdgcn_sdot4(static_cast<int>(w & kCodeMask), static_cast<int>(qd[d].w), a, false);
          }
          acc[m][n] = a;
        }
      }
    }
  }

#pragma unroll
  for (int m = 0; m < RPL; ++m) {
    const int64_t r = row0 + static_cast<int64_t>(m) * kSlots;
#pragma unroll
    for (int n = 0; n < NC; ++n) {
      const int total = lanes_sum<L>(acc[m][n]);
      if (r < rows && lam == n % L) {
        const float t = ws * asc[n];
        float v = epilogue(total, rsum[n], t);
        if (bias) v = add_bias(v, bv[m]);
        y[static_cast<int64_t>(n) * ldy + r] = v;
        if (dot_out) dot_out[static_cast<int64_t>(n) * ldy + r] = total;
      }
    }
  }
}


// ---------------------------------------------------------------------------
// Fused quantize + GEMV for small N*K (the decode shapes): one launch per
// step.  Each workgroup issues all of its weight loads first, then quantizes
// the N activation rows itself while they are in flight -- block-wide absmax,
// s = amax/127, q = clamp(roundf(x/s), +-127), block-wide int8 row sum, the
// same single IEEE operations as quantize_rowsum_kernel -- into LDS in the
// group-interleaved order, and runs the v_dot4 contraction of gemv_kernel on
// it.  Requires K <= 64*L*CPL (one weight batch) and K <= 4*T*XPT (T
// threads per workgroup, XPT float4 activation loads per thread per row).

template <int NC, int L, int RPL, int CPL, int XPT, int T>
__device__ __forceinline__ void fused_body(const uint8_t *__restrict__ packed, int64_t rows, int64_t K,
                                           const float *__restrict__ x, int64_t ldx, float *__restrict__ y,
                                           int32_t *__restrict__ dot_out, const float *__restrict__ bias,
                                           int64_t ldy, int64_t block,
                                           int8_t *qs /* NC x K group-interleaved int8, LDS */) {
  constexpr int kWaves = T / 64;
  __shared__ float red_f[NC][kWaves];
  __shared__ int red_i[NC][kWaves];
  constexpr int kSlots = 64 / L;
  constexpr int kRowsPerWave = kSlots * RPL;
  constexpr int kRowsPerBlock = kRowsPerWave * kWaves;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int lam = lane % L, slot = lane / L;
  const int C = static_cast<int>(K / 64);  // 16-byte chunks per packed row
  const int64_t row_bytes = K / 4;
  const int64_t row0 = block * kRowsPerBlock + wave * kRowsPerWave + slot;

  // 1. Activation rows first: their absmax is the critical path, and loads
  // retire in order, so they must not queue behind the weights.
  // Buffer loads: past the row they read 0, with no branch around them.
  const int k4 = static_cast<int>(K / 4);
  float4 xv[NC][XPT];
#pragma unroll
  for (int n = 0; n < NC; ++n) {
    const __amdgpu_buffer_rsrc_t xbuf = buffer_of(x + static_cast<int64_t>(n) * ldx, static_cast<uint32_t>(16 * k4));
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int idx = tid + T * i;
      const v4i v = __builtin_amdgcn_raw_buffer_load_b128(xbuf, idx < k4 ? static_cast<uint32_t>(16 * idx) : kOutOfRange, 0, 0);
      xv[n][i] = make_float4(__int_as_float(v[0]), __int_as_float(v[1]), __int_as_float(v[2]), __int_as_float(v[3]));
    }
  }

  // Epilogue constants next, ahead of the weights (buffer loads keep their
  // place; loaded at their use they would cost one more memory round trip
  // before the stores): the weight scale from the in-band slot and this
  // lane's biases.
  const float ws = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(buffer_of(packed + rows * row_bytes, 4), 0, 0, 0));
  float bv[RPL];
  {
    const __amdgpu_buffer_rsrc_t bbuf = buffer_of(bias, bias ? static_cast<uint32_t>(rows * 4) : 0u);
#pragma unroll
    for (int m = 0; m < RPL; ++m) {
      const int64_t r = row0 + static_cast<int64_t>(m) * kSlots;
      bv[m] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          bbuf, r < rows ? static_cast<uint32_t>(4 * r) : kOutOfRange, 0, 0));
    }
  }

  // 2. Weight loads for every row and chunk of this lane, unconditional:
  // rows past the end read as 0x00 bytes (all codes 0, which add nothing to
  // sum(code*q)) and are never stored.  (A load past the row still takes an
  // issue slot, and a branch around it costs more: the configurations size
  // CPL to the row.)
  const __amdgpu_buffer_rsrc_t wbuf = buffer_of(packed, static_cast<uint32_t>(rows * row_bytes));
  v4i wv[RPL][CPL];
#pragma unroll
  for (int m = 0; m < RPL; ++m) {
    const int64_t r = row0 + static_cast<int64_t>(m) * kSlots;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int j = lam + L * c;
      const uint32_t off = r < rows && j < C ? static_cast<uint32_t>(r * row_bytes + 16 * j) : kOutOfRange;
      wv[m][c] = __builtin_amdgcn_raw_buffer_load_b128(wbuf, off, 0, 0);
    }
  }

  float amax[NC];
#pragma unroll
  for (int n = 0; n < NC; ++n) {
    amax[n] = 0.0f;
#pragma unroll
    for (int i = 0; i < XPT; ++i)
      amax[n] = fmaxf(amax[n], fmaxf(fmaxf(fabsf(xv[n][i].x), fabsf(xv[n][i].y)),
                                     fmaxf(fabsf(xv[n][i].z), fabsf(xv[n][i].w))));
    amax[n] = wave_max(amax[n]);
    if (lane == 0) red_f[n][wave] = amax[n];
  }
  __syncthreads();

  // 3. Quantize into LDS: the 4 consecutive positions of a float4 land on 4
  // consecutive bytes of the interleaved order (position 128g + 32s + 4c + t
  // goes to 128g + 16c + 4s + t).
  float sc[NC];
#pragma unroll
  for (int n = 0; n < NC; ++n) {
    float a = red_f[n][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) a = fmaxf(a, red_f[n][w]);
    a = fmaxf(a, 1e-5f);
    sc[n] = a / 127.0f;
    uint32_t codes[XPT];
    quantize_codes<XPT>(xv[n], sc[n], codes);
    int sum = 0;
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int idx = tid + T * i;
      if (idx < k4) {
        sum = add_bytes(codes[i], sum);
        const int p = 4 * idx;
        const int jj = p & 127;
        const int off = (p & ~127) + 16 * ((jj & 31) >> 2) + 4 * (jj >> 5);
        *reinterpret_cast<uint32_t *>(qs + n * K + off) = codes[i];
      }
    }
    sum = wave_sum(sum);
    if (lane == 0) red_i[n][wave] = sum;
  }
  __syncthreads();

  // 4. Contraction from LDS: four independent int32 partial sums per
  // (row, activation row) -- one per dword of a chunk -- so that consecutive
  // v_dot4 do not wait on each other; integer sums are exact in any order.
  int acc[RPL][NC][4];
#pragma unroll
  for (int m = 0; m < RPL; ++m)
#pragma unroll
    for (int n = 0; n < NC; ++n)
#pragma unroll
      for (int d = 0; d < 4; ++d) acc[m][n][d] = 0;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int j = lam + L * c;
    if (j >= C) continue;
#pragma unroll
    for (int n = 0; n < NC; ++n) {
      const uint4 *qv = reinterpret_cast<const uint4 *>(qs + n * K + 64 * j);
      const uint4 qd[4] = {qv[0], qv[1], qv[2], qv[3]};
#pragma unroll
      for (int m = 0; m < RPL; ++m) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t w = static_cast<uint32_t>(wv[m][c][d]);
          int a = acc[m][n][d];
          a = __builtin_amdgcn_sdot4(static_cast<int>((w >> 6) & kCodeMask), static_cast<int>(qd[d].x), a, false);
          a = __builtin_amdgcn_sdot4(static_cast<int>((w >> 4) & kCodeMask), static_cast<int>(qd[d].y), a, false);
          a = __builtin_amdgcn_sdot4(static_cast<int>((w >> 2) & kCodeMask), static_cast<int>(qd[d].z), a, false);
          a = __builtin_amdgcn_sdot4(static_cast<int>(w & kCodeMask), static_cast<int>(qd[d].w), a, false);
          acc[m][n][d] = a;
        }
      }
    }
  }

  // 5. Epilogue.
#pragma unroll
  for (int m = 0; m < RPL; ++m) {
    const int64_t r = row0 + static_cast<int64_t>(m) * kSlots;
#pragma unroll
    for (int n = 0; n < NC; ++n) {
      const int total = lanes_sum<L>((acc[m][n][0] + acc[m][n][1]) + (acc[m][n][2] + acc[m][n][3]));
      if (r < rows && lam == n % L) {
        int32_t rs = red_i[n][0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) rs += red_i[n][w];
        const float t = ws * sc[n];
        float v = epilogue(total, rs, t);
        if (bias) v = add_bias(v, bv[m]);
        y[static_cast<int64_t>(n) * ldy + r] = v;
        if (dot_out) dot_out[static_cast<int64_t>(n) * ldy + r] = total;
      }
    }
  }
}

// The pointers first and the four sizes as 32-bit values: the 14 argument
// dwords are all preloaded into scalar registers at wave launch, so no
// scalar load is waited for before the weight loads (with 64-bit sizes the
// bias pointer came after the preloaded dwords).
template <int NC, int L, int RPL, int CPL, int XPT, int T>
__global__ void __launch_bounds__(T)
gemv_fused_kernel(const uint8_t *__restrict__ packed, const float *__restrict__ x, float *__restrict__ y,
                  const float *__restrict__ bias, int32_t *__restrict__ dot_out, int rows, int K, int ldx, int ldy) {
  extern __shared__ __attribute__((aligned(16))) int8_t qs[];
  fused_body<NC, L, RPL, CPL, XPT, T>(packed, rows, K, x, ldx, y, dot_out, bias, ldy, blockIdx.x, qs);
}

// Several projections of the same activation rows in one launch (the decoder
// layer's q/k/v, or gate/up): a two-dimensional grid, blockIdx.y the
// projection and blockIdx.x the workgroup within it (workgroups past a
// shorter projection's rows exit at once), and each workgroup quantizes the
// shared rows itself, as above, before its share of one projection.  With
// the projection in a register from the start, its pointers are one batch
// of kernel-argument loads; numbering workgroups through the projections
// instead needs a search over their boundaries first, a chain of dependent
// scalar loads ahead of the weight loads.
struct FusedGroup {
  int count = 0;
  const uint8_t *packed[I2S_GROUP_MAX] = {};
  int64_t rows[I2S_GROUP_MAX] = {};
  const float *bias[I2S_GROUP_MAX] = {};
  float *y[I2S_GROUP_MAX] = {};
  int32_t *dot[I2S_GROUP_MAX] = {};
};

template <int NC, int L, int RPL, int CPL, int XPT, int T>
__global__ void __launch_bounds__(T)
gemv_fused_group_kernel(const FusedGroup g, int64_t K, const float *__restrict__ x) {
  extern __shared__ __attribute__((aligned(16))) int8_t qs[];
  constexpr int64_t kRowsPerBlock = (64 / L) * RPL * (T / 64);
  const int p = static_cast<int>(blockIdx.y);
  const int64_t block = blockIdx.x;
  const uint8_t *packed = g.packed[p];
  const int64_t rows = g.rows[p];
  const float *bias = g.bias[p];
  float *y = g.y[p];
  int32_t *dot = g.dot[p];
  // Every kernel argument the workgroup needs, in one batch of scalar loads
  // ahead of the exit test (the empty asm takes them as operands; loaded
  // after the test they would be one more round trip before the first
  // vector load).
  __asm__ volatile("" ::"s"(packed), "s"(rows), "s"(bias), "s"(y), "s"(dot), "s"(x), "s"(K));
  if (block * kRowsPerBlock >= rows) return;  // the whole workgroup, before any barrier
  fused_body<NC, L, RPL, CPL, XPT, T>(packed, rows, K, x, K, y, dot, bias, rows, block, qs);
}

// One of two values, by value (a conditional between two named objects would
// select between their addresses, here kernel-argument slots in memory).
template <class T>
__device__ __forceinline__ T pick(bool c, T a, T b) {
  return c ? a : b;
}

// The same for a pair of projections without biases or dot outputs (the
// decoder layer's gate and up), with every argument plain: the weight
// pointers, row counts, K, x and the two outputs are the first 14 argument
// dwords, all preloaded into scalar registers at wave launch, so the
// activation and weight loads go out at once and no scalar load is waited
// for anywhere (the table of the general kernel is a struct argument, which
// is never preloaded, and x and K come after it: gate+up at N = 1 took 4.30
// us with it, 4.09 with bias and dot pointers read as further arguments,
// and less without them).  A projection without rows has its workgroups
// exit at once.
template <int NC, int L, int RPL, int CPL, int XPT, int T>
__global__ void __launch_bounds__(T)
gemv_fused_pair_kernel(const uint8_t *__restrict__ p0, const uint8_t *__restrict__ p1, int r0, int r1, int K,
                       const float *__restrict__ x, float *y0, float *y1) {
  extern __shared__ __attribute__((aligned(16))) int8_t qs[];
  constexpr int64_t kRowsPerBlock = (64 / L) * RPL * (T / 64);
  const bool second = blockIdx.y != 0;
  const int64_t block = blockIdx.x;
  const uint8_t *packed = pick(second, p1, p0);
  const int64_t rows = pick(second, r1, r0);
  if (block * kRowsPerBlock >= rows) return;  // the whole workgroup, before any barrier
  fused_body<NC, L, RPL, CPL, XPT, T>(packed, rows, static_cast<int64_t>(K), x, K, pick(second, y1, y0), nullptr, nullptr,
                                      rows, block, qs);
}

// ---------------------------------------------------------------------------
// GEMM for larger N: int8 MFMA (v_mfma_i32_16x16x64_i8).
//
// One MFMA multiplies a 16(out) x 64 tile of codes by a 64 x 16(N) tile of
// activations.  Lane l supplies row/column l%16 and k-block l/16 of both
// operands, and only the pairing of A and B bytes matters: for K-step kk (256
// positions = 64 packed bytes of a row), lane (i, kb) loads the 16 packed
// bytes 64kk+16kb..+15 of weight row i; their dword d unpacks, slice by
// slice, into that lane's 16 A bytes of MFMA d, whose group-interleaved
// activation partners are qp bytes 256kk+64kb+16d..+15 of each column.
//
// A workgroup has WAVES_M x WAVES_N waves; each wave owns WM x WN 16x16 output
// tiles.  Activation tiles for one K-step are staged in LDS (double buffered)
// and shared by the waves; weight tiles go from global memory straight to
// registers.  Accumulators are int32; the epilogue runs in registers.

template <int WM, int WN, int WAVES_M, int WAVES_N>
struct GemmCfg {
  static constexpr int kWM = WM, kWN = WN, kWavesM = WAVES_M, kWavesN = WAVES_N;
  static constexpr int kThreads = 64 * WAVES_M * WAVES_N;
  static constexpr int kBM = 16 * WM * WAVES_M;   // output features per block
  static constexpr int kBN = 16 * WN * WAVES_N;   // activation rows per block
  static constexpr int kLdsStride = 256 + 16;     // bytes per activation row in LDS (padded)
  static constexpr int kLdsStage = kBN * kLdsStride;
};


// The 16 codes of one packed dword as an MFMA operand: dword s holds slice s
// ((w >> (6-2s)) & 0x03030303), i.e. positions 32s+gp .. 32s+gp+3.
__device__ inline v4i unpack_codes(uint32_t w) {
  v4i a;
  a[0] = static_cast<int>((w >> 6) & kCodeMask);
  a[1] = static_cast<int>((w >> 4) & kCodeMask);
  a[2] = static_cast<int>((w >> 2) & kCodeMask);
  a[3] = static_cast<int>(w & kCodeMask);
  return a;
}

template <class Cfg>
__global__ void __launch_bounds__(Cfg::kThreads)
gemm_kernel(const uint8_t *__restrict__ packed, int64_t rows, int64_t K,
            const int8_t *__restrict__ qp, int64_t N, const float *__restrict__ act_scale,
            const int32_t *__restrict__ row_sum, float *__restrict__ y,
            int32_t *__restrict__ dot_out, const float *__restrict__ bias, int64_t ldy, int64_t tiles_m) {
  constexpr int WM = Cfg::kWM, WN = Cfg::kWN;
  __shared__ __attribute__((aligned(16))) int8_t lds[2 * Cfg::kLdsStage];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave % Cfg::kWavesM, wn = wave / Cfg::kWavesM;
  const int li = lane & 15, kb = lane >> 4;
  const int64_t tile_m = blockIdx.x % tiles_m, tile_n = blockIdx.x / tiles_m;
  const int64_t o_base = tile_m * Cfg::kBM + wm * 16 * WM;
  const int64_t n_blk = tile_n * Cfg::kBN;
  const int64_t row_bytes = K / 4;
  const int64_t steps = K / 256 + ((K % 256) ? 1 : 0);  // K is a multiple of 128

  v4i acc[WM][WN];
#pragma unroll
  for (int m = 0; m < WM; ++m)
#pragma unroll
    for (int n = 0; n < WN; ++n) acc[m][n] = v4i{0, 0, 0, 0};

  // Cooperative copy of one K-step of activations (kBN rows x 256 bytes):
  // global loads into registers first, LDS stores later, so the loads of step
  // kk+1 are in flight while step kk's MFMAs run.
  constexpr int kPieces = Cfg::kBN * 16;  // 16-byte pieces per step
  constexpr int kPer = (kPieces + Cfg::kThreads - 1) / Cfg::kThreads;
  auto load_act = [&](int64_t kk, uint4 (&v)[kPer]) {
    const int64_t kbytes = (K - 256 * kk) >= 256 ? 256 : (K - 256 * kk);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int p = tid + i * Cfg::kThreads;
      const int r = p / 16, c = p % 16;
      const int64_t n = n_blk + r;
      v[i] = make_uint4(0, 0, 0, 0);
      if (p < kPieces && n < N && 16 * c < kbytes) v[i] = *reinterpret_cast<const uint4 *>(qp + n * K + 256 * kk + 16 * c);
    }
  };
  auto store_act = [&](int buf, const uint4 (&v)[kPer]) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int p = tid + i * Cfg::kThreads;
      const int r = p / 16, c = p % 16;
      if (p < kPieces) *reinterpret_cast<uint4 *>(lds + buf * Cfg::kLdsStage + r * Cfg::kLdsStride + 16 * c) = v[i];
    }
  };

  auto load_w = [&](int64_t kk, uint4 (&wv)[WM]) {
    const int64_t kbytes = (K - 256 * kk) >= 256 ? 256 : (K - 256 * kk);
#pragma unroll
    for (int m = 0; m < WM; ++m) {
      const int64_t o = o_base + 16 * m + li;
      if (o < rows && 16 * kb < kbytes / 4)  // tail step: only 32 of the 64 packed bytes exist
        wv[m] = *reinterpret_cast<const uint4 *>(packed + o * row_bytes + 64 * kk + 16 * kb);
      else
        wv[m] = make_uint4(0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u);  // code 1 = weight 0
    }
  };

  uint4 wcur[WM], wnext[WM];
  uint4 anext[kPer];
  load_w(0, wcur);
  load_act(0, anext);
  store_act(0, anext);
  __syncthreads();

  for (int64_t kk = 0; kk < steps; ++kk) {
    const int buf = static_cast<int>(kk & 1);
    const bool more = kk + 1 < steps;
    if (more) {
      load_w(kk + 1, wnext);
      load_act(kk + 1, anext);
    }
    const int8_t *lb = lds + buf * Cfg::kLdsStage;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      v4i b[WN];
#pragma unroll
      for (int n = 0; n < WN; ++n) {
        const int r = wn * 16 * WN + 16 * n + li;
        b[n] = *reinterpret_cast<const v4i *>(lb + r * Cfg::kLdsStride + 64 * kb + 16 * d);
      }
#pragma unroll
      for (int m = 0; m < WM; ++m) {
        const uint32_t wd = d == 0 ? wcur[m].x : d == 1 ? wcur[m].y : d == 2 ? wcur[m].z : wcur[m].w;
        const v4i a = unpack_codes(wd);
#pragma unroll
        for (int n = 0; n < WN; ++n) acc[m][n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b[n], acc[m][n], 0, 0, 0);
      }
    }
    // The other buffer was last read in step kk-1, before the barrier that ended it.
    if (more) store_act(buf ^ 1, anext);
    __syncthreads();
#pragma unroll
    for (int m = 0; m < WM; ++m) wcur[m] = wnext[m];
  }

  // Epilogue: lane l holds C[4*(l/16) + r][l % 16], r = 0..3, of each tile,
  // i.e. four consecutive output features of one activation row.
  const float ws = *reinterpret_cast<const float *>(packed + rows * row_bytes);
  // 16-byte stores only where every output row starts 16-byte aligned.
  const bool vec4_out = (rows % 4) == 0 && (ldy % 4) == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0 &&
                        (reinterpret_cast<uintptr_t>(dot_out) & 15) == 0;
#pragma unroll
  for (int n = 0; n < WN; ++n) {
    const int64_t nn = n_blk + wn * 16 * WN + 16 * n + li;
    if (nn >= N) continue;
    const float t = ws * act_scale[nn];
    const int32_t rs = row_sum[nn];
#pragma unroll
    for (int m = 0; m < WM; ++m) {
      const int64_t o = o_base + 16 * m + 4 * kb;
      float *yr = y + nn * ldy;
      if (o + 3 < rows && vec4_out) {
        float4 v = make_float4(epilogue(acc[m][n][0], rs, t), epilogue(acc[m][n][1], rs, t),
                               epilogue(acc[m][n][2], rs, t), epilogue(acc[m][n][3], rs, t));
        if (bias) {
          const float4 b = *reinterpret_cast<const float4 *>(bias + o);
          v = make_float4(add_bias(v.x, b.x), add_bias(v.y, b.y), add_bias(v.z, b.z), add_bias(v.w, b.w));
        }
        *reinterpret_cast<float4 *>(yr + o) = v;
        if (dot_out)
          *reinterpret_cast<int4 *>(dot_out + nn * ldy + o) = make_int4(acc[m][n][0], acc[m][n][1], acc[m][n][2], acc[m][n][3]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (o + r < rows) {
            float v = epilogue(acc[m][n][r], rs, t);
            if (bias) v = add_bias(v, bias[o + r]);
            yr[o + r] = v;
            if (dot_out) dot_out[nn * ldy + o + r] = acc[m][n][r];
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Activation-resident GEMM (same MFMA operand mapping as above).
//
// The workgroup's activation tile -- BN = 16*WN rows by the whole K, padded
// with zeros to chunks*S*256 columns -- is copied into LDS once; each wave
// copies BN/WAVES whole rows with all of its loads in flight before the first
// LDS store.  The row pitch is 16 bytes past a multiple of 256, so the 16
// lanes that read one 16-byte column of 16 rows hit distinct banks.
//
// The tile's ms 16-row weight subtiles are dealt to the WAVES waves
// round-robin.  A wave works through its subtiles G at a time and through K
// in chunks of S steps (256 positions each).  Before computing a (group,
// chunk) it issues the loads of the next one -- G x S x 16 bytes per lane,
// straight from HBM into the other of two register sets -- so a chunk of MFMAs
// covers the memory latency.  Each finished group is stored at once, so output
// stores overlap later MFMAs.
//
// Every global access is a buffer access whose descriptor bounds the tensor
// (out-of-range loads read 0, out-of-range stores are dropped by the
// hardware), and no load or store sits under a branch.  The number of memory
// operations in flight is therefore known at compile time, so each wait is
// for the operations it needs (the weights of the current chunk) and never
// for the prefetch or the stores issued after them.  Weight reads past the
// last row, past K, or for a group shorter than G only ever meet zero
// activations or feed outputs that are not stored.

constexpr int kResMaxLds = 160 * 1024;
__host__ __device__ inline int64_t res_pitch(int64_t K, int S) { return (K + 256 * S - 1) / (256 * S) * (256 * S) + 16; }


// Accumulate GS subtiles x WN column blocks over one K-step (256 positions,
// res_mfma_step) or over the S steps of one chunk (res_mfma_chunk).  lb is the
// lane's LDS base for the first step of the activation tile (row pitch
// `pitch`).
template <int GS, int G, int WN, int S>
__device__ __forceinline__ void res_mfma_step(v4i (&acc)[G][WN], const v4i (&wv)[G][S], int st, const int8_t *lb,
                                              uint32_t pitch) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    v4i b[WN];
#pragma unroll
    for (int n = 0; n < WN; ++n) b[n] = *reinterpret_cast<const v4i *>(lb + 256 * st + 16 * n * pitch + 16 * d);
#pragma unroll
    for (int gi = 0; gi < GS; ++gi) {
      const v4i a = unpack_codes(static_cast<uint32_t>(wv[gi][st][d]));
#pragma unroll
      for (int n = 0; n < WN; ++n) acc[gi][n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b[n], acc[gi][n], 0, 0, 0);
    }
  }
}

template <int GS, int G, int WN, int S>
__device__ __forceinline__ void res_mfma_chunk(v4i (&acc)[G][WN], const v4i (&wv)[G][S], const int8_t *lb,
                                               uint32_t pitch) {
#pragma unroll
  for (int st = 0; st < S; ++st) res_mfma_step<GS, G, WN, S>(acc, wv, st, lb, pitch);
}

template <int G, int WN, int S, int WAVES, bool VEC4, bool DOT, bool SINGLE, bool PERM, bool PAIR>
__global__ void __launch_bounds__(64 * WAVES)
gemm_res_kernel(int tiles_m, int ms, const uint8_t *__restrict__ packed, int64_t rows, int64_t K,
                const int8_t *__restrict__ qp, int64_t N, const int32_t *__restrict__ row_sum,
                const float *__restrict__ act_scale, float *__restrict__ y,
                int32_t *__restrict__ dot_out, const float *__restrict__ bias, int64_t ldy) {
  // Argument order: the arguments up to row_sum are preloaded into scalar
  // registers at launch, and they are all that the loads issued before the
  // first weights need (the tile, the weights, the row sums); the scales,
  // the outputs and the bias come from a scalar load that completes while
  // the tile streams in.
  extern __shared__ __attribute__((aligned(16))) int8_t lds_res[];
  constexpr int BN = 16 * WN;
  static_assert(BN % WAVES == 0, "whole activation rows per wave");
  constexpr int kRowsPerWave = BN / WAVES;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, kb = lane >> 4;
  const int64_t tile_m = blockIdx.x % tiles_m, tile_n = blockIdx.x / tiles_m;
  const int64_t o_tile = tile_m * ms * 16;
  const int64_t n0 = tile_n * BN;
  const int64_t n_here = N - n0 < BN ? N - n0 : BN;  // activation rows present in this tile
  const uint32_t row_bytes = static_cast<uint32_t>(K / 4);
  const int steps = static_cast<int>((K + 255) / 256);
  const int chunks = (steps + S - 1) / S;
  const uint32_t pitch = static_cast<uint32_t>(res_pitch(K, S));
  const int64_t present = (rows - o_tile + 15) / 16;
  const int msub = static_cast<int>(present < ms ? present : ms);
  // The tile's subtiles dealt to waves: round-robin (wave, wave + WAVES,
  // ...), or with PAIR the first two of each wave adjacent (2*wave and
  // 2*wave + 1, so that their outputs share 128-byte lines) and the rest
  // round-robin from 2*WAVES.  A wave's subtiles are increasing, so those
  // below msub are a prefix of its list.
  auto local_sub = [&](int idx) __attribute__((always_inline)) -> int {
    if constexpr (PAIR)
      return idx < 2 ? 2 * wave + idx : 2 * WAVES + wave + WAVES * (idx - 2);
    else
      return wave + WAVES * idx;
  };
  int mine;
  if constexpr (PAIR)
    mine = (2 * wave < msub) + (2 * wave + 1 < msub) +
           (msub > 2 * WAVES + wave ? (msub - 2 * WAVES - wave + WAVES - 1) / WAVES : 0);
  else
    mine = msub > wave ? (msub - wave + WAVES - 1) / WAVES : 0;
  const int groups = (mine + G - 1) / G;
  const int iters = groups * chunks;

  // Weights: one descriptor over the payload; lane (li, kb) of subtile
  // (o_tile + 16*(wave + WAVES*idx)) reads row li's bytes 64*kk + 16*kb..
  const __amdgpu_buffer_rsrc_t wbuf = buffer_of(packed + o_tile * row_bytes, static_cast<uint32_t>((rows - o_tile) * row_bytes));
  // PERM: each lane loads row lane/4, bytes 16*(lane%4) of the step (4
  // consecutive lanes read 64 contiguous bytes), and ds_bpermute moves the
  // dwords into MFMA lane order before use; otherwise lane (li, kb) loads
  // its MFMA operand directly (16 rows x 64 bytes per instruction).
  const uint32_t lane_off = PERM ? (lane >> 2) * row_bytes + 16 * (lane & 3) : li * row_bytes + 16 * kb;
  const int perm_addr = 4 * (4 * li + kb);
  auto permute_step = [&](const v4i (&src)[G][S], v4i (&dst)[G][S], int st, auto gsc) __attribute__((always_inline)) {
#pragma unroll
    for (int gi = 0; gi < decltype(gsc)::value; ++gi)
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[gi][st][e] = __builtin_amdgcn_ds_bpermute(perm_addr, src[gi][st][e]);
  };
  // Subtiles of a short group past this wave's last one read nothing (an
  // out-of-range offset: no memory traffic, and the same number of loads in
  // flight, so every wait below stays as it is).
  auto load_w = [&](int grp, int ch, v4i (&wv)[G][S]) __attribute__((always_inline)) {
    const int gs = grp + 1 < groups ? G : mine - grp * G;
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const uint32_t sub_off = static_cast<uint32_t>(16 * local_sub(grp * G + gi)) * row_bytes + 64 * S * ch;
#pragma unroll
      for (int st = 0; st < S; ++st)
        wv[gi][st] = __builtin_amdgcn_raw_buffer_load_b128(wbuf, gi < gs ? lane_off + sub_off + 64 * st : kOutOfRange,
                                                           0, 0);
    }
  };

  // Row sums of this lane's activation rows (clamped inside the tensor;
  // lanes past N never store), loaded before any prefetch so that waiting
  // for them (the accumulators start at -row_sum) never waits for the
  // prefetches; buffer loads keep their place (a plain read-only load may be
  // sunk to its first use, behind them).  The scales and the weight scale,
  // needed only by the epilogue, go out after the first weights
  // (load_scales).
  int32_t rsn[WN];
  {
    const __amdgpu_buffer_rsrc_t rbuf = buffer_of(row_sum + n0, static_cast<uint32_t>(4 * n_here));
#pragma unroll
    for (int n = 0; n < WN; ++n)
      rsn[n] = __builtin_amdgcn_raw_buffer_load_b32(rbuf, static_cast<uint32_t>(4 * (16 * n + li)), 0, 0);
  }
  float sn[WN], ws;
  constexpr int kScaleLoads = WN + 1;
  auto load_scales = [&]() __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t sbuf = buffer_of(act_scale + n0, static_cast<uint32_t>(4 * n_here));
#pragma unroll
    for (int n = 0; n < WN; ++n)
      sn[n] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(sbuf, static_cast<uint32_t>(4 * (16 * n + li)), 0, 0));
    ws = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(buffer_of(packed + rows * static_cast<int64_t>(row_bytes), 4),
                                                             0, 0, 0));
  };

  v4i wa[G][S], wb[G][S];
  const int k_pieces = static_cast<int>(K / 16);
  const __amdgpu_buffer_rsrc_t qbuf = buffer_of(qp + n0 * K, static_cast<uint32_t>(n_here * K));

  // Activation-tile pieces of one K-step for this wave: kRowsPerWave rows x
  // 16 pieces of 16 bytes, kPieceLanes per lane.
  constexpr int kStepPieces = kRowsPerWave * 16;
  constexpr int kPieceLanes = (kStepPieces + 63) / 64;
  auto step_goff = [&](int st, int p) __attribute__((always_inline)) -> uint32_t {
    const int pc = 64 * p + lane;
    const int r = wave * kRowsPerWave + pc / 16;
    const int c = 16 * st + pc % 16;  // 16-byte piece index within the padded row
    return pc < kStepPieces && c < k_pieces ? static_cast<uint32_t>(r * K + 16 * c) : kOutOfRange;
  };
  auto step_loff = [&](int st, int p) __attribute__((always_inline)) -> uint32_t {
    const int pc = 64 * p + lane;
    const int r = wave * kRowsPerWave + pc / 16;
    return static_cast<uint32_t>(r) * pitch + 16 * (16 * st + pc % 16);
  };

  v4i bst[SINGLE ? S : 1][kPieceLanes];
  if constexpr (SINGLE) {
    // Pipelined prologue: the loads of activation step st and of the first
    // group's weights for step st go out together, step by step, followed by
    // the next group's weights.  Below, the steps are written to LDS and
    // multiplied one at a time, so the first MFMAs wait for 256 columns of
    // the tile, not for all of it.
#pragma unroll
    for (int st = 0; st < S; ++st) {
#pragma unroll
      for (int p = 0; p < kPieceLanes; ++p) bst[st][p] = __builtin_amdgcn_raw_buffer_load_b128(qbuf, step_goff(st, p), 0, 0);
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        const uint32_t sub_off = static_cast<uint32_t>(16 * local_sub(gi)) * row_bytes;
        wa[gi][st] = __builtin_amdgcn_raw_buffer_load_b128(
            wbuf, gi < (groups > 1 ? G : mine) ? lane_off + sub_off + 64 * st : kOutOfRange, 0, 0);
      }
    }
    load_w(groups > 1 ? 1 : 0, 0, wb);
    load_scales();
  } else {
    // The whole activation tile goes from memory straight into LDS (buffer
    // loads with the LDS-direct bit: no registers, no wait per piece), issued
    // before the first group's weights so that the tile does not queue behind
    // them.  The tile is a run of 16-byte slots, pitch/16 per row; load
    // instruction i fills slots 64i..64i+63, lane l slot 64i+l, i.e. piece c
    // of row r for slot r*(pitch/16) + c.  Slots past K (the row's padding),
    // rows past N and slots past the tile read out of range, so they hold
    // zeros.  The LDS allocation is a whole number of these KiB runs.
    const int P = static_cast<int>(pitch / 16);
    const int insts = (BN * P + 63) / 64;
    int r = (64 * wave + lane) / P, c = (64 * wave + lane) % P;
    const int dr = (64 * WAVES) / P, dc = (64 * WAVES) % P;
    for (int i = wave; i < insts; i += WAVES) {
      const uint32_t off = r < n_here && c < k_pieces ? static_cast<uint32_t>(r * K + 16 * c) : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          qbuf, (__attribute__((address_space(3))) void *)(lds_res + 1024 * i), 16, off, 0, 0, 0);
      r += dr;
      c += dc;
      if (c >= P) {
        c -= P;
        ++r;
      }
    }
    load_w(0, 0, wa);
    load_scales();
    // This wave's tile loads are complete once at most the G*S weight loads
    // and the scale loads issued after them are outstanding; the barrier
    // then publishes every wave's part of the tile.
    constexpr int kWeightLoads = G * S + kScaleLoads;
    static_assert(kWeightLoads < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((kWeightLoads & 15) | ((kWeightLoads >> 4) << 14) | (7 << 4) | (15 << 8));
    __syncthreads();
  }

  // Output rows n0.. of this tile, ldy elements apart.
  const uint32_t out_bytes = static_cast<uint32_t>(((n_here - 1) * ldy + rows) * 4);
  const __amdgpu_buffer_rsrc_t ybuf = buffer_of(y + n0 * ldy, out_bytes);
  const __amdgpu_buffer_rsrc_t dbuf = buffer_of(DOT ? dot_out + n0 * ldy : nullptr, DOT ? out_bytes : 0);
  const int8_t *lb0 = lds_res + li * pitch + 64 * kb;

  // Bias of the outputs of a group (this lane's 4 consecutive output features
  // of each subtile), loaded unconditionally ahead of its MFMAs; without a
  // bias, or past the tensor, it reads 0 and is not added.
  const bool has_bias = bias != nullptr;
  const __amdgpu_buffer_rsrc_t bbuf = buffer_of(bias, has_bias ? static_cast<uint32_t>(4 * rows) : 0);
  v4i bv[G];
  auto load_bias = [&](int grp) __attribute__((always_inline)) {
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const uint32_t o = static_cast<uint32_t>(o_tile + 16 * static_cast<int64_t>(local_sub(grp * G + gi)) + 4 * kb);
      if constexpr (VEC4) {
        bv[gi] = __builtin_amdgcn_raw_buffer_load_b128(bbuf, 4 * o, 0, 0);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) bv[gi][r] = __builtin_amdgcn_raw_buffer_load_b32(bbuf, 4 * (o + r), 0, 0);
      }
    }
  };

  v4i acc[G][WN];
  // Stores of a finished group; subtiles past the group (gi >= gs) and
  // outputs past the tensor get an out-of-range offset instead of a branch.
  // Non-temporal where the wave has a single group: its stores all come
  // after its last MFMA and streaming them past the cache measured faster
  // (8960 x 1536 at N = 512: 10.7 against 12.4 us); with several groups,
  // ordinary stores, which the L2 absorbs and writes back while later
  // groups compute (N = 2048: 35.9 against 36.8 us).  The
  // accumulators start at -row_sum (init_acc), so each holds dot - row_sum
  // and the epilogue is one conversion and one multiply; with DOT the raw
  // dot is that plus the row sum.  The bias test is one wave-uniform branch
  // around the whole group.
  auto store_group = [&](int grp, int gs, auto biased, auto aux) __attribute__((always_inline)) {
    constexpr bool kBias = decltype(biased)::value;
    constexpr int kStreamStore = decltype(aux)::value;  // buffer-store cache policy bits
    float tn[WN];  // the epilogue's t = ws * s, formed here so that only the epilogue waits for the scales
#pragma unroll
    for (int n = 0; n < WN; ++n) tn[n] = ws * sn[n];
    // The values of subtile gi for activation block n, scaled and biased.
    auto values = [&](int gi, int n) __attribute__((always_inline)) {
      v4i yv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = static_cast<float>(acc[gi][n][r]) * tn[n];
        if constexpr (kBias) v = add_bias(v, __int_as_float(bv[gi][r]));
        yv[r] = __float_as_int(v);
      }
      return yv;
    };
    // PAIR: the first group's first two subtiles are adjacent (32 output
    // features).  Lane (li, kb) holds 4 features of each for activation row
    // li; the second subtile's values move to lane li ^ 8 (a DPP rotation by
    // 8 within each row of 16 lanes), and each store then writes 8 rows x
    // 128 contiguous bytes: rows 0-7 of the block from lanes li < 8 (first
    // subtile, their own values) and li >= 8 (second subtile, the moved
    // values), then rows 8-15 the other way round.  Whole lines, where
    // each 16 x 16 tile alone covers half lines.
    int g_first = 0;
    if constexpr (PAIR && VEC4 && G >= 2) {
      if (grp == 0 && gs >= 2) {
        g_first = 2;
        const bool lo = li < 8;
        const int64_t o0 = o_tile + 16 * static_cast<int64_t>(local_sub(0)) + 4 * kb;
        const int64_t oa = o0 + (lo ? 0 : 16), ob = o0 + (lo ? 16 : 0);
#pragma unroll
        for (int n = 0; n < WN; ++n) {
          const uint32_t ra = static_cast<uint32_t>((16 * n + (li & 7)) * ldy);
          const uint32_t rb = static_cast<uint32_t>((16 * n + 8 + (li & 7)) * ldy);
          const uint32_t offa = oa < rows ? 4 * (ra + static_cast<uint32_t>(oa)) : kOutOfRange;
          const uint32_t offb = ob < rows ? 4 * (rb + static_cast<uint32_t>(ob)) : kOutOfRange;
          const v4i y0 = values(0, n), y1 = values(1, n);
          v4i x1;
#pragma unroll
          for (int r = 0; r < 4; ++r) x1[r] = dpp_move<kDppRowRor8>(y1[r]);
          __builtin_amdgcn_raw_buffer_store_b128(lo ? y0 : x1, ybuf, offa, 0, kStreamStore);
          __builtin_amdgcn_raw_buffer_store_b128(lo ? x1 : y0, ybuf, offb, 0, kStreamStore);
          if constexpr (DOT) {
            const v4i rs4 = v4i{rsn[n], rsn[n], rsn[n], rsn[n]};
            const v4i d0 = acc[0][n] + rs4, d1 = acc[1][n] + rs4;
            v4i xd;
#pragma unroll
            for (int r = 0; r < 4; ++r) xd[r] = dpp_move<kDppRowRor8>(d1[r]);
            __builtin_amdgcn_raw_buffer_store_b128(lo ? d0 : xd, dbuf, offa, 0, kStreamStore);
            __builtin_amdgcn_raw_buffer_store_b128(lo ? xd : d0, dbuf, offb, 0, kStreamStore);
          }
        }
      }
    }
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      if (gi < g_first) continue;
      const bool sub_ok = gi < gs;
      const int64_t o = o_tile + 16 * static_cast<int64_t>(local_sub(grp * G + gi)) + 4 * kb;
#pragma unroll
      for (int n = 0; n < WN; ++n) {
        const uint32_t base = static_cast<uint32_t>((16 * n + li) * ldy);  // element offset of this lane's row
        const v4i yv = values(gi, n);
        if constexpr (VEC4) {
          const uint32_t off = sub_ok && o < rows ? 4 * (base + static_cast<uint32_t>(o)) : kOutOfRange;
          __builtin_amdgcn_raw_buffer_store_b128(yv, ybuf, off, 0, kStreamStore);
          if constexpr (DOT) {
            const v4i dv = acc[gi][n] + v4i{rsn[n], rsn[n], rsn[n], rsn[n]};
            __builtin_amdgcn_raw_buffer_store_b128(dv, dbuf, off, 0, kStreamStore);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t off = sub_ok && o + r < rows ? 4 * (base + static_cast<uint32_t>(o + r)) : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b32(yv[r], ybuf, off, 0, kStreamStore);
            if constexpr (DOT) __builtin_amdgcn_raw_buffer_store_b32(acc[gi][n][r] + rsn[n], dbuf, off, 0, kStreamStore);
          }
        }
      }
    }
  };
  auto epilogue_group = [&](int grp, int gs) __attribute__((always_inline)) {
    using kNonTemporal = std::integral_constant<int, 2>;
    using kCached = std::integral_constant<int, 0>;
    if (groups == 1) {
      if (has_bias) store_group(grp, gs, std::true_type{}, kNonTemporal{});
      else store_group(grp, gs, std::false_type{}, kNonTemporal{});
    } else {
      if (has_bias) store_group(grp, gs, std::true_type{}, kCached{});
      else store_group(grp, gs, std::false_type{}, kCached{});
    }
  };

  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
#pragma unroll
      for (int n = 0; n < WN; ++n) acc[gi][n] = v4i{-rsn[n], -rsn[n], -rsn[n], -rsn[n]};
  };

  // The MFMAs (and, with PERM, the permutes) of the group's gs subtiles only.
  auto mfma_group = [&](const v4i (&cur_in)[G][S], int gs, const int8_t *lb) __attribute__((always_inline)) {
    auto run = [&](auto gsc) __attribute__((always_inline)) {
      constexpr int GS = decltype(gsc)::value;
      v4i pm[G][S];
      if constexpr (PERM) {
#pragma unroll
        for (int st = 0; st < S; ++st) permute_step(cur_in, pm, st, gsc);
        __builtin_amdgcn_sched_barrier(0);  // all permutes in flight before the first use
      }
      const v4i(&cur)[G][S] = PERM ? pm : cur_in;
      res_mfma_chunk<GS, G, WN, S>(acc, cur, lb, pitch);
    };
    if (gs == G) {
      run(std::integral_constant<int, G>{});
    } else {
      switch (gs) {
        case 1: run(std::integral_constant<int, 1>{}); break;
        case 2: if constexpr (G > 2) run(std::integral_constant<int, 2>{}); break;
        case 3: if constexpr (G > 3) run(std::integral_constant<int, 3>{}); break;
        case 4: if constexpr (G > 4) run(std::integral_constant<int, 4>{}); break;
        default: break;
      }
    }
  };

  // One (group, chunk) item: prefetch the next item into `nxt` (past the last
  // item this re-reads the first one, harmlessly), then compute `cur`.  With
  // a single chunk (K <= 256*S) an item is a whole group and the body has no
  // branch around any memory operation.
  int grp = 0, ch = 0;
  auto item = [&](const v4i (&cur)[G][S], v4i (&nxt)[G][S]) __attribute__((always_inline)) {
    const int gs = grp + 1 < groups ? G : mine - grp * G;
    if constexpr (SINGLE) {
      load_bias(grp);
      load_w(grp + 1 < groups ? grp + 1 : 0, 0, nxt);
      zero_acc();
      mfma_group(cur, gs, lb0);
      epilogue_group(grp, gs);
      ++grp;
    } else {
      const int ngrp = ch + 1 < chunks ? grp : grp + 1;
      const int nch = ch + 1 < chunks ? ch + 1 : 0;
      load_bias(grp);
      load_w(ngrp < groups ? ngrp : 0, nch, nxt);
      if (ch == 0) zero_acc();
      mfma_group(cur, gs, lb0 + 256 * S * ch);
      if (ch == chunks - 1) epilogue_group(grp, gs);
      grp = ngrp;
      ch = nch;
    }
  };

  if constexpr (SINGLE) {
    // First group, step by step, interleaved with the activation copy; waves
    // without subtiles (gs0 == 0) still copy and meet every barrier.
    const int gs0 = groups > 1 ? G : mine;
    load_bias(0);
    zero_acc();
#pragma unroll
    for (int st = 0; st < S; ++st) {
#pragma unroll
      for (int p = 0; p < kPieceLanes; ++p)
        if (64 * p + lane < kStepPieces) *reinterpret_cast<v4i *>(lds_res + step_loff(st, p)) = bst[st][p];
      __syncthreads();
      auto run0 = [&](auto gsc) __attribute__((always_inline)) {
        constexpr int GS = decltype(gsc)::value;
        v4i pw[G][S];
        if constexpr (PERM) permute_step(wa, pw, st, gsc);
        const v4i(&w0)[G][S] = PERM ? pw : wa;
        res_mfma_step<GS, G, WN, S>(acc, w0, st, lb0, pitch);
      };
      if (gs0 == G) {
        run0(std::integral_constant<int, G>{});
      } else {
        switch (gs0) {
          case 1: run0(std::integral_constant<int, 1>{}); break;
          case 2: if constexpr (G > 2) run0(std::integral_constant<int, 2>{}); break;
          case 3: if constexpr (G > 3) run0(std::integral_constant<int, 3>{}); break;
          case 4: if constexpr (G > 4) run0(std::integral_constant<int, 4>{}); break;
          default: break;
        }
      }
    }
    epilogue_group(0, gs0);
    grp = 1;
    for (int g = 1; g < groups; g += 2) {
      item(wb, wa);
      if (g + 1 >= groups) break;
      item(wa, wb);
    }
  } else {
    for (int it = 0; it < iters; it += 2) {
      item(wa, wb);
      if (it + 1 >= iters) break;
      item(wb, wa);
    }
  }
}

// ---------------------------------------------------------------------------
// Weight-resident MFMA GEMM for the prefill shapes (K <= 256*CH, at most 8*G
// weight subtiles per block; positions past K are zeros on both sides).
// Same operand pairing as gemm_res_kernel; the schedule differs:
//  * loads go out chunk by chunk (256 positions), a window of three chunks
//    ahead of the MFMAs: the chunk's slice of the block's activation tile
//    (64 rows x 256 bytes, straight into LDS with LDS-direct buffer loads,
//    two of the chunk's sixteen 1 KiB runs per wave), then this wave's
//    weights for the chunk (G subtiles x 16 bytes per lane, row-contiguous:
//    lane l reads row l/4, bytes 16*(l%4) of the chunk).  Every group of 4
//    lanes reads 64 contiguous bytes, and the MFMAs of chunk c wait only for
//    chunk c (one barrier per chunk publishes the other waves' parts of the
//    tile).  A compute unit's vector-memory path takes about one 1 KiB load
//    every 30 cycles, so issuing every load up front held each wave in its
//    load instructions for microseconds before its first MFMA;
//  * the weights stay in registers; each chunk is moved into MFMA lane order
//    (ds_bpermute) during the chunk before it, and its four 64-position steps
//    are unpacked one step ahead of their MFMAs;
//  * the B operands of the next step are read from LDS while the current
//    step's MFMAs run (two register sets), and sched_group_barrier keeps the
//    VALU and LDS work between the MFMAs;
//  * the accumulators start at -row_sum, so the epilogue is one conversion
//    and one multiply (plus the bias add when there is a bias);
//  * wave w holds subtiles 2w and 2w+1 (then 16+w, 24+w, ...): the two
//    subtiles' stores fill whole 128-byte lines of y.
// LDS layout of the activation tile: chunk-major, 16 KiB per chunk; piece p
// (16 bytes) of row r in chunk c at 16 * (1024c + 16r + (p ^ (r % 16))).  A
// B read (16 lanes: rows 16n..16n+15 at one piece) then touches 16 different
// bank groups, and an LDS-direct run (64 consecutive slots: 4 rows x 16
// pieces) fetches 64 contiguous bytes per 4 consecutive lanes.

// The subtile (block-relative) that slot g of wave w (of WAVES) holds: one
// per wave with G = 1; otherwise adjacent pairs 2w, 2w+1 for the first
// WAVES/2 waves (8 waves: all of them), then one more per wave.
template <int G, int WAVES>
__device__ __forceinline__ int wk_subtile(int w, int g) {
  if constexpr (G == 1) return w;
  if constexpr (WAVES == 8) return g < 2 ? 2 * w + g : 16 + 8 * (g - 2) + w;
  // 12 waves, G = 2: waves 0..5 hold 2w, 2w+1; waves 6..11 hold w+6, w+12.
  return g == 0 ? (w < 6 ? 2 * w : w + 6) : (w < 6 ? 2 * w + 1 : w + 12);
}

constexpr int kWkChunkBytes = 64 * 256;  // one chunk of the 64-row activation tile
constexpr int kWkStore = 2;              // output stores non-temporal (not read again by this kernel)

// One LDS-direct buffer load: lane l's 16 bytes at buffer offset `off` go to
// LDS byte lds + 16*l (out-of-range offsets write zeros).
__device__ __forceinline__ void lds_direct16(__amdgpu_buffer_rsrc_t rsrc, int8_t *lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)lds, 16, off, 0, 0, 0);
}

template <int G, int CH, int WAVES, bool VEC4, bool DOT>
__global__ void __launch_bounds__(64 * WAVES)
gemm_wk_kernel(int tiles_m, int ms, const uint8_t *__restrict__ packed, int64_t rows, int K,
               const int8_t *__restrict__ qp, int64_t N, const int32_t *__restrict__ row_sum,
               const float *__restrict__ act_scale, const float *__restrict__ bias, float *__restrict__ y,
               int32_t *__restrict__ dot_out, int64_t ldy) {
  // Argument order: the arguments up to row_sum are preloaded into scalar
  // registers at launch, and they are all that the loads issued before the
  // first chunks need; the rest come from a scalar load that completes while
  // the first chunks stream in.
  extern __shared__ __attribute__((aligned(16))) int8_t lds_wk[];
  constexpr int WN = 4, BN = 64;
  const int KB = K / 4;           // packed bytes per row
  const int k_pieces = K / 16;    // 16-byte activation pieces per row
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, kb = lane >> 4;
  const int tile_m = static_cast<int>(blockIdx.x) % tiles_m, tile_n = static_cast<int>(blockIdx.x) / tiles_m;
  const int64_t o_tile = static_cast<int64_t>(tile_m) * ms * 16;
  const int64_t n0 = static_cast<int64_t>(tile_n) * BN;
  const int n_here = static_cast<int>(N - n0 < BN ? N - n0 : BN);
  const int64_t present = (rows - o_tile + 15) / 16;
  const int msub = static_cast<int>(present < ms ? present : ms);
  int mine = 0;
#pragma unroll
  for (int g = 0; g < G; ++g) mine += wk_subtile<G, WAVES>(wave, g) < msub ? 1 : 0;

  const __amdgpu_buffer_rsrc_t qbuf = buffer_of(qp + n0 * K, static_cast<uint32_t>(n_here * K));
  const __amdgpu_buffer_rsrc_t wbuf =
      buffer_of(packed + o_tile * KB, static_cast<uint32_t>((rows - o_tile) * KB));
  const int perm_addr = 4 * (4 * li + kb);
  // LDS-direct run j of chunk c fills slots 1024c + 64j + lane: row 4j +
  // lane/16, piece (lane % 16) ^ (row % 16) of the chunk.
  const int dma_r0 = lane >> 4;
  auto dma_off = [&](int c, int j) -> uint32_t {
    const int r = 4 * j + dma_r0;
    const int p = 16 * c + ((lane & 15) ^ (r & 15));
    return r < n_here && p < k_pieces ? static_cast<uint32_t>(r * K + 16 * p) : kOutOfRange;
  };
  // LDS byte of the B operand of column block n, chunk c, step d for this
  // lane: row 16n + li, piece 4kb + d of the chunk.
  uint32_t bbase[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) bbase[d] = static_cast<uint32_t>(256 * li + 16 * ((4 * kb + d) ^ li));

  auto run = [&](auto gsc) {
    constexpr int GS = decltype(gsc)::value;
    constexpr int STEPS = 4 * CH;
    // Loads per chunk: this wave's tile runs (runs wave, wave + WAVES, ... of
    // the chunk's 16), then its GS weight chunks.
    const int nruns = (16 - wave + WAVES - 1) / WAVES;
    const int kPerChunk = nruns + GS;
    // The row sums the accumulators start from: small loads, issued before
    // the big ones so that waiting for them never waits for the tile or the
    // weights.  The epilogue constants (scales, weight scale, biases) go out
    // after the first chunks (load_small), whose loads need only the
    // preloaded arguments.
    float tn[WN], ws = 0.0f;
    int32_t rsn[WN];
    v4i bv[GS > 0 ? GS : 1];
    if constexpr (GS > 0) {
      const __amdgpu_buffer_rsrc_t rbuf = buffer_of(row_sum + n0, static_cast<uint32_t>(4 * n_here));
#pragma unroll
      for (int n = 0; n < WN; ++n) rsn[n] = __builtin_amdgcn_raw_buffer_load_b32(rbuf, 4 * (16 * n + li), 0, 0);
    }
    constexpr int kSmall = GS > 0 ? WN + 1 + GS : 0;  // loads of load_small
    auto load_small = [&]() {
      if constexpr (GS > 0) {
        ws = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            buffer_of(packed + rows * static_cast<int64_t>(KB), 4), 0, 0, 0));
        const __amdgpu_buffer_rsrc_t sbuf = buffer_of(act_scale + n0, static_cast<uint32_t>(4 * n_here));
#pragma unroll
        for (int n = 0; n < WN; ++n)
          tn[n] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(sbuf, 4 * (16 * n + li), 0, 0));
        const bool with_bias = bias != nullptr;
        const __amdgpu_buffer_rsrc_t bbuf =
            buffer_of(with_bias ? bias + o_tile : nullptr, with_bias ? static_cast<uint32_t>(4 * (rows - o_tile)) : 0u);
#pragma unroll
        for (int g = 0; g < GS; ++g)
          bv[g] = __builtin_amdgcn_raw_buffer_load_b128(bbuf, 4 * (16 * wk_subtile<G, WAVES>(wave, g) + 4 * kb), 0, 0);
      }
    };
    // Loads of chunk c: its two tile runs, then this wave's GS weight chunks.
    // Chunks 0..PD-1 are issued at the start, chunk c+PD during the first
    // step of chunk c: the memory path accepts one 1 KiB load about every 16
    // cycles per compute unit, so issuing everything up front would hold
    // every wave in its load instructions for microseconds before its first
    // MFMA.
    constexpr int PD = CH < 3 ? CH : 3;
    v4i wr[CH][GS > 0 ? GS : 1];
    uint32_t woff[GS > 0 ? GS : 1];
#pragma unroll
    for (int g = 0; g < GS; ++g)
      woff[g] = static_cast<uint32_t>((16 * wk_subtile<G, WAVES>(wave, g) + (lane >> 2)) * KB + 16 * (lane & 3));
    auto issue_chunk = [&](int c) {
#pragma unroll
      for (int j = wave; j < 16; j += WAVES) lds_direct16(qbuf, lds_wk + c * kWkChunkBytes + 1024 * j, dma_off(c, j));
      const bool piece_ok = 4 * c + (lane & 3) < K / 64;
#pragma unroll
      for (int g = 0; g < GS; ++g)
        wr[c][g] = __builtin_amdgcn_raw_buffer_load_b128(wbuf, piece_ok ? woff[g] + 64 * c : kOutOfRange, 0, 0);
    };
#pragma unroll
    for (int c = 0; c < PD; ++c) issue_chunk(c);
    load_small();
    // Output descriptors and the bias test from the arguments that are not
    // preloaded, after the first loads.
    const uint32_t out_bytes = static_cast<uint32_t>((static_cast<int64_t>(n_here - 1) * ldy + rows) * 4);
    const __amdgpu_buffer_rsrc_t ybuf = buffer_of(y + n0 * ldy, out_bytes);
    const __amdgpu_buffer_rsrc_t dbuf = buffer_of(DOT ? dot_out + n0 * ldy : nullptr, DOT ? out_bytes : 0);
    const bool has_bias = bias != nullptr;
    // Chunk c of the tile is in LDS once this wave has at most the loads
    // issued after its chunk-c runs outstanding (the chunk's GS weight loads,
    // those of chunks c+1..last, the last chunk issued so far, and, for the
    // first PD chunks, the kSmall loads issued after them), and the barrier
    // has seen every wave get there.
    auto tile_wait = [&](int c, int last) {
      const int after = GS + (last - c) * kPerChunk + (c < PD ? kSmall : 0);
      switch (after) {
#define I2S_WK_WAIT(n) case n: __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8)); break;
        I2S_WK_WAIT(0) I2S_WK_WAIT(1) I2S_WK_WAIT(2) I2S_WK_WAIT(3) I2S_WK_WAIT(4) I2S_WK_WAIT(5) I2S_WK_WAIT(6)
        I2S_WK_WAIT(7) I2S_WK_WAIT(8) I2S_WK_WAIT(9) I2S_WK_WAIT(10) I2S_WK_WAIT(11) I2S_WK_WAIT(12) I2S_WK_WAIT(13)
        I2S_WK_WAIT(14) I2S_WK_WAIT(15) I2S_WK_WAIT(16) I2S_WK_WAIT(17) I2S_WK_WAIT(18) I2S_WK_WAIT(19) I2S_WK_WAIT(20)
        I2S_WK_WAIT(21) I2S_WK_WAIT(22) I2S_WK_WAIT(23) I2S_WK_WAIT(24) I2S_WK_WAIT(25) I2S_WK_WAIT(26) I2S_WK_WAIT(27)
        I2S_WK_WAIT(28) I2S_WK_WAIT(29) I2S_WK_WAIT(30) I2S_WK_WAIT(31) I2S_WK_WAIT(32) I2S_WK_WAIT(33) I2S_WK_WAIT(34)
        I2S_WK_WAIT(35) I2S_WK_WAIT(36) I2S_WK_WAIT(37) I2S_WK_WAIT(38) I2S_WK_WAIT(39) I2S_WK_WAIT(40) I2S_WK_WAIT(41)
        I2S_WK_WAIT(42) I2S_WK_WAIT(43) I2S_WK_WAIT(44) I2S_WK_WAIT(45) I2S_WK_WAIT(46) I2S_WK_WAIT(47) I2S_WK_WAIT(48)
        I2S_WK_WAIT(49) I2S_WK_WAIT(50) I2S_WK_WAIT(51) I2S_WK_WAIT(52) I2S_WK_WAIT(53) I2S_WK_WAIT(54) I2S_WK_WAIT(55)
        I2S_WK_WAIT(56) I2S_WK_WAIT(57) I2S_WK_WAIT(58) I2S_WK_WAIT(59) I2S_WK_WAIT(60) I2S_WK_WAIT(61) I2S_WK_WAIT(62)
#undef I2S_WK_WAIT
        default: __builtin_amdgcn_s_waitcnt(0); break;
      }
      __builtin_amdgcn_s_barrier();
    };

    if constexpr (GS == 0) {
      // No subtiles: this wave only loads its part of the tile and meets
      // every barrier of the waves that compute.
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        if (c >= 1 && c - 1 + PD < CH) issue_chunk(c - 1 + PD);
        tile_wait(c, c == 0 ? PD - 1 : (c - 1 + PD < CH ? c - 1 + PD : CH - 1));
      }
    } else {
      v4i acc[GS][WN], a[2][GS], b[2][WN];
      auto bread = [&](int n, int c, int d) -> v4i {
        return *reinterpret_cast<const v4i *>(lds_wk + bbase[d] + c * kWkChunkBytes + n * 4096);
      };
      tile_wait(0, PD - 1);
#pragma unroll
      for (int g = 0; g < GS; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) wr[0][g][e] = __builtin_amdgcn_ds_bpermute(perm_addr, wr[0][g][e]);
#pragma unroll
      for (int n = 0; n < WN; ++n) b[0][n] = bread(n, 0, 0);
#pragma unroll
      for (int g = 0; g < GS; ++g) a[0][g] = unpack_codes(static_cast<uint32_t>(wr[0][g][0]));
#pragma unroll
      for (int g = 0; g < GS; ++g)
#pragma unroll
        for (int n = 0; n < WN; ++n) acc[g][n] = v4i{-rsn[n], -rsn[n], -rsn[n], -rsn[n]};
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < STEPS; ++t) {
        const int cur = t & 1, nxt = cur ^ 1;
        const int c = t >> 2, d = t & 3;
        // The loads of chunk c+PD go out in the first step of chunk c.
        if (d == 0 && c + PD < CH) issue_chunk(c + PD);
        // Before the first B read of the next chunk, that chunk of the tile
        // must be complete.
        if (d == 3 && c + 1 < CH) {
          tile_wait(c + 1, c + PD < CH ? c + PD : CH - 1);
          __builtin_amdgcn_sched_barrier(0);
        }
        // Next chunk's permutes, a quarter per step.
        if (c + 1 < CH) {
#pragma unroll
          for (int g = 0; g < GS; ++g) wr[c + 1][g][d] = __builtin_amdgcn_ds_bpermute(perm_addr, wr[c + 1][g][d]);
        }
        if (t + 1 < STEPS) {
          const int c1 = (t + 1) >> 2, d1 = (t + 1) & 3;
#pragma unroll
          for (int n = 0; n < WN; ++n) b[nxt][n] = bread(n, c1, d1);
#pragma unroll
          for (int g = 0; g < GS; ++g) a[nxt][g] = unpack_codes(static_cast<uint32_t>(wr[c1][g][d1]));
        }
#pragma unroll
        for (int g = 0; g < GS; ++g)
#pragma unroll
          for (int n = 0; n < WN; ++n)
            acc[g][n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[cur][g], b[cur][n], acc[g][n], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < GS * WN; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x080, 1, 0);  // one LDS operation (read or permute)
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // two VALU
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // Outputs: activation row n0 + 16n + li, output features
      // o_tile + 16*subtile + 4kb .. +3.
      float t_n[WN];
#pragma unroll
      for (int n = 0; n < WN; ++n) t_n[n] = ws * tn[n];
      auto store = [&](auto biased) {
        constexpr bool kBias = decltype(biased)::value;
#pragma unroll
        for (int g = 0; g < GS; ++g) {
          const int64_t o = o_tile + 16 * static_cast<int64_t>(wk_subtile<G, WAVES>(wave, g)) + 4 * kb;
#pragma unroll
          for (int n = 0; n < WN; ++n) {
            const uint32_t base = static_cast<uint32_t>((16 * n + li) * ldy);
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              v[r] = static_cast<float>(acc[g][n][r]) * t_n[n];
              if constexpr (kBias) v[r] = add_bias(v[r], __int_as_float(bv[g][r]));
            }
            if constexpr (VEC4) {
              const uint32_t off = o < rows ? 4 * (base + static_cast<uint32_t>(o)) : kOutOfRange;
              const v4i yv = {__float_as_int(v[0]), __float_as_int(v[1]), __float_as_int(v[2]), __float_as_int(v[3])};
              __builtin_amdgcn_raw_buffer_store_b128(yv, ybuf, off, 0, kWkStore);
              if constexpr (DOT)
                __builtin_amdgcn_raw_buffer_store_b128(acc[g][n] + v4i{rsn[n], rsn[n], rsn[n], rsn[n]}, dbuf, off, 0, kWkStore);
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const uint32_t off = o + r < rows ? 4 * (base + static_cast<uint32_t>(o + r)) : kOutOfRange;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(v[r]), ybuf, off, 0, kWkStore);
                if constexpr (DOT) __builtin_amdgcn_raw_buffer_store_b32(acc[g][n][r] + rsn[n], dbuf, off, 0, kWkStore);
              }
            }
          }
        }
      };
      if (has_bias)
        store(std::true_type{});
      else
        store(std::false_type{});
    }
  };
  switch (mine) {
    case 0: run(std::integral_constant<int, 0>{}); break;
    case 1: run(std::integral_constant<int, 1>{}); break;
    case 2: if constexpr (G >= 2) run(std::integral_constant<int, 2>{}); break;
    case 3: if constexpr (G >= 3) run(std::integral_constant<int, 3>{}); break;
    default: break;
  }
}

// ---------------------------------------------------------------------------
// Pipelined GEMM for K <= 256*SM (the prefill shapes), same MFMA operand
// mapping as above.
//
// A workgroup owns BN = 16*WN activation rows and ms 16-row weight subtiles,
// dealt to its WAVES waves round-robin.  A wave works through its subtiles G
// at a time, each group over the whole K, and stores every finished group at
// once.  The activation tile (BN rows x K, zero past K and past N) stays in
// LDS for the whole kernel; it is written step by step (256 positions)
// during the first group, whose MFMAs start on the first step's data rather
// than on the whole tile.  Every load of the first group -- activation pieces
// and weights, step by step -- is issued at the start.
//
// Memory access shapes follow the rule that a group of 4 consecutive lanes
// should touch 64 contiguous bytes (measured on MI355X: global loads that
// break it run about 2.5x slower out of L2, LDS reads about 1.7x slower):
//  * weights are loaded row-contiguous -- lane l reads 16 bytes of row l/4 of
//    the subtile at byte 16*(l%4) of the step -- and moved into MFMA lane
//    order (lane i + 16*kb holds row i, bytes 16*kb..) by ds_bpermute;
//  * the LDS activation tile interleaves 4 rows at 16-byte granularity:
//    piece q (16 bytes, along K) of row r sits at
//    (r/4)*4*pitch + 64*q + 16*(r%4), so the 16 lanes that read one column
//    piece of 16 rows read 4 runs of 64 contiguous bytes.
// Blocks dispatched to one XCD walk K from different steps (rotation by
// blockIdx/8), so blocks sharing weight rows or an activation tile do not all
// miss the XCD's L2 on the same lines at once; integer sums do not depend on
// the order of their terms.  As in gemm_res_kernel, every global access is an
// unconditional buffer access, so each wait is for exactly the loads it needs.
// Two weight register sets: the next group's weights load during the current
// group's MFMAs.

template <int G, int WN, int GS = G>
__device__ __forceinline__ void pipe_mfma_step(v4i (&acc)[G][WN], const v4i (&w)[G], const int8_t *lb,
                                               uint32_t group_stride, int perm) {
  v4i a4[G];
#pragma unroll
  for (int j = 0; j < GS; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) a4[j][e] = __builtin_amdgcn_ds_bpermute(perm, w[j][e]);
  // All permutes in flight before the first use (else they go out one by one).
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    v4i b[WN];
#pragma unroll
    for (int n = 0; n < WN; ++n) b[n] = *reinterpret_cast<const v4i *>(lb + 4 * n * group_stride + 64 * d);
#pragma unroll
    for (int j = 0; j < GS; ++j) {
      const v4i a = unpack_codes(static_cast<uint32_t>(a4[j][d]));
#pragma unroll
      for (int n = 0; n < WN; ++n) acc[j][n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b[n], acc[j][n], 0, 0, 0);
    }
  }
}

template <int G, int WN, int WAVES, int SM, bool VEC4, bool DOT>
__global__ void __launch_bounds__(64 * WAVES)
gemm_pipe_kernel(const uint8_t *__restrict__ packed, int64_t rows, int64_t K,
                 const int8_t *__restrict__ qp, int64_t N, const float *__restrict__ act_scale,
                 const int32_t *__restrict__ row_sum, float *__restrict__ y,
                 int32_t *__restrict__ dot_out, const float *__restrict__ bias, int64_t ldy, int64_t tiles_m,
                 int ms) {
  extern __shared__ __attribute__((aligned(16))) int8_t lds_pipe[];
  constexpr int BN = 16 * WN;
  constexpr int kThreads = 64 * WAVES;
  constexpr int kStepPieces = BN * 16;  // 16-byte activation pieces per step
  constexpr int kPieceLanes = (kStepPieces + kThreads - 1) / kThreads;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, kb = lane >> 4;
  const int64_t tile_m = blockIdx.x % tiles_m, tile_n = blockIdx.x / tiles_m;
  const int64_t o_tile = tile_m * ms * 16;
  const int64_t n0 = tile_n * BN;
  const int64_t n_here = N - n0 < BN ? N - n0 : BN;
  const uint32_t row_bytes = static_cast<uint32_t>(K / 4);
  const int steps = static_cast<int>((K + 255) / 256);
  const int k_pieces = static_cast<int>(K / 16);
  const uint32_t pitch = static_cast<uint32_t>(256 * steps + 16);
  const uint32_t group_stride = 4 * pitch;           // 4 interleaved rows
  const int64_t present = (rows - o_tile + 15) / 16;
  const int msub = static_cast<int>(present < ms ? present : ms);
  const int mine = msub > wave ? (msub - wave + WAVES - 1) / WAVES : 0;  // subtiles wave, wave+WAVES, ...
  const int groups = (mine + G - 1) / G;
  const int rot = static_cast<int>((blockIdx.x / 8) % steps);
  auto phys = [&](int st) -> int { return st + rot < steps ? st + rot : st + rot - steps; };

  // Weights, row-contiguous: lane l reads row 16*s + l/4 of subtile s, bytes
  // 64*step + 16*(l%4); subtiles past the wave's share read nothing (0).
  // (24-bit multiplies: operands below 2^24, products below 2^31, checked
  // on the host.)
  const __amdgpu_buffer_rsrc_t wbuf =
      buffer_of(packed + o_tile * row_bytes, static_cast<uint32_t>((rows - o_tile) * row_bytes));
  const uint32_t lane_off = __umul24(lane >> 2, row_bytes) + 16 * (lane & 3);
  const int perm = 4 * (4 * li + kb);  // ds_bpermute source lane (bytes) of MFMA lane (li, kb)
  auto w_off = [&](int grp, int j, int st) -> uint32_t {
    const int t = G * grp + j;
    return t < mine && st < steps ? __umul24(16 * (wave + WAVES * t), row_bytes) + lane_off + 64 * phys(st)
                                  : kOutOfRange;
  };
  auto load_w = [&](int grp, v4i (&wv)[G][SM]) {
#pragma unroll
    for (int st = 0; st < SM; ++st)
#pragma unroll
      for (int j = 0; j < G; ++j) wv[j][st] = __builtin_amdgcn_raw_buffer_load_b128(wbuf, w_off(grp, j, st), 0, 0);
  };

  // Activation pieces of step st: piece pc = tid + kThreads*p is row pc/16,
  // piece 16*step + pc%16 along K; pieces past K or past N read as zero.
  const __amdgpu_buffer_rsrc_t qbuf = buffer_of(qp + n0 * K, static_cast<uint32_t>(n_here * K));
  auto act_goff = [&](int st, int p) -> uint32_t {
    const int pc = tid + kThreads * p;
    const int c = 16 * phys(st) + (pc & 15);
    return pc < kStepPieces && c < k_pieces ? __umul24(pc >> 4, static_cast<uint32_t>(K)) + 16 * c : kOutOfRange;
  };
  auto act_loff = [&](int st, int p) -> uint32_t {
    const int pc = tid + kThreads * p;
    const int r = pc >> 4;
    return static_cast<uint32_t>(r >> 2) * group_stride + 64 * (16 * phys(st) + (pc & 15)) + 16 * (r & 3);
  };

  v4i wa[G][SM], wb[G][SM];
  v4i bst[SM][kPieceLanes];
#pragma unroll
  for (int st = 0; st < SM; ++st) {
#pragma unroll
    for (int p = 0; p < kPieceLanes; ++p) bst[st][p] = __builtin_amdgcn_raw_buffer_load_b128(qbuf, act_goff(st, p), 0, 0);
#pragma unroll
    for (int j = 0; j < G; ++j) wa[j][st] = __builtin_amdgcn_raw_buffer_load_b128(wbuf, w_off(0, j, st), 0, 0);
  }
  load_w(1, wb);
  // Epilogue constants last: the first group's epilogue needs them only after
  // all of its steps.
  const __amdgpu_buffer_rsrc_t cbuf = buffer_of(packed + rows * static_cast<int64_t>(row_bytes), 4);
  const __amdgpu_buffer_rsrc_t sbuf = buffer_of(act_scale + n0, static_cast<uint32_t>(4 * n_here));
  const __amdgpu_buffer_rsrc_t rbuf = buffer_of(row_sum + n0, static_cast<uint32_t>(4 * n_here));
  const float ws = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(cbuf, 0, 0, 0));
  float sn[WN];
  int32_t rsn[WN];
#pragma unroll
  for (int n = 0; n < WN; ++n) {
    const uint32_t off = static_cast<uint32_t>(4 * (16 * n + li));  // past N: reads 0, never stored
    sn[n] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(sbuf, off, 0, 0));
    rsn[n] = __builtin_amdgcn_raw_buffer_load_b32(rbuf, off, 0, 0);
  }
  // Bias of a group's outputs (this lane's 4 consecutive output features of
  // each subtile): reads 0 without a bias or past the tensor, and is then
  // not added.
  const bool has_bias = bias != nullptr;
  const __amdgpu_buffer_rsrc_t bbuf = buffer_of(bias, has_bias ? static_cast<uint32_t>(4 * rows) : 0);
  v4i bv[G];
  auto load_bias = [&](int grp) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const uint32_t o = static_cast<uint32_t>(o_tile + 16 * static_cast<int64_t>(wave + WAVES * (G * grp + j)) + 4 * kb);
      if constexpr (VEC4) {
        bv[j] = __builtin_amdgcn_raw_buffer_load_b128(bbuf, 4 * o, 0, 0);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) bv[j][r] = __builtin_amdgcn_raw_buffer_load_b32(bbuf, 4 * (o + r), 0, 0);
      }
    }
  };
  load_bias(0);
  // Keep every load above ahead of the first wait below.
  __builtin_amdgcn_sched_barrier(0);

  // Output rows n0.. of this tile, ldy elements apart.
  const uint32_t out_bytes = static_cast<uint32_t>(((n_here - 1) * ldy + rows) * 4);
  const __amdgpu_buffer_rsrc_t ybuf = buffer_of(y + n0 * ldy, out_bytes);
  const __amdgpu_buffer_rsrc_t dbuf = buffer_of(DOT ? dot_out + n0 * ldy : nullptr, DOT ? out_bytes : 0);
  // This lane's B base: row li of column block 0, piece 4*kb of step 0.
  const int8_t *lb0 = lds_pipe + (li >> 2) * group_stride + 256 * kb + 16 * (li & 3);

  float tn[WN];
#pragma unroll
  for (int n = 0; n < WN; ++n) tn[n] = ws * sn[n];

  v4i acc[G][WN];
  auto zero_acc = [&]() {
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int n = 0; n < WN; ++n) acc[j][n] = v4i{0, 0, 0, 0};
  };

  // Non-temporal stores of a finished group; subtiles past the wave's share
  // and outputs past the tensor get an out-of-range offset instead of a
  // branch.  The stored values sit in registers of their own, kept allocated
  // to the end, so that the MFMAs of the next group never wait for this
  // group's stores to release a register.
  constexpr int kStreamStore = 2;
  v4i yst[G][WN] = {};
  v4i dst[G][DOT ? WN : 1] = {};
  auto epilogue_group = [&](int grp) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int t = G * grp + j;
      const int64_t o = o_tile + 16 * static_cast<int64_t>(wave + WAVES * t) + 4 * kb;
      const bool ok = t < mine;
#pragma unroll
      for (int n = 0; n < WN; ++n) {
        const uint32_t base = static_cast<uint32_t>((16 * n + li) * ldy);  // element offset of this lane's row
        v4i &yv = yst[j][n];
        v4i &dv = dst[j][DOT ? n : 0];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = epilogue(acc[j][n][r], rsn[n], tn[n]);
          yv[r] = __float_as_int(has_bias ? add_bias(v, __int_as_float(bv[j][r])) : v);
        }
        if constexpr (DOT) dv = acc[j][n];
        if constexpr (VEC4) {
          const uint32_t off = ok && o < rows ? 4 * (base + static_cast<uint32_t>(o)) : kOutOfRange;
          __builtin_amdgcn_raw_buffer_store_b128(yv, ybuf, off, 0, kStreamStore);
          if constexpr (DOT) __builtin_amdgcn_raw_buffer_store_b128(dv, dbuf, off, 0, kStreamStore);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t off = ok && o + r < rows ? 4 * (base + static_cast<uint32_t>(o + r)) : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b32(yv[r], ybuf, off, 0, kStreamStore);
            if constexpr (DOT) __builtin_amdgcn_raw_buffer_store_b32(dv[r], dbuf, off, 0, kStreamStore);
          }
        }
      }
    }
  };

  auto step_ptr = [&](int st) { return lb0 + 1024 * phys(st); };
  // One step's permutes and MFMAs for the gs subtiles a group has (a short
  // last group runs none for the subtiles it lacks).
  auto mfma_step_gs = [&](const v4i (&w)[G], const int8_t *lb, int gs) {
    if (gs >= G) {
      pipe_mfma_step<G, WN>(acc, w, lb, group_stride, perm);
    } else {
      switch (gs) {
        case 1: pipe_mfma_step<G, WN, 1>(acc, w, lb, group_stride, perm); break;
        case 2: if constexpr (G > 2) pipe_mfma_step<G, WN, 2>(acc, w, lb, group_stride, perm); break;
        case 3: if constexpr (G > 3) pipe_mfma_step<G, WN, 3>(acc, w, lb, group_stride, perm); break;
        default: break;
      }
    }
  };
  auto group_size = [&](int grp) { return mine - G * grp < G ? mine - G * grp : G; };
  auto mfma_group = [&](const v4i (&cur)[G][SM], int grp) {
    const int gs = group_size(grp);
#pragma unroll
    for (int st = 0; st < SM; ++st)
      if (st < steps) {
        v4i w[G];
#pragma unroll
        for (int j = 0; j < G; ++j) w[j] = cur[j][st];
        mfma_step_gs(w, step_ptr(st), gs);
      }
  };

  // First group, step by step, interleaved with the activation tile's LDS
  // writes; every wave meets every barrier, with or without subtiles.
  zero_acc();
#pragma unroll
  for (int st = 0; st < SM; ++st) {
    if (st < steps) {
#pragma unroll
      for (int p = 0; p < kPieceLanes; ++p)
        if (tid + kThreads * p < kStepPieces) *reinterpret_cast<v4i *>(lds_pipe + act_loff(st, p)) = bst[st][p];
      __syncthreads();
      v4i w[G];
#pragma unroll
      for (int j = 0; j < G; ++j) w[j] = wa[j][st];
      mfma_step_gs(w, step_ptr(st), group_size(0));
    }
  }

  // Each group's MFMAs are followed by the loads of the group two ahead, into
  // the register set they have just finished with, then its stores; a
  // group's bias loads ahead of its MFMAs.
  load_w(2, wa);
  __builtin_amdgcn_sched_barrier(0);
  epilogue_group(0);
  for (int g = 1; g < groups; g += 2) {
    load_bias(g);
    zero_acc();
    mfma_group(wb, g);
    load_w(g + 2, wb);
    __builtin_amdgcn_sched_barrier(0);
    epilogue_group(g);
    if (g + 1 >= groups) break;
    load_bias(g + 1);
    zero_acc();
    mfma_group(wa, g + 1);
    load_w(g + 3, wa);
    __builtin_amdgcn_sched_barrier(0);
    epilogue_group(g + 1);
  }
  // Keep the store registers allocated up to here (see above).
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int n = 0; n < WN; ++n) {
      asm volatile("" ::"v"(yst[j][n]));
      if constexpr (DOT) asm volatile("" ::"v"(dst[j][n]));
    }
}

// ---------------------------------------------------------------------------
// Skinny int8-MFMA contraction for 1 <= N <= 64 activation rows (the small
// batches).  At N = 8 the v_dot4 GEMV spends most of its time on VALU work
// (one v_dot4 per 4 codes per activation row); one v_mfma_i32_16x16x64_i8
// does the same for 16 weight rows x 64 positions x 16 activation rows.
//
// One workgroup per 16-row weight subtile; its W waves take the K-steps (256
// positions) round-robin, so every wave streams an equal share of the
// subtile's weights, and their int32 partial dots are summed through LDS.
// The weights go in as operand A (lane i + 16*kb: row i; loaded
// row-contiguous -- lane l reads row l/4, bytes 16*(l%4) of the step -- and
// moved into that order by ds_bpermute), the activations as operand B, NB
// blocks of 16 rows (lane j + 16*kb of block b: activation row 16*b + j,
// zero for rows >= N) read from the workspace's MFMA-tiled copy, one
// contiguous KiB per operand when the rows start on a 16-row block (a
// batch's rows may not; each lane's address is computed on its own): each
// unpacked weight operand feeds NB MFMAs.  A wave issues the loads of SPW steps at a time, into one of two
// register sets, before computing the previous SPW steps.  After the LDS
// reduction, wave b writes the outputs of activation block b.

template <int W, int NB, int SPW, bool VEC4, bool DOT>
__global__ void __launch_bounds__(64 * W)
gemv_mfma_kernel(const uint8_t *__restrict__ packed, const int8_t *__restrict__ qt,
                 const float *__restrict__ act_scale, const int32_t *__restrict__ row_sum,
                 const float *__restrict__ bias, int rows32, int K32, uint32_t qt_bytes, int row0_n,
                 float *__restrict__ y, int32_t *__restrict__ dot_out, int64_t ldy) {
  // Argument layout: everything the loads before the contraction need fits
  // in the 14 argument dwords preloaded into scalar registers at launch --
  // rows and K as 32-bit values, and the tiled copy's first row (< 16) and
  // N (<= 64) in one word, row0_n = (qt_row0 << 16) | N.
  const int64_t rows = rows32, K = K32, N = row0_n & 0xffff, qt_row0 = row0_n >> 16;
  static_assert(NB >= 1 && NB <= W, "one epilogue wave per activation block");
  __shared__ __attribute__((aligned(16))) v4i part[W][NB][64];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, kb = lane >> 4;
  const int64_t o0 = static_cast<int64_t>(blockIdx.x) * 16;
  const uint32_t row_bytes = static_cast<uint32_t>(K / 4);
  const int steps = static_cast<int>((K + 255) / 256);
  const int64_t rows_here = rows - o0 < 16 ? rows - o0 : 16;
  const __amdgpu_buffer_rsrc_t wbuf = buffer_of(packed + o0 * row_bytes, static_cast<uint32_t>(rows_here * row_bytes));
  const __amdgpu_buffer_rsrc_t qbuf = buffer_of(qt, static_cast<uint32_t>(qt_bytes));
  const uint32_t w_lane = (lane >> 2) * row_bytes + 16 * (lane & 3);
  const int perm = 4 * (4 * li + kb);  // ds_bpermute source lane (bytes) of MFMA lane (li, kb)
  // Tiled-copy offset of this lane's 16 bytes of block b, step 0, chunk 0;
  // step st adds 4 KiB, chunk d adds 1 KiB.
  uint32_t q_lane[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int64_t ng = qt_row0 + 16 * b + li;
    q_lane[b] = static_cast<uint32_t>(((ng >> 4) * steps * 4 << 10) + 16 * ((ng & 15) + 16 * kb));
  }

  // Epilogue constants of this lane as an epilogue wave (activation row
  // 16*wave + li, weight rows o0 + 4*kb + r), loaded before the weight
  // stream: the weight scale from the in-band slot, the row's scale and sum,
  // the biases.  Buffer loads keep their place; loaded at their use they
  // would add a memory round trip before the stores.
  const int64_t n_ep = 16 * static_cast<int64_t>(wave) + li;
  const float ws = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(
      buffer_of(packed + rows * static_cast<int64_t>(row_bytes), 4), 0, 0, 0));
  const uint32_t n_off = wave < NB && n_ep < N ? static_cast<uint32_t>(4 * n_ep) : kOutOfRange;
  const float asc = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(buffer_of(act_scale, static_cast<uint32_t>(4 * N)), n_off, 0, 0));
  const int32_t rsm = __builtin_amdgcn_raw_buffer_load_b32(buffer_of(row_sum, static_cast<uint32_t>(4 * N)), n_off, 0, 0);
  float bvr[4];
  {
    const __amdgpu_buffer_rsrc_t bbuf = buffer_of(bias, bias ? static_cast<uint32_t>(rows * 4) : 0u);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t o = o0 + 4 * kb + r;
      bvr[r] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(bbuf, wave < NB && o < rows ? static_cast<uint32_t>(4 * o) : kOutOfRange, 0, 0));
    }
  }

  // Step slot i of batch g of this wave: K-step wave + W*(SPW*g + i).  Slots
  // past the last step and blocks past row N issue no loads and no MFMAs
  // (wave-uniform branches; their registers are never read).
  auto load = [&](int g, v4i (&wv)[SPW], v4i (&qv)[SPW][NB][4]) {
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int st = wave + W * (SPW * g + i);
      if (st >= steps) continue;
      wv[i] = __builtin_amdgcn_raw_buffer_load_b128(wbuf, w_lane + 64 * st, 0, 0);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (16 * b >= N) continue;
        const bool row_ok = 16 * b + li < N;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t qo = q_lane[b] + (4 * st + d) * 1024;  // past K (the half step of an odd group count) reads 0
          qv[i][b][d] = __builtin_amdgcn_raw_buffer_load_b128(
              qbuf, row_ok && 256 * st + 64 * kb + 16 * d < K ? qo : kOutOfRange, 0, 0);
        }
      }
    }
  };
  v4i acc[NB][2];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b][0] = acc[b][1] = v4i{0, 0, 0, 0};
  auto compute = [&](int g, const v4i (&wv)[SPW], const v4i (&qv)[SPW][NB][4]) {
    v4i a4[SPW];
#pragma unroll
    for (int i = 0; i < SPW; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) a4[i][e] = __builtin_amdgcn_ds_bpermute(perm, wv[i][e]);
    __builtin_amdgcn_sched_barrier(0);  // all permutes in flight before the first use
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      if (wave + W * (SPW * g + i) >= steps) continue;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const v4i a = unpack_codes(static_cast<uint32_t>(a4[i][d]));
#pragma unroll
        for (int b = 0; b < NB; ++b)
          if (16 * b < N) acc[b][d & 1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, qv[i][b][d], acc[b][d & 1], 0, 0, 0);
      }
    }
  };

  const int mine = steps > wave ? (steps - wave + W - 1) / W : 0;  // this wave's steps
  const int batches = (mine + SPW - 1) / SPW;
  v4i wa[SPW], wb[SPW], qa[SPW][NB][4], qb[SPW][NB][4];
  load(0, wa, qa);
  for (int g = 0; g < batches; g += 2) {
    load(g + 1, wb, qb);
    compute(g, wa, qa);
    if (g + 1 >= batches) break;
    load(g + 2, wa, qa);
    compute(g + 1, wb, qb);
  }

#pragma unroll
  for (int b = 0; b < NB; ++b) part[wave][b][lane] = acc[b][0] + acc[b][1];
  __syncthreads();
  if (wave >= NB) return;
  v4i tot = part[0][wave][lane];
#pragma unroll
  for (int w = 1; w < W; ++w) tot += part[w][wave][lane];

  // Lane (li, kb) of wave b holds the dots of weight rows o0 + 4*kb + r
  // (r = 0..3) with activation row n_ep = 16*b + li.
  const float t = ws * asc;
  const int32_t rs = rsm;
  const int64_t o = o0 + 4 * kb;
  const uint32_t out_bytes = static_cast<uint32_t>(((N - 1) * ldy + rows - o0) * 4);
  const __amdgpu_buffer_rsrc_t ybuf = buffer_of(y + o0, out_bytes);
  const __amdgpu_buffer_rsrc_t dbuf = buffer_of(DOT ? dot_out + o0 : nullptr, DOT ? out_bytes : 0);
  const bool n_ok = n_ep < N;
  const uint32_t base = n_ok ? static_cast<uint32_t>(n_ep * ldy + 4 * kb) : 0u;  // element offset from y + o0
  float v[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = epilogue(tot[r], rs, t);
  if (bias) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (o + r < rows) v[r] = add_bias(v[r], bvr[r]);
  }
  if constexpr (VEC4) {
    const uint32_t off = n_ok && o < rows ? 4 * base : kOutOfRange;
    const v4i yv = {__float_as_int(v[0]), __float_as_int(v[1]), __float_as_int(v[2]), __float_as_int(v[3])};
    __builtin_amdgcn_raw_buffer_store_b128(yv, ybuf, off, 0, kWkStore);
    if constexpr (DOT) __builtin_amdgcn_raw_buffer_store_b128(tot, dbuf, off, 0, 0);
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t off = n_ok && o + r < rows ? 4 * (base + r) : kOutOfRange;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(v[r]), ybuf, off, 0, kWkStore);
      if constexpr (DOT) __builtin_amdgcn_raw_buffer_store_b32(tot[r], dbuf, off, 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side launch helpers.

inline int hip_status() { return hipGetLastError() == hipSuccess ? I2S_OK : I2S_EHIP; }

template <int NC, int L, int RPL, int CPL>
int launch_gemv_cfg(const uint8_t *packed, int64_t rows, int64_t K, const ActWorkspace &ws,
                    float *y, int32_t *dot_out, const float *bias, int64_t ldy, hipStream_t stream) {
  constexpr int kRowsPerBlock = (64 / L) * RPL * (kGemvThreads / 64);
  const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (blocks > kMaxDim || rows > kMaxDim || K > kMaxDim || ldy > kMaxDim) return I2S_ERANGE;
  hipLaunchKernelGGL((gemv_kernel<NC, L, RPL, CPL>), dim3(static_cast<unsigned>(blocks)), dim3(kGemvThreads), 0,
                     stream, packed, ws.q, ws.scale, ws.row_sum, bias, static_cast<int>(rows), static_cast<int>(K),
                     static_cast<int>(ldy), y, dot_out);
  return hip_status();
}

// GEMV tile configurations: (lanes per row, rows per lane pass, chunk batch).
// Variant v selects the v-th entry (1-based); 0 picks by K.
int gemv_auto_variant(int64_t K) {
  const int64_t C = K / 64;
  return C <= 8 ? 1 : (C <= 32 ? 2 : 3);
}

template <int NC>
int launch_gemv_nc(int variant, const uint8_t *packed, int64_t rows, int64_t K, const ActWorkspace &ws,
                   float *y, int32_t *dot_out, const float *bias, int64_t ldy, hipStream_t stream) {
  if (variant == 0) variant = gemv_auto_variant(K);
  switch (variant) {
    case 1: return launch_gemv_cfg<NC, 4, 1, 2>(packed, rows, K, ws, y, dot_out, bias, ldy, stream);
    case 2: return launch_gemv_cfg<NC, 8, 1, 4>(packed, rows, K, ws, y, dot_out, bias, ldy, stream);
    case 3: return launch_gemv_cfg<NC, 64, 1, 3>(packed, rows, K, ws, y, dot_out, bias, ldy, stream);
    case 4: return launch_gemv_cfg<NC, 8, 2, 3>(packed, rows, K, ws, y, dot_out, bias, ldy, stream);
    case 5: return launch_gemv_cfg<NC, 16, 1, 2>(packed, rows, K, ws, y, dot_out, bias, ldy, stream);
    default: return I2S_EKERNEL;
  }
}
constexpr int kGemvVariants = 5;

int launch_gemv(int variant, const uint8_t *packed, int64_t rows, int64_t K, int64_t N, const ActWorkspace &ws,
                float *y, int32_t *dot_out, const float *bias, int64_t ldy, hipStream_t stream) {
  switch (N) {
    case 1: return launch_gemv_nc<1>(variant, packed, rows, K, ws, y, dot_out, bias, ldy, stream);
    case 2: return launch_gemv_nc<2>(variant, packed, rows, K, ws, y, dot_out, bias, ldy, stream);
    case 3: return launch_gemv_nc<3>(variant, packed, rows, K, ws, y, dot_out, bias, ldy, stream);
    case 4: return launch_gemv_nc<4>(variant, packed, rows, K, ws, y, dot_out, bias, ldy, stream);
    case 5: return launch_gemv_nc<5>(variant, packed, rows, K, ws, y, dot_out, bias, ldy, stream);
    case 6: return launch_gemv_nc<6>(variant, packed, rows, K, ws, y, dot_out, bias, ldy, stream);
    case 7: return launch_gemv_nc<7>(variant, packed, rows, K, ws, y, dot_out, bias, ldy, stream);
    case 8: return launch_gemv_nc<8>(variant, packed, rows, K, ws, y, dot_out, bias, ldy, stream);
    default: return I2S_EKERNEL;
  }
}

template <int NC, int L, int RPL, int CPL, int XPT, int T = kGemvThreads>
int launch_fused_cfg(const uint8_t *packed, int64_t rows, int64_t K, const float *x, int64_t ldx, float *y,
                     int32_t *dot_out, const float *bias, int64_t ldy,
                     hipStream_t stream) {
  if (K > 64 * L * CPL || K > 4 * T * XPT) return I2S_EKERNEL;
  if (rows * (K / 4) >= (int64_t{1} << 31)) return I2S_EKERNEL;  // 32-bit buffer offsets
  constexpr int kRowsPerBlock = (64 / L) * RPL * (T / 64);
  const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (blocks > kMaxDim) return I2S_ERANGE;
  if (ldx > kMaxDim || ldy > kMaxDim) return I2S_ERANGE;  // the kernel takes 32-bit sizes
  hipLaunchKernelGGL((gemv_fused_kernel<NC, L, RPL, CPL, XPT, T>), dim3(static_cast<unsigned>(blocks)),
                     dim3(T), static_cast<size_t>(NC * K), stream, packed, x, y, bias, dot_out, static_cast<int>(rows),
                     static_cast<int>(K), static_cast<int>(ldx), static_cast<int>(ldy));
  return hip_status();
}

// Fused quantize + GEMV configurations (1-based): (L, RPL, CPL, XPT) =
// (8, 2, 3, 2), (8, 1, 4, 2), (16, 1, 2, 2) for K <= 1536/2048/2048,
// (64, 1, 3, 9), (32, 1, 5, 9) for K <= 9216 (the down projection),
// (8, 1, 3, 2) for K <= 1536 (variant 2 without its fourth chunk batch,
// which at K = 1536 would be a load past every row), all with 256 threads;
// and (8, 1, 3, 1) with 384 threads (48 rows per workgroup) for K <= 1536.
// Automatic: measured fastest on MI355X for the decoder shapes (8960 rows
// at K = 1536: 3.00 us with variant 7 against 3.21 with variant 6, whose
// 280 workgroups exceed the compute units; 6144 rows: 2.54 with variant 6
// against 2.98; 17920 rows: 3.77 against 4.08).
constexpr int kFusedVariants = 8;
constexpr int64_t kFusedMaxK = 9216;

int fused_auto_variant(int64_t rows, int64_t K) {
  if (K > 2048) return 5;
  if (rows <= 2048) return 3;
  // More than 256 workgroups of 32 rows put a second workgroup on some
  // compute units, whose activation loads then queue behind the first one's
  // weights; up to 256 workgroups of 48 rows (6 waves) avoid that
  // (8960 x 1536: 2.84 us against 3.10; 8960 x 2048: 3.16 against 3.38).
  // With fewer rows the 32-row workgroups fill more of the chip.
  if (rows > 8192 && rows <= 12288) return K <= 1536 ? 7 : 8;
  return K <= 1536 ? 6 : 2;
}

template <int NC>
int launch_fused_nc(int variant, const uint8_t *packed, int64_t rows, int64_t K, const float *x, int64_t ldx, float *y,
                    int32_t *dot_out, const float *bias, int64_t ldy, hipStream_t stream) {
  if (variant == 0) variant = fused_auto_variant(rows, K);
  switch (variant) {
    case 1: return launch_fused_cfg<NC, 8, 2, 3, 2>(packed, rows, K, x, ldx, y, dot_out, bias, ldy, stream);
    case 2: return launch_fused_cfg<NC, 8, 1, 4, 2>(packed, rows, K, x, ldx, y, dot_out, bias, ldy, stream);
    case 3: return launch_fused_cfg<NC, 16, 1, 2, 2>(packed, rows, K, x, ldx, y, dot_out, bias, ldy, stream);
    case 4: return launch_fused_cfg<NC, 64, 1, 3, 9>(packed, rows, K, x, ldx, y, dot_out, bias, ldy, stream);
    case 5: return launch_fused_cfg<NC, 32, 1, 5, 9>(packed, rows, K, x, ldx, y, dot_out, bias, ldy, stream);
    case 6: return launch_fused_cfg<NC, 8, 1, 3, 2>(packed, rows, K, x, ldx, y, dot_out, bias, ldy, stream);
    case 7: return launch_fused_cfg<NC, 8, 1, 3, 1, 384>(packed, rows, K, x, ldx, y, dot_out, bias, ldy, stream);
    case 8: return launch_fused_cfg<NC, 8, 1, 4, 2, 384>(packed, rows, K, x, ldx, y, dot_out, bias, ldy, stream);
    default: return I2S_EKERNEL;
  }
}

int launch_fused(int variant, const uint8_t *packed, int64_t rows, int64_t K, int64_t N, const float *x, int64_t ldx, float *y,
                 int32_t *dot_out, const float *bias, int64_t ldy, hipStream_t stream) {
  switch (N) {
    case 1: return launch_fused_nc<1>(variant, packed, rows, K, x, ldx, y, dot_out, bias, ldy, stream);
    case 2: return launch_fused_nc<2>(variant, packed, rows, K, x, ldx, y, dot_out, bias, ldy, stream);
    case 3: return launch_fused_nc<3>(variant, packed, rows, K, x, ldx, y, dot_out, bias, ldy, stream);
    case 4: return launch_fused_nc<4>(variant, packed, rows, K, x, ldx, y, dot_out, bias, ldy, stream);
    default: return I2S_EKERNEL;
  }
}

template <int NC, int L, int RPL, int CPL, int XPT, int T = kGemvThreads>
int launch_fused_group_cfg(const FusedGroup &g, int64_t K, const float *x, hipStream_t stream) {
  if (K > 64 * L * CPL || K > 4 * T * XPT) return I2S_EKERNEL;
  constexpr int kRowsPerBlock = (64 / L) * RPL * (T / 64);
  int64_t widest = 0;  // workgroups of the projection with the most rows
  for (int p = 0; p < g.count; ++p) {
    if (g.rows[p] * (K / 4) >= (int64_t{1} << 31)) return I2S_EKERNEL;  // 32-bit buffer offsets
    const int64_t b = (g.rows[p] + kRowsPerBlock - 1) / kRowsPerBlock;
    widest = b > widest ? b : widest;
  }
  if (widest == 0) return I2S_OK;
  if (widest > kMaxDim) return I2S_ERANGE;
  if (g.count == 2 && !g.bias[0] && !g.bias[1] && !g.dot[0] && !g.dot[1]) {
    hipLaunchKernelGGL((gemv_fused_pair_kernel<NC, L, RPL, CPL, XPT, T>), dim3(static_cast<unsigned>(widest), 2u), dim3(T),
                       static_cast<size_t>(NC * K), stream, g.packed[0], g.packed[1], static_cast<int>(g.rows[0]),
                       static_cast<int>(g.rows[1]), static_cast<int>(K), x, g.y[0], g.y[1]);
    return hip_status();
  }
  hipLaunchKernelGGL((gemv_fused_group_kernel<NC, L, RPL, CPL, XPT, T>),
                     dim3(static_cast<unsigned>(widest), static_cast<unsigned>(g.count)), dim3(T),
                     static_cast<size_t>(NC * K), stream, g, K, x);
  return hip_status();
}

template <int NC>
int launch_fused_group_nc(int variant, const FusedGroup &g, int64_t total_rows, int64_t K, const float *x,
                          hipStream_t stream) {
  if (variant == 0) variant = fused_auto_variant(total_rows, K);
  switch (variant) {
    case 1: return launch_fused_group_cfg<NC, 8, 2, 3, 2>(g, K, x, stream);
    case 2: return launch_fused_group_cfg<NC, 8, 1, 4, 2>(g, K, x, stream);
    case 3: return launch_fused_group_cfg<NC, 16, 1, 2, 2>(g, K, x, stream);
    case 4: return launch_fused_group_cfg<NC, 64, 1, 3, 9>(g, K, x, stream);
    case 5: return launch_fused_group_cfg<NC, 32, 1, 5, 9>(g, K, x, stream);
    case 6: return launch_fused_group_cfg<NC, 8, 1, 3, 2>(g, K, x, stream);
    case 7: return launch_fused_group_cfg<NC, 8, 1, 3, 1, 384>(g, K, x, stream);
    case 8: return launch_fused_group_cfg<NC, 8, 1, 4, 2, 384>(g, K, x, stream);
    default: return I2S_EKERNEL;
  }
}

int launch_fused_group(int variant, const FusedGroup &g, int64_t total_rows, int64_t K, int64_t N, const float *x,
                       hipStream_t stream) {
  switch (N) {
    case 1: return launch_fused_group_nc<1>(variant, g, total_rows, K, x, stream);
    case 2: return launch_fused_group_nc<2>(variant, g, total_rows, K, x, stream);
    case 3: return launch_fused_group_nc<3>(variant, g, total_rows, K, x, stream);
    case 4: return launch_fused_group_nc<4>(variant, g, total_rows, K, x, stream);
    default: return I2S_EKERNEL;
  }
}

// The fused path is chosen automatically for N <= 4 activation rows (each
// workgroup quantizes them itself; measured faster than a separate quantize
// launch up to N = 4 on the decoder shapes).
// Automatic choices, measured on MI355X (decoder projection shapes): the
// fused quantize + GEMV for N <= 3; otherwise the v_dot4 GEMV for N = 1 (and
// N = 2 at short K), the skinny MFMA kernel up to N = 16, the MFMA GEMM above.
inline bool fused_auto(int64_t rows, int64_t N, int64_t K) {
  return N <= 3 && K <= kFusedMaxK && rows * (K / 4) < (int64_t{1} << 31);
}

template <class Cfg>
int launch_gemm_cfg(const uint8_t *packed, int64_t rows, int64_t K, int64_t N, const ActWorkspace &ws,
                    float *y, int32_t *dot_out, const float *bias, int64_t ldy, hipStream_t stream) {
  const int64_t tiles_m = (rows + Cfg::kBM - 1) / Cfg::kBM;
  const int64_t tiles_n = (N + Cfg::kBN - 1) / Cfg::kBN;
  const int64_t blocks = tiles_m * tiles_n;
  if (blocks > kMaxDim) return I2S_ERANGE;
  hipLaunchKernelGGL((gemm_kernel<Cfg>), dim3(static_cast<unsigned>(blocks)), dim3(Cfg::kThreads), 0, stream,
                     packed, rows, K, ws.q, N, ws.scale, ws.row_sum, y, dot_out, bias, ldy, tiles_m);
  return hip_status();
}

using GemmA = GemmCfg<4, 4, 4, 1>;  // 256 x 64 block, 4 waves
using GemmB = GemmCfg<4, 2, 2, 2>;  // 128 x 64 block, 4 waves
using GemmC = GemmCfg<5, 4, 4, 1>;  // 320 x 64 block, 4 waves
using GemmD = GemmCfg<2, 2, 4, 1>;  // 128 x 32 block, 4 waves

template <class Cfg>
int64_t gemm_blocks(int64_t rows, int64_t N) {
  return ((rows + Cfg::kBM - 1) / Cfg::kBM) * ((N + Cfg::kBN - 1) / Cfg::kBN);
}

// Pick the streaming configuration whose most loaded compute unit (256 CUs,
// one block each at a time) does the least padded MFMA work.
int pick_stream_variant(int64_t rows, int64_t N) {
  const int64_t cus = 256;
  int64_t best_cost = -1;
  int best = 1;
  const int64_t blocks[4] = {gemm_blocks<GemmA>(rows, N), gemm_blocks<GemmB>(rows, N),
                             gemm_blocks<GemmC>(rows, N), gemm_blocks<GemmD>(rows, N)};
  const int64_t area[4] = {GemmA::kBM * GemmA::kBN, GemmB::kBM * GemmB::kBN, GemmC::kBM * GemmC::kBN,
                           GemmD::kBM * GemmD::kBN};
  for (int v = 0; v < 4; ++v) {
    const int64_t rounds = (blocks[v] + cus - 1) / cus;
    const int64_t cost = rounds * area[v];
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = v + 1;
    }
  }
  return best;
}

// Activation-resident launch: BN = 16*WN activation rows per block; the
// output features are split into tiles of ms 16-row subtiles so that the grid
// is about one block per compute unit.  Buffer offsets are 32-bit, so the
// packed payload, the activation tile and the block's outputs must stay below
// 2^31 bytes (else I2S_EKERNEL, and the automatic choice streams instead).
template <int G, int WN, int S, int WAVES, bool VEC4, bool DOT, bool SINGLE, bool PERM, bool PAIR>
int launch_res_inst(int64_t blocks, int64_t lds, const uint8_t *packed, int64_t rows, int64_t K, int64_t N,
                    const ActWorkspace &ws, float *y, int32_t *dot_out, const float *bias, int64_t ldy,
                    int64_t tiles_m, int64_t ms,
                    hipStream_t stream) {
  // Allow up to 160 KiB of dynamic LDS, once per device for this instantiation
  // (repeating it from racing threads is harmless).
  static std::atomic<uint64_t> attr_done{0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return I2S_EHIP;
  const uint64_t bit = dev < 64 ? (uint64_t{1} << dev) : 0;
  if (!bit || !(attr_done.load(std::memory_order_acquire) & bit)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(&gemm_res_kernel<G, WN, S, WAVES, VEC4, DOT, SINGLE, PERM, PAIR>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kResMaxLds) != hipSuccess)
      return I2S_EHIP;
    attr_done.fetch_or(bit, std::memory_order_acq_rel);
  }
  hipLaunchKernelGGL((gemm_res_kernel<G, WN, S, WAVES, VEC4, DOT, SINGLE, PERM, PAIR>), dim3(static_cast<unsigned>(blocks)),
                     dim3(64 * WAVES), static_cast<size_t>(lds), stream, static_cast<int>(tiles_m), static_cast<int>(ms),
                     packed, rows, K, ws.q, N, ws.row_sum, ws.scale, y, dot_out, bias, ldy);
  return hip_status();
}

template <int G, int WN, int S, int WAVES, bool PERM = false, bool PAIR = false>
int launch_res_cfg(const uint8_t *packed, int64_t rows, int64_t K, int64_t N, const ActWorkspace &ws, float *y,
                   int32_t *dot_out, const float *bias, int64_t ldy, hipStream_t stream) {
  constexpr int64_t BN = 16 * WN;
  // Whole KiB: the tile is filled by 1 KiB LDS-direct load runs.
  const int64_t lds = (BN * res_pitch(K, S) + 1023) / 1024 * 1024;
  if (lds > kResMaxLds) return I2S_EKERNEL;
  const int64_t lim = int64_t{1} << 31;
  // Largest weight offset: rows past the tile by up to 16*WAVES*G (re-reads of
  // a short or finished group), plus a chunk padded up to S steps.
  if ((rows + 16 * WAVES * G + 16) * (K / 4) + 64 * S * ((K + 255) / 256 + S) >= lim || BN * K >= lim ||
      BN * ldy * 4 >= lim)
    return I2S_EKERNEL;
  const int64_t tiles_n = (N + BN - 1) / BN;
  const int64_t mt = (rows + 15) / 16;
  int64_t tiles_m = 256 / tiles_n;
  if (tiles_m < 1) tiles_m = 1;
  int64_t ms = (mt + tiles_m - 1) / tiles_m;
  if (ms < 1) ms = 1;
  tiles_m = (mt + ms - 1) / ms;
  const int64_t blocks = tiles_m * tiles_n;
  if (blocks > kMaxDim || ms > kMaxDim) return I2S_ERANGE;
  const bool vec4 = (rows % 4) == 0 && (ldy % 4) == 0 && aligned16(y) && (!dot_out || aligned16(dot_out));
  const bool single = (K + 255) / 256 <= S;
#define I2S_RES(V, D, SG)                                                                                         \
  return launch_res_inst<G, WN, S, WAVES, V, D, SG, PERM, PAIR>(blocks, lds, packed, rows, K, N, ws, y, dot_out, bias, ldy, tiles_m, ms, \
                                                    stream)
  if (single) {
    if (vec4) {
      if (dot_out) I2S_RES(true, true, true);
      I2S_RES(true, false, true);
    }
    if (dot_out) I2S_RES(false, true, true);
    I2S_RES(false, false, true);
  }
  if (vec4) {
    if (dot_out) I2S_RES(true, true, false);
    I2S_RES(true, false, false);
  }
  if (dot_out) I2S_RES(false, true, false);
  I2S_RES(false, false, false);
#undef I2S_RES
}

// Pipelined launch: BN = 16*WN activation rows per block, about one block per
// compute unit; K must fit in SM steps and the activation tile in LDS, and
// buffer offsets must stay below 2^31 bytes (else I2S_EKERNEL).
template <int G, int WN, int WAVES, int SM, bool VEC4, bool DOT>
int launch_pipe_inst(int64_t blocks, int64_t lds, const uint8_t *packed, int64_t rows, int64_t K, int64_t N,
                    const ActWorkspace &ws, float *y, int32_t *dot_out, const float *bias, int64_t ldy,
                    int64_t tiles_m, int64_t ms,
                    hipStream_t stream) {
  static std::atomic<uint64_t> attr_done{0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return I2S_EHIP;
  const uint64_t bit = dev < 64 ? (uint64_t{1} << dev) : 0;
  if (!bit || !(attr_done.load(std::memory_order_acquire) & bit)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(&gemm_pipe_kernel<G, WN, WAVES, SM, VEC4, DOT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kResMaxLds) != hipSuccess)
      return I2S_EHIP;
    attr_done.fetch_or(bit, std::memory_order_acq_rel);
  }
  hipLaunchKernelGGL((gemm_pipe_kernel<G, WN, WAVES, SM, VEC4, DOT>), dim3(static_cast<unsigned>(blocks)),
                     dim3(64 * WAVES), static_cast<size_t>(lds), stream, packed, rows, K, ws.q, N, ws.scale,
                     ws.row_sum, y, dot_out, bias, ldy, tiles_m, static_cast<int>(ms));
  return hip_status();
}

template <int G, int WN, int WAVES, int SM>
int launch_pipe_cfg(const uint8_t *packed, int64_t rows, int64_t K, int64_t N, const ActWorkspace &ws, float *y,
                   int32_t *dot_out, const float *bias, int64_t ldy, hipStream_t stream) {
  constexpr int64_t BN = 16 * WN;
  const int64_t steps = (K + 255) / 256;
  const int64_t lds = BN * (256 * steps + 16);
  if (steps > SM || lds > kResMaxLds) return I2S_EKERNEL;
  const int64_t lim = int64_t{1} << 31;
  if ((rows + 16) * (K / 4) >= lim || BN * K >= lim || BN * ldy * 4 >= lim || rows >= (int64_t{1} << 24))
    return I2S_EKERNEL;
  const int64_t tiles_n = (N + BN - 1) / BN;
  const int64_t mt = (rows + 15) / 16;
  int64_t tiles_m = 256 / tiles_n;
  if (tiles_m < 1) tiles_m = 1;
  int64_t ms = (mt + tiles_m - 1) / tiles_m;
  if (ms < 1) ms = 1;
  tiles_m = (mt + ms - 1) / ms;
  const int64_t blocks = tiles_m * tiles_n;
  if (blocks > kMaxDim || ms > kMaxDim) return I2S_ERANGE;
  const bool vec4 = (rows % 4) == 0 && (ldy % 4) == 0 && aligned16(y) && (!dot_out || aligned16(dot_out));
#define I2S_SEQ(V, D) \
  return launch_pipe_inst<G, WN, WAVES, SM, V, D>(blocks, lds, packed, rows, K, N, ws, y, dot_out, bias, ldy, tiles_m, ms, \
                                                         stream)
  if (vec4) {
    if (dot_out) I2S_SEQ(true, true);
    I2S_SEQ(true, false);
  }
  if (dot_out) I2S_SEQ(false, true);
  I2S_SEQ(false, false);
#undef I2S_SEQ
}


// Weight-resident launch (variant 15; the kernel also builds with 12 waves per
// block, which measured no faster on the prefill shapes):
// K up to 1536 (the decoder's q/k/v/o/gate/up input width, CH = 6 chunks;
// shorter K runs its missing positions as zeros), 64-row activation tiles,
// about one block per compute unit, at most 24 subtiles per block (G = 1, 2,
// 3 for 8, 16, 24).
template <int G, int CH, int WAVES, bool VEC4, bool DOT>
int launch_wk_inst(int64_t blocks, const uint8_t *packed, int64_t rows, int64_t K, int64_t N, const ActWorkspace &ws,
                   float *y, int32_t *dot_out, const float *bias, int64_t ldy, int64_t tiles_m, int64_t ms,
                   hipStream_t stream) {
  static std::atomic<uint64_t> attr_done{0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return I2S_EHIP;
  const uint64_t bit = dev < 64 ? (uint64_t{1} << dev) : 0;
  if (!bit || !(attr_done.load(std::memory_order_acquire) & bit)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(&gemm_wk_kernel<G, CH, WAVES, VEC4, DOT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kResMaxLds) != hipSuccess)
      return I2S_EHIP;
    attr_done.fetch_or(bit, std::memory_order_acq_rel);
  }
  hipLaunchKernelGGL((gemm_wk_kernel<G, CH, WAVES, VEC4, DOT>), dim3(static_cast<unsigned>(blocks)), dim3(64 * WAVES),
                     static_cast<size_t>(CH * kWkChunkBytes), stream, static_cast<int>(tiles_m), static_cast<int>(ms),
                     packed, rows, static_cast<int>(K), ws.q, N, ws.row_sum, ws.scale, bias, y, dot_out, ldy);
  return hip_status();
}

template <int G, int CH, int WAVES>
int launch_wk_g(int64_t blocks, const uint8_t *packed, int64_t rows, int64_t K, int64_t N, const ActWorkspace &ws,
                float *y, int32_t *dot_out, const float *bias, int64_t ldy, int64_t tiles_m, int64_t ms,
                hipStream_t stream) {
  const bool vec4 = (rows % 4) == 0 && (ldy % 4) == 0 && aligned16(y) && (!dot_out || aligned16(dot_out));
  if (vec4) {
    if (dot_out) return launch_wk_inst<G, CH, WAVES, true, true>(blocks, packed, rows, K, N, ws, y, dot_out, bias, ldy, tiles_m, ms, stream);
    return launch_wk_inst<G, CH, WAVES, true, false>(blocks, packed, rows, K, N, ws, y, dot_out, bias, ldy, tiles_m, ms, stream);
  }
  if (dot_out) return launch_wk_inst<G, CH, WAVES, false, true>(blocks, packed, rows, K, N, ws, y, dot_out, bias, ldy, tiles_m, ms, stream);
  return launch_wk_inst<G, CH, WAVES, false, false>(blocks, packed, rows, K, N, ws, y, dot_out, bias, ldy, tiles_m, ms, stream);
}

// The block grid of the weight-resident kernel: tiles of 64 activation rows,
// weight tiles of ms subtiles, about one block per compute unit.
inline void wk_grid(int64_t rows, int64_t N, int64_t *tiles_m, int64_t *ms, int64_t *blocks) {
  const int64_t tiles_n = (N + 63) / 64;
  const int64_t mt = (rows + 15) / 16;
  int64_t tm = 256 / tiles_n;
  if (tm < 1) tm = 1;
  int64_t m = (mt + tm - 1) / tm;
  if (m < 1) m = 1;
  *ms = m;
  *tiles_m = (mt + m - 1) / m;
  *blocks = *tiles_m * tiles_n;
}

bool wk_fits(int64_t rows, int64_t K, int64_t N) {
  if (K > 1536 || N < 1) return false;
  int64_t tm, ms, blocks;
  wk_grid(rows, N, &tm, &ms, &blocks);
  return ms <= 24 && blocks <= kMaxDim && (rows + 16) * (K / 4) < (int64_t{1} << 31) && 64 * K < (int64_t{1} << 31);
}

template <int WAVES>
int launch_wk(const uint8_t *packed, int64_t rows, int64_t K, int64_t N, const ActWorkspace &ws, float *y,
              int32_t *dot_out, const float *bias, int64_t ldy, hipStream_t stream) {
  if (!wk_fits(rows, K, N) || 64 * ldy * 4 >= (int64_t{1} << 31)) return I2S_EKERNEL;
  int64_t tiles_m, ms, blocks;
  wk_grid(rows, N, &tiles_m, &ms, &blocks);
  if (ms <= WAVES) return launch_wk_g<1, 6, WAVES>(blocks, packed, rows, K, N, ws, y, dot_out, bias, ldy, tiles_m, ms, stream);
  if constexpr (WAVES == 8) {
    if (ms <= 16) return launch_wk_g<2, 6, 8>(blocks, packed, rows, K, N, ws, y, dot_out, bias, ldy, tiles_m, ms, stream);
    return launch_wk_g<3, 6, 8>(blocks, packed, rows, K, N, ws, y, dot_out, bias, ldy, tiles_m, ms, stream);
  } else {
    return launch_wk_g<2, 6, WAVES>(blocks, packed, rows, K, N, ws, y, dot_out, bias, ldy, tiles_m, ms, stream);
  }
}

// GEMM variants (1-based): 1-4 streaming (GemmA..D), 5-9 activation-resident
// (G, WN, S, waves) = (3,4,6,4), (2,4,6,8), (3,4,3,8), (3,2,6,8), (3,1,6,8), 10 pipelined
// (G, WN, waves, steps) = (2,2,4,6), 11 = 7 with row-contiguous weight loads
// permuted into MFMA lane order, 12-14 the same in 2-step chunks with groups
// of 2, 4 and 3, 15 weight-resident (K <= 1536).
constexpr int kGemmVariants = 18;

int gemm_auto_variant(int64_t rows, int64_t K, int64_t N) {
  int variant;
  // Measured on MI355X (rows 256 .. 8960, K 1024 .. 8960, N 64 .. 2048; K =
  // 1536 swept again for the weight-resident kernel): with at most 16
  // subtiles per block (two per wave) the weight-resident kernel is fastest
  // where K fits it (1536 x 1536 at N = 512: 5.7 against 7.2 us for the
  // pipelined kernel; 256 x 1536: 4.5 against 6.0; 8960 x 1536 at N = 128:
  // 7.0 against 7.7, at N = 256: 9.0 against 9.2; 4096 x 1536 at N = 512:
  // 8.2 against 8.8); beyond, the 8-wave resident kernel with row-contiguous
  // weight loads, its group size by the subtiles each wave holds (at 18
  // subtiles per block the two kernels are within run-to-run spread).  Where K is too long for either, the 4-wave pipelined kernel from
  // few subtiles, narrower resident tiles for longer K.
  const int64_t tiles_n = (N + 63) / 64;
  const int64_t tiles_m = tiles_n < 256 ? 256 / tiles_n : 1;
  const int64_t ms7 = ((rows + 15) / 16 + tiles_m - 1) / tiles_m;  // subtiles per block of variant 7
  const bool fits7 = 64 * res_pitch(K, 3) <= kResMaxLds && N > 16;
  const bool fits2 = 64 * res_pitch(K, 2) <= kResMaxLds && N > 16;
  if (wk_fits(rows, K, N) && ms7 <= 16) {
    variant = 15;
  } else if ((K + 255) / 256 <= 6 && (!fits7 || ms7 < (fits2 ? 4 : 8))) {
    variant = 10;
  } else if (fits2) {
    // Row-contiguous weight loads and 2-step chunks; the group size follows
    // the subtiles each wave holds (spw): whole groups of 2 with up to 2,
    // groups of 3 for 3 (8960 x 1536 at N = 512: 11.9 against 12.2 us with
    // groups of 4), groups of 4 for 4-5, groups of 3 beyond.  Groups of 3
    // store each wave's first two subtiles as whole 128-byte lines (variant
    // 16: 8960 x 1536 at N = 512, 11.0 against 11.6 us; at N = 2048, 37.8
    // against 39.4); with groups of 4 the pairing measured slower (N = 1024:
    // 21.2 against 20.8).
    const int64_t spw = (ms7 + 7) / 8;
    variant = spw <= 2 ? 12 : (spw == 3 ? 16 : (spw <= 5 ? 13 : 16));
  } else if (fits7) {
    variant = 11;  // variant 7's tiles with row-contiguous weight loads: 4-6% faster, measured
  } else if (16 * res_pitch(K, 6) <= kResMaxLds) {
    variant = 9;
  } else {
    variant = pick_stream_variant(rows, N);
  }
  return variant;
}

int launch_gemm(int variant, const uint8_t *packed, int64_t rows, int64_t K, int64_t N, const ActWorkspace &ws,
                float *y, int32_t *dot_out, const float *bias, int64_t ldy, hipStream_t stream) {
  if (variant == 0) variant = gemm_auto_variant(rows, K, N);
  switch (variant) {
    case 1: return launch_gemm_cfg<GemmA>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream);
    case 2: return launch_gemm_cfg<GemmB>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream);
    case 3: return launch_gemm_cfg<GemmC>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream);
    case 4: return launch_gemm_cfg<GemmD>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream);
    case 5: return launch_res_cfg<3, 4, 6, 4>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream);
    case 6: return launch_res_cfg<2, 4, 6, 8>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream);
    case 7: return launch_res_cfg<3, 4, 3, 8>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream);
    case 8: return launch_res_cfg<3, 2, 6, 8>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream);
    case 9: return launch_res_cfg<3, 1, 6, 8>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream);
    case 10: return launch_pipe_cfg<2, 2, 4, 6>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream);
    case 11: return launch_res_cfg<3, 4, 3, 8, true>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream);
    case 12: return launch_res_cfg<2, 4, 2, 8, true>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream);
    case 13: return launch_res_cfg<4, 4, 2, 8, true>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream);
    case 14: return launch_res_cfg<3, 4, 2, 8, true>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream);
    case 15: return launch_wk<8>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream);
    case 16: return launch_res_cfg<3, 4, 2, 8, true, true>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream);
    case 17: return launch_res_cfg<2, 4, 2, 8, true, true>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream);
    case 18: return launch_res_cfg<4, 4, 2, 8, true, true>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream);
    default: return I2S_EKERNEL;
  }
}

// Skinny MFMA launch (kernel 4): one block per 16-row subtile, NB = 1, 2 or 4
// blocks of 16 activation rows (N <= 16, 32, 64); 8 waves, except 4 at
// NB = 4 with more than 256 subtiles (its ~170 registers per lane allow one
// 8-wave block per compute unit, or two 4-wave blocks: with more blocks than
// compute units the shorter blocks win, measured on the decoder shapes).  Variant 1 issues
// 2 steps per batch at NB = 1 and 1 step otherwise, variant 2 twice as many
// where the activation registers allow (4, 2, 1; measured slower on the
// decoder shapes, kept for parity coverage of deeper batches).
constexpr int kSkinnyVariants = 2;
constexpr int kSkinnyMaxN = 64;

int skinny_auto_variant(int64_t) { return 1; }

bool skinny_fits(int64_t rows, int64_t K, int64_t N) {
  const int64_t lim = int64_t{1} << 31;
  return N <= kSkinnyMaxN && N * rows * 4 < lim && N * K < lim && 16 * (K / 4) + 64 < lim && (rows + 15) / 16 <= kMaxDim;
}

template <int NB, int SPW, bool VEC4, bool DOT>
int launch_skinny_inst(const uint8_t *packed, int64_t rows, int64_t K, int64_t N, const ActWorkspace &ws, float *y,
                       int32_t *dot_out, const float *bias, int64_t ldy, hipStream_t stream) {
  // The tiled copy from the 16-row block holding this call's first row: the
  // kernel's offsets stay 32-bit however many batches precede it.
  const int64_t row0 = ws.qt_row0 & 15;
  const int8_t *qt = ws.qt + (ws.qt_row0 >> 4) * ((K + 255) / 256) * 4096;
  const int64_t tiles = (rows + 15) / 16;
  const int64_t qbytes = static_cast<int64_t>(tiled_bytes(row0 + N, K));
  // More subtiles than compute units: 4 waves per workgroup (measured on
  // the 8960-row projections: 3.9 against 4.8 us at N = 8, 5.5 against 5.8
  // at N = 32); fewer: 8 waves split each subtile's K-steps further.
  if (tiles > 256) {
    hipLaunchKernelGGL((gemv_mfma_kernel<4, NB, SPW, VEC4, DOT>), dim3(static_cast<unsigned>(tiles)), dim3(256), 0,
                       stream, packed, qt, ws.scale, ws.row_sum, bias, static_cast<int>(rows), static_cast<int>(K),
                       static_cast<uint32_t>(qbytes), static_cast<int>((row0 << 16) | N), y, dot_out, ldy);
    return hip_status();
  }
  hipLaunchKernelGGL((gemv_mfma_kernel<8, NB, SPW, VEC4, DOT>), dim3(static_cast<unsigned>(tiles)), dim3(512), 0, stream,
                     packed, qt, ws.scale, ws.row_sum, bias, static_cast<int>(rows), static_cast<int>(K),
                     static_cast<uint32_t>(qbytes), static_cast<int>((row0 << 16) | N), y, dot_out, ldy);
  return hip_status();
}

template <int NB, int SPW>
int launch_skinny_cfg(const uint8_t *packed, int64_t rows, int64_t K, int64_t N, const ActWorkspace &ws, float *y,
                      int32_t *dot_out, const float *bias, int64_t ldy, hipStream_t stream) {
  // 32-bit buffer offsets: activation rows (N*K), one subtile's weights and
  // the outputs past the block's first row (N*rows*4) stay below 2^31.
  if (!skinny_fits(rows, K, N) || N > 16 * NB || N * ldy * 4 >= (int64_t{1} << 31) || !ws.qt ||
      tiled_bytes(15 + N, K) >= (size_t{1} << 31))
    return I2S_EKERNEL;
  const bool vec4 = (rows % 4) == 0 && (ldy % 4) == 0 && aligned16(y) && (!dot_out || aligned16(dot_out));
  if (vec4) return dot_out ? launch_skinny_inst<NB, SPW, true, true>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream)
                           : launch_skinny_inst<NB, SPW, true, false>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream);
  return dot_out ? launch_skinny_inst<NB, SPW, false, true>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream)
                 : launch_skinny_inst<NB, SPW, false, false>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream);
}

int launch_skinny(int variant, const uint8_t *packed, int64_t rows, int64_t K, int64_t N, const ActWorkspace &ws,
                  float *y, int32_t *dot_out, const float *bias, int64_t ldy, hipStream_t stream) {
  if (variant == 0) variant = skinny_auto_variant(K);
  if (variant < 1 || variant > kSkinnyVariants) return I2S_EKERNEL;
  const bool deep = variant == 2;
  if (N <= 16)
    return deep ? launch_skinny_cfg<1, 4>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream)
                : launch_skinny_cfg<1, 2>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream);
  if (N <= 32)
    return deep ? launch_skinny_cfg<2, 2>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream)
                : launch_skinny_cfg<2, 1>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream);
  return launch_skinny_cfg<4, 1>(packed, rows, K, N, ws, y, dot_out, bias, ldy, stream);
}

inline bool k_ok(int64_t K) { return K > 0 && K % kGroupValues == 0; }

int check_common(int64_t rows, int64_t K) {
  if (rows < 0) return I2S_EINVAL;
  if (!k_ok(K)) return I2S_EALIGN;
  if (K > kMaxK || rows > kMaxDim) return I2S_ERANGE;
  return I2S_OK;
}

int quantize_launch(const float *x, int64_t N, int64_t K, int64_t n_inner, int64_t ldx, int64_t bsx, int8_t *q,
                    float *s, int32_t *rs, bool interleaved, int8_t *qt,
                    hipStream_t stream) {
  if (N > kMaxDim) return I2S_ERANGE;
  // The row sits in registers: XPT float4 per thread; longer rows get more
  // threads (a row is one workgroup), so that each holds few values.
#define I2S_QREG(XPT, T)                                                                                   \
  do {                                                                                                     \
    if (interleaved)                                                                                       \
      hipLaunchKernelGGL((quantize_rowsum_reg_kernel<true, XPT, T>), dim3(static_cast<unsigned>(N)),       \
                         dim3(T), 0, stream, x, K, n_inner, ldx, bsx, q, qt, s, rs);                              \
    else                                                                                                   \
      hipLaunchKernelGGL((quantize_rowsum_reg_kernel<false, XPT, T>), dim3(static_cast<unsigned>(N)),      \
                         dim3(T), 0, stream, x, K, n_inner, ldx, bsx, q, nullptr, s, rs);                         \
    return hip_status();                                                                                   \
  } while (0)
  if (K <= 4 * 256 * 2) I2S_QREG(2, 256);
  if (K <= 4 * 512 * 2) I2S_QREG(2, 512);
  if (K <= 4 * 1024 * 3) I2S_QREG(3, 1024);
#undef I2S_QREG
  if (interleaved)
    hipLaunchKernelGGL((quantize_rowsum_kernel<true>), dim3(static_cast<unsigned>(N)), dim3(kQuantThreads), 0, stream,
                       x, K, n_inner, ldx, bsx, q, s, rs, qt);
  else
    hipLaunchKernelGGL((quantize_rowsum_kernel<false>), dim3(static_cast<unsigned>(N)), dim3(kQuantThreads), 0, stream,
                       x, K, n_inner, ldx, bsx, q, s, rs, nullptr);
  return hip_status();
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI.

extern "C" size_t i2s_packed_bytes(int64_t rows, int64_t K) {
  if (rows < 0 || !k_ok(K)) return 0;
  return static_cast<size_t>(rows) * static_cast<size_t>(K / 4) + kScaleSlot;
}

extern "C" size_t i2s_act_workspace_bytes(int64_t N, int64_t K) {
  if (N < 0 || !k_ok(K)) return 0;
  return align_up(static_cast<size_t>(N) * static_cast<size_t>(K), 256) + 2 * align_up(static_cast<size_t>(N) * 4, 256) +
         tiled_bytes(N, K);
}

extern "C" int i2s_pack(const int8_t *w, float weight_scale, int64_t rows, int64_t K, uint8_t *packed, void *stream) {
  int st = check_common(rows, K);
  if (st != I2S_OK) return st;
  if (!packed || (rows > 0 && !w)) return I2S_EINVAL;
  if (!aligned16(packed) || (rows > 0 && !aligned16(w))) return I2S_EINVAL;
  const int64_t units = rows * K / 64;
  const int64_t blocks = units > 0 ? (units + kPackThreads - 1) / kPackThreads : 1;
  if (blocks > kMaxDim) return I2S_ERANGE;
  hipLaunchKernelGGL(pack_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kPackThreads), 0,
                     static_cast<hipStream_t>(stream), w, weight_scale, units, rows * K / 4, packed);
  return hip_status();
}

extern "C" int i2s_quantize_act(const float *x, int64_t N, int64_t K, int8_t *q, float *act_scale, int32_t *row_sum,
                                void *stream) {
  if (N < 0) return I2S_EINVAL;
  int st = check_common(0, K);
  if (st != I2S_OK) return st;
  if (N == 0) return I2S_OK;
  if (!x || !q || !act_scale || !row_sum) return I2S_EINVAL;
  if (!aligned16(x) || !aligned16(q)) return I2S_EINVAL;
  return quantize_launch(x, N, K, N, K, N * K, q, act_scale, row_sum, false, nullptr, static_cast<hipStream_t>(stream));
}

namespace {

// Host-side checks shared by the matmul entry points; I2S_OK means launchable
// (or a no-op when N == 0 or rows == 0, reported through *noop).
int check_mul_mat(const uint8_t *packed, int64_t rows, int64_t K, int64_t N, const void *workspace,
                  size_t workspace_bytes, const float *y, const int32_t *dot_out, int kernel, int variant,
                  bool *noop) {
  *noop = false;
  if (N < 0) return I2S_EINVAL;
  int st = check_common(rows, K);
  if (st != I2S_OK) return st;
  if (kernel < 0 || kernel > 4 || variant < 0) return I2S_EKERNEL;
  if (kernel == 1 && (N > 8 || variant > kGemvVariants)) return I2S_EKERNEL;
  if (kernel == 2 && variant > kGemmVariants) return I2S_EKERNEL;
  if (kernel == 3 && (N > 4 || variant > kFusedVariants || K > kFusedMaxK)) return I2S_EKERNEL;
  if (kernel == 4 && (N > kSkinnyMaxN || variant > kSkinnyVariants)) return I2S_EKERNEL;
  if (kernel == 0 && variant != 0) return I2S_EKERNEL;
  if (N == 0 || rows == 0) {
    *noop = true;
    return I2S_OK;
  }
  if (N > kMaxDim) return I2S_ERANGE;
  if (!packed || !y) return I2S_EINVAL;
  if (!aligned16(packed) || !aligned16(y) || (dot_out && !aligned16(dot_out))) return I2S_EINVAL;
  if (!workspace || workspace_bytes < i2s_act_workspace_bytes(N, K)) return I2S_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return I2S_EWORKSPACE;
  return I2S_OK;
}

// The skinny kernel up to N = 32, and up to N = 64 with at most 256 weight
// subtiles (rows <= 4096); measured on the decoder shapes against the GEMM.
bool skinny_auto(int64_t rows, int64_t K, int64_t N) {
  if (!skinny_fits(rows, K, N)) return false;
  return N <= 32 || (N <= kSkinnyMaxN && (rows + 15) / 16 <= 256);
}

int contract_auto_kernel(int64_t rows, int64_t K, int64_t N) {
  if (N == 1 || (N == 2 && K <= 2048)) return 1;
  if (skinny_auto(rows, K, N)) return 4;
  return N <= 8 ? 1 : 2;
}

int contract(const uint8_t *packed, int64_t rows, int64_t K, int64_t N, const ActWorkspace &ws, float *y,
             int32_t *dot_out, const float *bias, int64_t ldy, int kernel, int variant, hipStream_t s) {
  if (kernel == 0) kernel = contract_auto_kernel(rows, K, N);
  if (kernel == 4) return launch_skinny(variant, packed, rows, K, N, ws, y, dot_out, bias, ldy, s);
  if (kernel == 1) return launch_gemv(variant, packed, rows, K, N, ws, y, dot_out, bias, ldy, s);
  return launch_gemm(variant, packed, rows, K, N, ws, y, dot_out, bias, ldy, s);
}

}  // namespace

extern "C" int i2s_quantize_act_ws(const float *x, int64_t N, int64_t K, void *workspace, size_t workspace_bytes,
                                   void *stream) {
  if (N < 0) return I2S_EINVAL;
  int st = check_common(0, K);
  if (st != I2S_OK) return st;
  if (N == 0) return I2S_OK;
  if (N > kMaxDim) return I2S_ERANGE;
  if (!x || !aligned16(x)) return I2S_EINVAL;
  if (!workspace || workspace_bytes < i2s_act_workspace_bytes(N, K)) return I2S_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return I2S_EWORKSPACE;
  ActWorkspace ws = carve_workspace(workspace, N, K, N);
  return quantize_launch(x, N, K, N, K, N * K, ws.q, ws.scale, ws.row_sum, true, ws.qt, static_cast<hipStream_t>(stream));
}

extern "C" int i2s_mul_mat_ws(const uint8_t *packed, int64_t rows, int64_t K, int64_t N, const void *workspace,
                              size_t workspace_bytes, float *y, int32_t *dot_out, int kernel, int variant,
                              void *stream) {
  bool noop;
  if (kernel == 3) return I2S_EKERNEL;  // the fused kernel quantizes x itself; x is not an argument here
  int st = check_mul_mat(packed, rows, K, N, workspace, workspace_bytes, y, dot_out, kernel, variant, &noop);
  if (st != I2S_OK || noop) return st;
  ActWorkspace ws = carve_workspace(const_cast<void *>(workspace), N, K, N);
  return contract(packed, rows, K, N, ws, y, dot_out, nullptr, rows, kernel, variant, static_cast<hipStream_t>(stream));
}

extern "C" int i2s_mul_mat_ex(const uint8_t *packed, int64_t rows, int64_t K, const float *x, int64_t N,
                              void *workspace, size_t workspace_bytes, float *y, int32_t *dot_out, int kernel,
                              int variant, void *stream) {
  bool noop;
  int st = check_mul_mat(packed, rows, K, N, workspace, workspace_bytes, y, dot_out, kernel, variant, &noop);
  if (st != I2S_OK || noop) return st;
  if (!x || !aligned16(x)) return I2S_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kernel == 3 || (kernel == 0 && fused_auto(rows, N, K)))
    return launch_fused(variant, packed, rows, K, N, x, K, y, dot_out, nullptr, rows, s);
  ActWorkspace ws = carve_workspace(workspace, N, K, N);
  st = quantize_launch(x, N, K, N, K, N * K, ws.q, ws.scale, ws.row_sum, true, ws.qt, s);
  if (st != I2S_OK) return st;
  return contract(packed, rows, K, N, ws, y, dot_out, nullptr, rows, kernel, variant, s);
}

extern "C" int i2s_mul_mat(const uint8_t *packed, int64_t rows, int64_t K, const float *x, int64_t N,
                           void *workspace, size_t workspace_bytes, float *y, int32_t *dot_out, void *stream) {
  return i2s_mul_mat_ex(packed, rows, K, x, N, workspace, workspace_bytes, y, dot_out, 0, 0, stream);
}

extern "C" int i2s_mul_mat_group_ex(const i2s_proj *projs, int count, int64_t K, const float *x, int64_t N,
                                    void *workspace, size_t workspace_bytes, int kernel, int variant,
                                    void *stream) {
  if (!projs || count < 1 || count > I2S_GROUP_MAX) return I2S_EINVAL;
  bool all_noop = true;
  int64_t total_rows = 0;
  bool fits = true;
  for (int p = 0; p < count; ++p) {
    bool noop;
    const int st = check_mul_mat(projs[p].packed, projs[p].rows, K, N, workspace, workspace_bytes, projs[p].y,
                                 projs[p].dot_out, kernel, variant, &noop);
    if (st != I2S_OK) return st;
    if (!noop && projs[p].bias && !aligned16(projs[p].bias)) return I2S_EINVAL;
    all_noop = all_noop && noop;
    total_rows += projs[p].rows;
    fits = fits && projs[p].rows * (K / 4) < (int64_t{1} << 31);
  }
  if (all_noop) return I2S_OK;
  if (!x || !aligned16(x)) return I2S_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kernel == 3 || (kernel == 0 && N <= 3 && K <= kFusedMaxK && fits)) {
    // One projection: the single-weight kernel, whose pointers arrive in
    // preloaded argument registers (the group's table is a struct argument,
    // read with a scalar load first: 4.39 against 3.99 us for the down
    // projection at N = 1).  Same body, same variants, same results.
    if (count == 1)
      return launch_fused(variant, projs[0].packed, projs[0].rows, K, N, x, K, projs[0].y, projs[0].dot_out,
                          projs[0].bias, projs[0].rows, s);
    FusedGroup g{};
    g.count = count;
    for (int p = 0; p < count; ++p) {
      g.packed[p] = projs[p].packed;
      g.rows[p] = projs[p].rows;
      g.bias[p] = projs[p].bias;
      g.y[p] = projs[p].y;
      g.dot[p] = projs[p].dot_out;
    }
    return launch_fused_group(variant, g, total_rows, K, N, x, s);
  }
  ActWorkspace ws = carve_workspace(workspace, N, K, N);
  int st = quantize_launch(x, N, K, N, K, N * K, ws.q, ws.scale, ws.row_sum, true, ws.qt, s);
  for (int p = 0; p < count && st == I2S_OK; ++p)
    if (projs[p].rows > 0)
      st = contract(projs[p].packed, projs[p].rows, K, N, ws, projs[p].y, projs[p].dot_out, projs[p].bias,
                    projs[p].rows, kernel, variant, s);
  return st;
}

extern "C" int i2s_mul_mat_group(const i2s_proj *projs, int count, int64_t K, const float *x, int64_t N,
                                 void *workspace, size_t workspace_bytes, void *stream) {
  return i2s_mul_mat_group_ex(projs, count, K, x, N, workspace, workspace_bytes, 0, 0, stream);
}

extern "C" int i2s_mul_mat_batched(const uint8_t *packed, int64_t rows, int64_t K, const float *x, int64_t N,
                                   int64_t B, int64_t ldx, int64_t bsx, void *workspace, size_t workspace_bytes,
                                   float *y, int64_t ldy, int64_t bsy, int32_t *dot_out, void *stream) {
  if (N < 0 || B < 0 || N > kMaxDim || B > kMaxDim) return N < 0 || B < 0 ? I2S_EINVAL : I2S_ERANGE;
  const int64_t NB = N * B;
  if (NB > kMaxDim) return I2S_ERANGE;
  bool noop;
  int st = check_mul_mat(packed, rows, K, NB, workspace, workspace_bytes, y, dot_out, 0, 0, &noop);
  if (st != I2S_OK || noop) return st;
  if (!x || !aligned16(x)) return I2S_EINVAL;
  // Rows of x start 16-byte aligned (float4 loads); outputs never overlap.
  if (ldx < K || ldx % 4 != 0 || bsx < 0 || bsx % 4 != 0) return I2S_EINVAL;
  if (ldy < rows || bsy < 0) return I2S_EINVAL;
  if (B > 1 && bsy < (N - 1) * ldy + rows) return I2S_EINVAL;
  if (ldx > kMaxDim || ldy > kMaxDim) return I2S_ERANGE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool dense = ldx == K && ldy == rows && (B == 1 || (bsx == N * K && bsy == N * rows));
  if (dense) return i2s_mul_mat_ex(packed, rows, K, x, NB, workspace, workspace_bytes, y, dot_out, 0, 0, stream);
  if (fused_auto(rows, N, K)) {
    for (int64_t b = 0; b < B && st == I2S_OK; ++b)
      st = launch_fused(0, packed, rows, K, N, x + b * bsx, ldx, y + b * bsy, dot_out ? dot_out + b * bsy : nullptr,
                        nullptr, ldy, s);
    return st;
  }
  ActWorkspace ws = carve_workspace(workspace, NB, K, N);
  st = quantize_launch(x, NB, K, N, ldx, bsx, ws.q, ws.scale, ws.row_sum, true, ws.qt, s);
  for (int64_t b = 0; b < B && st == I2S_OK; ++b) {
    ActWorkspace wb = ws;
    wb.q = ws.q + b * N * K;
    wb.scale = ws.scale + b * N;
    wb.row_sum = ws.row_sum + b * N;
    wb.qt_row0 = b * N;
    st = contract(packed, rows, K, N, wb, y + b * bsy, dot_out ? dot_out + b * bsy : nullptr, nullptr, ldy, 0, 0, s);
  }
  return st;
}

extern "C" int i2s_mul_mat_kernel(int64_t rows, int64_t K, int64_t N) {
  if (rows < 0 || N < 0) return -I2S_EINVAL;
  if (!k_ok(K)) return -I2S_EALIGN;
  if (fused_auto(rows, N, K)) return 3;
  return contract_auto_kernel(rows, K, N);
}

extern "C" int i2s_mul_mat_variant(int64_t rows, int64_t K, int64_t N) {
  const int kernel = i2s_mul_mat_kernel(rows, K, N);
  switch (kernel) {
    case 1: return gemv_auto_variant(K);
    case 2: return gemm_auto_variant(rows, K, N);
    case 3: return fused_auto_variant(rows, K);
    case 4: return skinny_auto_variant(K);
    default: return kernel;  // a negative status
  }
}

extern "C" int i2s_kernel_variants(int kernel) {
  if (kernel == 1) return kGemvVariants;
  if (kernel == 2) return kGemmVariants;
  if (kernel == 3) return kFusedVariants;
  if (kernel == 4) return kSkinnyVariants;
  return 0;
}

extern "C" const char *i2s_strerror(int status) {
  switch (status) {
    case I2S_OK: return "success";
    case I2S_EINVAL: return "invalid argument: null pointer, negative size, or pointer not 16-byte aligned";
    case I2S_EALIGN: return "K must be a positive multiple of 128";
    case I2S_EWORKSPACE: return "workspace missing, not 256-byte aligned, or smaller than i2s_act_workspace_bytes";
    case I2S_EHIP: return "HIP runtime error at launch";
    case I2S_ERANGE: return "size beyond what the library addresses";
    case I2S_EKERNEL: return "unknown kernel or variant, or one that does not accept this N or K";
    case I2S_ESCRATCH: return "the shape needs more workspace than i2s_mul_mat_noalloc's fixed array holds";
    default: return "unknown status";
  }
}
