// gfx950 (MI355X) kernels and C ABI for the I8_S per-tensor int8 type and its
// fused mul_mat_add / mul_mat_add_relu.  The ABI is declared, with its
// contract, in include/i8s.h.
//
// I8_S ("ggml: additive INT8/ternary types, fused CPU ops, and kernels for
// VibeASR (1/2)", Two new types): n int8 payload bytes, then the F32
// multiplier scale amax/127 in band, in a 32-byte slot.
//
// mul_mat_add (same page, Five fused INT8 ops): int32 acc = w . x, then
// f = (float)acc * (ws * xs) + bias[o] (ReLU in the relu form), then one
// per-tensor requantization of f.  The requantization needs max|f| over the
// whole output before any value can be written, so the op runs the same
// contraction twice: pass 1 reduces max|f| per workgroup into the workspace,
// pass 2 reduces those partial maxima to the tensor's scale and writes the
// int8 values.  Recomputing the integer contraction is cheaper than writing
// and re-reading the F32 tensor (4 bytes out and 4 back per output against
// the 1-byte result) for the encoder's shapes, whose IC is small.
//
// Every float operation is one IEEE operation: the library is built without
// fast-math and without FP contraction, and '/' is the correctly rounded
// division, so results match the definition bit for bit.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "i8s.h"
#include "w8a8.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;          // every kernel here: 4 wave64s
constexpr int kMaxParts = 1024;        // workgroups of a two-pass launch (partial maxima)
constexpr int kResidentGroups = 512;   // MFMA contraction grid: 2 workgroups per CU
constexpr int64_t kSkinnyFewWavesItems = 256;  // skinny items from which a workgroup has 4 waves
constexpr int64_t kMaxBytes = 0x7fff0000;  // largest tensor a buffer descriptor covers here
constexpr uint32_t kOutOfRange = 0x7ffffff0u;  // buffer offset beyond every descriptor range
constexpr int kBufferFlags = 0x00020000;       // raw buffer, 32-bit data format
constexpr float kAmaxFloor = 1e-5f;

__device__ inline __amdgpu_buffer_rsrc_t buffer_of(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           kBufferFlags);
}

// Max over the wave, in every lane: DPP moves within each quad, 8 and 16
// lanes (VALU, a few cycles each, where ds_bpermute shuffles would be an LDS
// round trip each), then one lane of each row of 16.  Max does not depend on
// the order of its terms.
template <int CTRL>
__device__ inline int dpp_move(int v) { return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false); }

__device__ inline float wave_max(float v) {
  v = fmaxf(v, __int_as_float(dpp_move<0xB1>(__float_as_int(v))));   // quad_perm(1,0,3,2)
  v = fmaxf(v, __int_as_float(dpp_move<0x4E>(__float_as_int(v))));   // quad_perm(2,3,0,1)
  v = fmaxf(v, __int_as_float(dpp_move<0x141>(__float_as_int(v))));  // row_half_mirror
  v = fmaxf(v, __int_as_float(dpp_move<0x140>(__float_as_int(v))));  // row_mirror
  const int b = __float_as_int(v);
  return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 0)), __int_as_float(__builtin_amdgcn_readlane(b, 16))),
               fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 32)), __int_as_float(__builtin_amdgcn_readlane(b, 48))));
}

// max over the workgroup; red is 4 floats of LDS; every thread gets the result.
__device__ inline float block_max(float v, float *red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}

// An in-band F32 scale at any byte address (the payload length need not be a
// multiple of 4).
__device__ inline float load_scale(const uint8_t *p) {
  const uint32_t b = static_cast<uint32_t>(p[0]) | (static_cast<uint32_t>(p[1]) << 8) |
                     (static_cast<uint32_t>(p[2]) << 16) | (static_cast<uint32_t>(p[3]) << 24);
  return __uint_as_float(b);
}

// The tensor scale from the partial maxima: amax floored at 1e-5, s = amax/127.
__device__ inline float scale_from_parts(const float *parts, int count, float *red) {
  float m = 0.0f;
  for (int i = threadIdx.x; i < count; i += kThreads) m = fmaxf(m, parts[i]);
  m = block_max(m, red);
  if (m < kAmaxFloor) m = kAmaxFloor;
  return m / 127.0f;
}

// The 32-byte scale slot after the payload: the F32 scale, then 28 zeros.
// Called by every thread of workgroup 0; threads 0..31 write one byte each.
__device__ inline void write_slot(uint8_t *slot, float s) {
  if (threadIdx.x < I8S_SCALE_SLOT) {
    const uint32_t b = __float_as_uint(s);
    slot[threadIdx.x] = threadIdx.x < 4 ? static_cast<uint8_t>(b >> (8 * threadIdx.x)) : 0;
  }
}

// q = f/s rounded half away from zero (roundf), clamped to [-127, 127].
__device__ inline int quant(float v, float s) {
  float r = roundf(v / s);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return static_cast<int>(r);
}

// The same q for 16 values at once, with the division replaced by a multiply
// by inv = 1/s (correctly rounded) wherever that provably gives the same q.
// The values are within the tensor's range (|v| <= amax, so |v/s| <= 127.0001;
// ReLU is applied before), r = fl(v * inv) is within |v/s| * 2^-23 (1.6e-5)
// of v/s, and fl(v/s) within 2^-18 of it.  So if the fraction of |r| is more
// than 2^-14 from 1/2, r and fl(v/s) lie strictly between the same two
// half-integers: both round to the integer nearest r, whatever the tie rule,
// and rint(r) (ties to even, one instruction) gives q, already within +-127.
// A group with any value nearer a tie takes the exact division for all 16.
// The result is returned as floats whose low byte is q: x + 1.5 * 2^23, for
// |x| <= 127.0001, lands where floats are one apart, so the sum is x rounded
// to nearest even (ties to even, as rint; exact for the division path's
// integers) and its low byte is that integer's two's-complement byte
// (1.5 * 2^23 = 0x4B400000 has a zero low byte).
constexpr float kTieMargin = 6.103515625e-05f;  // 2^-14
constexpr float kRoundMagic = 0x1.8p23f;

__device__ inline void quant16(const float (&v)[16], float s, float inv, uint32_t (&qb)[16]) {
  bool near = false;
  float r[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    r[j] = v[j] * inv;
    near |= fabsf(__builtin_amdgcn_fractf(fabsf(r[j])) - 0.5f) <= kTieMargin;
  }
  if (near) {
#pragma unroll
    for (int j = 0; j < 16; ++j) r[j] = static_cast<float>(quant(v[j], s));
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) qb[j] = __float_as_uint(r[j] + kRoundMagic);
}

// The low bytes of four dwords packed little-endian into one dword.
__device__ inline uint32_t pack_low_bytes(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
  const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);  // b0.0, b1.0, 0, 0
  const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);  // b2.0, b3.0, 0, 0
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// Four int8 values (each in [-127, 127]) packed little-endian into one dword.
__device__ inline int pack4(int q0, int q1, int q2, int q3) {
  return static_cast<int>((static_cast<uint32_t>(q0) & 0xffu) | ((static_cast<uint32_t>(q1) & 0xffu) << 8) |
                          ((static_cast<uint32_t>(q2) & 0xffu) << 16) | (static_cast<uint32_t>(q3) << 24));
}

inline int hip_status() { return hipGetLastError() == hipSuccess ? I2S_OK : I2S_EHIP; }
inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

inline int parts_for(int64_t units) {
  if (units < 1) return 1;
  return units < kMaxParts ? static_cast<int>(units) : kMaxParts;
}

// ---------------------------------------------------------------------------
// F32 -> I8_S over a whole tensor.  Both passes walk the tensor in chunks of
// 16 values (four float4 loads per thread-step); the last n % 16 values are
// handled one by one by workgroup 0.

__global__ void __launch_bounds__(kThreads) i8s_absmax_kernel(const float *__restrict__ x, int64_t n,
                                                              float *__restrict__ parts) {
  __shared__ float red[4];
  const int64_t chunks = n / 16;
  float m = 0.0f;
  for (int64_t c = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x; c < chunks;
       c += static_cast<int64_t>(gridDim.x) * kThreads) {
    const float4 *p = reinterpret_cast<const float4 *>(x + 16 * c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 v = p[j];
      m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
  }
  if (blockIdx.x == 0 && threadIdx.x < n - 16 * chunks) m = fmaxf(m, fabsf(x[16 * chunks + threadIdx.x]));
  m = block_max(m, red);
  if (threadIdx.x == 0) parts[blockIdx.x] = m;
}

__global__ void __launch_bounds__(kThreads) i8s_quantize_kernel(const float *__restrict__ x, int64_t n,
                                                                const float *__restrict__ parts, int nparts,
                                                                uint8_t *__restrict__ out) {
  __shared__ float red[4];
  const float s = scale_from_parts(parts, nparts, red);
  if (blockIdx.x == 0) write_slot(out + n, s);
  const int64_t chunks = n / 16;
  for (int64_t c = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x; c < chunks;
       c += static_cast<int64_t>(gridDim.x) * kThreads) {
    const float4 *p = reinterpret_cast<const float4 *>(x + 16 * c);
    v4i pk;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 v = p[j];
      pk[j] = pack4(quant(v.x, s), quant(v.y, s), quant(v.z, s), quant(v.w, s));
    }
    *reinterpret_cast<v4i *>(out + 16 * c) = pk;
  }
  if (blockIdx.x == 0 && threadIdx.x < n - 16 * chunks) {
    const int64_t i = 16 * chunks + threadIdx.x;
    out[i] = static_cast<uint8_t>(quant(x[i], s));
  }
}

__global__ void __launch_bounds__(kThreads) i8s_dequantize_kernel(const uint8_t *__restrict__ t, int64_t n,
                                                                  float *__restrict__ y) {
  const float s = load_scale(t + n);
  const int64_t chunks = n / 16;
  for (int64_t c = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x; c < chunks;
       c += static_cast<int64_t>(gridDim.x) * kThreads) {
    const v4i pk = *reinterpret_cast<const v4i *>(t + 16 * c);
    float4 *p = reinterpret_cast<float4 *>(y + 16 * c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int w = pk[j];
      p[j] = make_float4(static_cast<float>(static_cast<int8_t>(w)) * s,
                         static_cast<float>(static_cast<int8_t>(w >> 8)) * s,
                         static_cast<float>(static_cast<int8_t>(w >> 16)) * s,
                         static_cast<float>(static_cast<int8_t>(w >> 24)) * s);
    }
  }
  if (blockIdx.x == 0 && threadIdx.x < n - 16 * chunks) {
    const int64_t i = 16 * chunks + threadIdx.x;
    y[i] = static_cast<float>(static_cast<int8_t>(t[i])) * s;
  }
}

// ---------------------------------------------------------------------------
// mul_mat_add arguments shared by both passes and both contraction kernels.

struct MatArgs {
  // Every member has a default, so a default-constructed MatArgs is inert:
  // null pointers (no bias, no dot output, no F32 output) and zero sizes.
  const int8_t *w = nullptr;      // [OC][IC] payload
  const int8_t *x = nullptr;      // [N][IC] payload
  const uint8_t *ws = nullptr;    // in-band scale of w
  const uint8_t *xs = nullptr;    // in-band scale of x
  const float *bias = nullptr;    // [OC] or null
  float *parts = nullptr;         // pass 1 writes parts[blockIdx.x]; pass 2 reads nparts of them
  int8_t *out = nullptr;          // [N][OC] payload (pass 2)
  int32_t *dot = nullptr;         // [N][OC] or null (pass 2)
  int64_t OC = 0, IC = 0, N = 0;
  int nparts = 0;
  int relu = 0;
  int vec = 0;                    // OC % 16 == 0: 16-byte int8 stores, 16-byte dot stores
                                  // (W8A8: OC % 4 == 0 and y, dot 16-byte aligned)
  const float *cscale = nullptr;  // W8A8: per-channel weight scales [OC]
  const float *rscale = nullptr;  // W8A8: per-row activation scales [N]
  float *y = nullptr;             // W8A8: [N][OC] F32 output
  int map = 0;                    // tile assignment: kMapStride, kMapXLocal or kMapWLocal
  int rep = 1;                    // XCD-local maps: workgroups per XCD per block of the local operand
};

// The contraction kernels take MatArgs as scalar arguments: the launch
// preloads the first 14 argument dwords into SGPRs (a struct argument is
// never preloaded), so the operand pointers, the sizes (as 32-bit values),
// the tile map and the per-channel vector (the bias, or W8A8's weight
// scales) and W8A8's row scales come first -- everything the first loads
// need, with the grid size (gridDim.x is itself an argument load) -- and
// the kernel rebuilds its MatArgs from them.  cvec serves as
// both bias and cscale: the F32 (W8A8) kernels read only cscale, the others
// only bias.  The tenth argument is the row scales in F32 mode and the
// partial maxima (the same array as parts) otherwise, so that the
// quantizing pass finds them in a preloaded dword; it aliases parts, hence
// no restrict on it.
#define I8S_KARGS                                                                                                \
  const int8_t *__restrict__ kw, const int8_t *__restrict__ kx, int kOC, int kIC, int kN, int kmap, int krep, int kG, \
      const float *__restrict__ kcvec, const float *krscale, int kvec, const uint8_t *__restrict__ kws,           \
      const uint8_t *__restrict__ kxs, float *__restrict__ kparts, int8_t *__restrict__ kout,                   \
      int32_t *__restrict__ kdot, float *__restrict__ ky, int knparts, int krelu
#define I8S_KARGS_OF(a, f32, g)                                                                                  \
  (a).w, (a).x, static_cast<int>((a).OC), static_cast<int>((a).IC), static_cast<int>((a).N), (a).map, (a).rep,  \
      static_cast<int>(g), (f32) ? (a).cscale : (a).bias, (f32) ? (a).rscale : (a).parts, (a).vec, (a).ws,     \
      (a).xs, (a).parts, (a).out, (a).dot, (a).y, (a).nparts, (a).relu
#define I8S_MAT_ARGS()                                                                                           \
  MatArgs a;                                                                                                     \
  a.w = kw;                                                                                                      \
  a.x = kx;                                                                                                      \
  a.OC = kOC;                                                                                                    \
  a.IC = kIC;                                                                                                    \
  a.N = kN;                                                                                                      \
  a.map = kmap;                                                                                                  \
  a.rep = krep;                                                                                                  \
  a.vec = kvec;                                                                                                  \
  a.bias = kcvec;                                                                                                \
  a.cscale = kcvec;                                                                                              \
  a.rscale = krscale;                                                                                            \
  a.ws = kws;                                                                                                    \
  a.xs = kxs;                                                                                                    \
  a.parts = kparts;                                                                                              \
  a.out = kout;                                                                                                  \
  a.dot = kdot;                                                                                                  \
  a.y = ky;                                                                                                      \
  a.nparts = knparts;                                                                                            \
  a.relu = krelu

// Tile assignment of the MFMA contraction.  Workgroup b runs on XCD b % 8
// (workgroups are dealt round-robin over the 8 XCDs, each with its own L2).
//   kMapStride: tiles b, b + G, b + 2G, ... (channel block fastest).
//   kMapXLocal: XCD x takes the row blocks nb = x (mod 8) with every channel
//     block, so each block of activations is fetched by one XCD only and the
//     (smaller) weights are fetched once per XCD; a workgroup keeps one channel
//     block and steps its row block by 8 * rep.
//   kMapWLocal: the same with the roles swapped, for weights larger than the
//     activations.
constexpr int kMapStride = 0, kMapXLocal = 1, kMapWLocal = 2;
constexpr int kXcds = 8;

// Epilogues of the MFMA contraction: the two passes of mul_mat_add, and the
// F32 dequantization of the per-channel W8A8 product.
constexpr int kModeMax = 0, kModeQuant = 1, kModeF32 = 2;

// f of one output from its accumulator: (float)acc * t, + bias, ReLU.
__device__ inline float value_of(int32_t acc, float t, float b, bool has_bias, int relu) {
  float v = static_cast<float>(acc) * t;
  if (has_bias) v = v + b;
  if (relu && !(v > 0.0f)) v = 0.0f;
  return v;
}

// Plain per-output contraction for any IC (byte loads); one thread per
// output, grid-stride.  Used when IC % 16 != 0.
template <bool QUANT>
__global__ void __launch_bounds__(kThreads) i8s_mm_plain_kernel(I8S_KARGS) {
  I8S_MAT_ARGS();
  __shared__ float red[4];
  const float t = load_scale(a.ws) * load_scale(a.xs);
  float s = 1.0f;
  if constexpr (QUANT) {
    s = scale_from_parts(a.parts, a.nparts, red);
    if (blockIdx.x == 0) write_slot(reinterpret_cast<uint8_t *>(a.out) + a.N * a.OC, s);
  }
  float m = 0.0f;
  const int64_t total = a.N * a.OC;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x; i < total;
       i += static_cast<int64_t>(kG) * kThreads) {
    const int64_t n = i / a.OC, o = i - n * a.OC;
    const int8_t *wr = a.w + o * a.IC;
    const int8_t *xr = a.x + n * a.IC;
    int32_t acc = 0;
    for (int64_t k = 0; k < a.IC; ++k) acc += static_cast<int32_t>(wr[k]) * static_cast<int32_t>(xr[k]);
    const float v = value_of(acc, t, a.bias ? a.bias[o] : 0.0f, a.bias != nullptr, a.relu);
    if constexpr (QUANT) {
      a.out[i] = static_cast<int8_t>(quant(v, s));
      if (a.dot) a.dot[i] = acc;
    } else {
      m = fmaxf(m, fabsf(v));
    }
  }
  if constexpr (!QUANT) {
    m = block_max(m, red);
    if (threadIdx.x == 0) a.parts[blockIdx.x] = m;
  }
}

// int8 MFMA contraction (v_mfma_i32_16x16x64_i8), IC % 16 == 0.
//
// A workgroup owns TM output channels x TN activation rows per tile and walks
// tiles with a grid stride (the grid is at most kMaxParts workgroups, one
// partial maximum each; the host makes it a multiple of the number of channel
// blocks when it can, so that a workgroup keeps one channel block).  Four
// waves; each wave owns 64 channels x TN/WAVES_N rows, i.e. 4 channel blocks x
// FN row blocks of 16 x 16.
//
// Work items are (tile, K chunk) pairs, a chunk being KS steps of 64 bytes.
// For each item all 256 threads load the chunk's rows into registers (four
// consecutive lanes read one row's 64 contiguous bytes of a step), then store
// them to LDS; right after the store they issue the next item's loads -- the
// next chunk, or the first chunk of the next tile -- so that memory latency
// overlaps this item's MFMAs and the epilogue.  One LDS buffer, two barriers
// per item.
//
// LDS layout of a step: row r's 16-byte chunk c at r*64 + 16*(c ^ sw(r)),
// sw(r) = ((r >> 2) ^ (r >> 4)) & 3.  Sixteen lanes reading chunk c of rows
// r0..r0+15 (activation operand) or of rows {16p + 4b + j} (weight operand,
// below) then touch sixteen different 16-byte bank groups, and four lanes
// writing one row's four chunks fill 64 contiguous bytes.
//
// Channel order inside a wave: MFMA block b's operand row i is channel
// 16*(i>>2) + 4*b + (i&3) of the wave's 64.  The accumulator element r of
// lane (li, kq) in block b is MFMA row 4*kq + r, i.e. channel
// 16*kq + 4*b + r: lane (li, kq) ends up holding the 16 consecutive channels
// 16*kq .. 16*kq+15 of activation row li -- one 16-byte int8 store.
//
// Pass 1 needs max|f| only.  For a fixed channel, f = max(fl(fl(acc) * t) +
// b, lo) is a monotone function of acc (every rounding is monotone; the
// direction is the sign of t), so max|f| over a set of rows is reached at the
// smallest or the largest acc among them.  Each lane therefore keeps, per
// channel, the min and max of its valid accumulators (two integer operations
// per output) and evaluates f at those two points when its channel block
// changes or at the end -- exactly the maximum the definition asks for.
//
// The bias is always added (0 for a missing bias: adding +0 only turns a -0
// into +0, which neither |f| nor q can see), and lo is 0 for the relu form and
// -inf otherwise, so the value has no data-dependent branch.
template <int TM, int TN, int KS, int MODE>
__global__ void __launch_bounds__(kThreads) i8s_mm_mfma_kernel(I8S_KARGS) {
  I8S_MAT_ARGS();
  constexpr bool QUANT = MODE == kModeQuant;
  constexpr int WAVES_M = TM / 64;
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int WTN = TN / WAVES_N;  // activation rows per wave
  constexpr int FN = WTN / 16;
  constexpr int LA = TM * 64, LB = TN * 64;  // bytes of one 64-byte step of each operand
  constexpr int LS = LA + LB;
  constexpr int RA = TM / 64, RB = TN / 64;  // 16-byte loads per thread per step
  static_assert(WAVES_M * WAVES_N == 4 && FN >= 1 && RA >= 1 && RB >= 1, "tile shape");
  __shared__ __attribute__((aligned(16))) int8_t lds[KS * LS];
  __shared__ __attribute__((aligned(16))) float lbias[TM];  // bias (W8A8: weight scales) of the item's channels
  __shared__ float lrs[MODE == kModeF32 ? TN : 1];           // W8A8: activation scales of the item's rows
  __shared__ float red[4];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, kq = lane >> 4;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  const int OC = static_cast<int>(a.OC), IC = static_cast<int>(a.IC), N = static_cast<int>(a.N);
  const __amdgpu_buffer_rsrc_t wbuf = buffer_of(a.w, static_cast<uint32_t>(a.OC * a.IC));
  const __amdgpu_buffer_rsrc_t xbuf = buffer_of(a.x, static_cast<uint32_t>(a.N * a.IC));
  const float *cvec = MODE == kModeF32 ? a.cscale : a.bias;
  const __amdgpu_buffer_rsrc_t bbuf = buffer_of(cvec, cvec ? static_cast<uint32_t>(a.OC * 4) : 0u);
  const __amdgpu_buffer_rsrc_t rbuf = buffer_of(a.rscale, MODE == kModeF32 ? static_cast<uint32_t>(a.N * 4) : 0u);
  const __amdgpu_buffer_rsrc_t ybuf = buffer_of(a.y, MODE == kModeF32 ? static_cast<uint32_t>(a.N * a.OC * 4) : 0u);
  const __amdgpu_buffer_rsrc_t obuf = buffer_of(a.out, static_cast<uint32_t>(a.N * a.OC));
  const __amdgpu_buffer_rsrc_t dbuf = buffer_of(a.dot, a.dot ? static_cast<uint32_t>(a.N * a.OC * 4) : 0u);

  // Tiles: channel block ob = tile % tiles_o, row block nb = tile / tiles_o;
  // this workgroup takes tiles blockIdx.x, +G, +2G, ...  Cursors step through
  // them (and through the K chunks of each) without divisions.
  const int tiles_o = (OC + TM - 1) / TM, tiles_n = (N + TN - 1) / TN;
  const int tiles = tiles_o * tiles_n;
  const int G = kG, b = static_cast<int>(blockIdx.x);
  const int kchunks = IC > 0 ? (IC + 64 * KS - 1) / (64 * KS) : 1;
  struct Cursor {
    int ob, nb, kc;
  };
  Cursor first = {0, 0, 0};
  int my_tiles = 0, step_o = 0, step_n = 0;
  if (tiles == 0) {
    // empty output: no tile (pass 1 still writes its partial, pass 2 the scale slot)
  } else if (a.map == kMapStride) {
    first = {b % tiles_o, b / tiles_o, 0};
    step_o = G % tiles_o;
    step_n = G / tiles_o;
    my_tiles = b < tiles ? (tiles - b + G - 1) / G : 0;
  } else {
    const int xcd = b % kXcds, sl = b / kXcds, stride = kXcds * a.rep;
    const int fixed_n = a.map == kMapXLocal ? tiles_o : tiles_n;  // blocks of the replicated operand
    const int fixed = sl % fixed_n, start = xcd + kXcds * (sl / fixed_n);
    const int local_n = a.map == kMapXLocal ? tiles_n : tiles_o;
    my_tiles = start < local_n ? (local_n - start + stride - 1) / stride : 0;
    if (a.map == kMapXLocal) {
      first = {fixed, start, 0};
      step_o = 0;
      step_n = stride;
    } else {
      first = {start, fixed, 0};
      step_o = stride;
      step_n = 0;
    }
  }
  const int items = my_tiles * kchunks;
  auto advance = [&](Cursor &c) {
    if (++c.kc < kchunks) return;
    c.kc = 0;
    c.ob += step_o;
    c.nb += step_n;
    if (a.map == kMapStride && c.ob >= tiles_o) {
      c.ob -= tiles_o;
      c.nb += 1;
    }
  };
  const int lrow = tid >> 2, lchunk = tid & 3;  // this thread's load slot: row lrow (+64j), chunk lchunk

  auto swz = [](int r, int c) { return r * 64 + 16 * (c ^ (((r >> 2) ^ (r >> 4)) & 3)); };

  // Each item's loads include the bias of its channel block (thread t < TM
  // loads channel o0 + t; 0 past OC or without a bias), staged through LDS
  // with the operands so that no epilogue waits on global memory.
  v4i ra[KS][RA], rb[KS][RB];
  float rbias = 0.0f;
  auto gload = [&](const Cursor &c) {
    const int o0 = c.ob * TM, n0 = c.nb * TN;
    if (tid < TM)
      rbias = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          bbuf, o0 + tid < OC ? static_cast<uint32_t>(4 * (o0 + tid)) : kOutOfRange, 0, 0));
    else if (MODE == kModeF32 && tid < TM + TN)
      rbias = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          rbuf, n0 + tid - TM < N ? static_cast<uint32_t>(4 * (n0 + tid - TM)) : kOutOfRange, 0, 0));
    const int kbase = c.kc * (64 * KS) + 16 * lchunk;
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      const int k = kbase + 64 * st;
      const bool kok = k < IC;
#pragma unroll
      for (int j = 0; j < RA; ++j) {
        const int o = o0 + lrow + 64 * j;
        ra[st][j] = __builtin_amdgcn_raw_buffer_load_b128(
            wbuf, kok && o < OC ? static_cast<uint32_t>(o) * static_cast<uint32_t>(IC) + k : kOutOfRange, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        const int n = n0 + lrow + 64 * j;
        rb[st][j] = __builtin_amdgcn_raw_buffer_load_b128(
            xbuf, kok && n < N ? static_cast<uint32_t>(n) * static_cast<uint32_t>(IC) + k : kOutOfRange, 0, 0);
      }
    }
  };
  auto lstore = [&]() {
    if (tid < TM) lbias[tid] = rbias;
    else if (MODE == kModeF32 && tid < TM + TN) lrs[tid - TM] = rbias;
#pragma unroll
    for (int st = 0; st < KS; ++st) {
#pragma unroll
      for (int j = 0; j < RA; ++j) *reinterpret_cast<v4i *>(&lds[st * LS + swz(lrow + 64 * j, lchunk)]) = ra[st][j];
#pragma unroll
      for (int j = 0; j < RB; ++j) *reinterpret_cast<v4i *>(&lds[st * LS + LA + swz(lrow + 64 * j, lchunk)]) = rb[st][j];
    }
  };
  // Bias of this lane's 16 channels, from LDS (the current item's block).
  auto lds_bias = [&](float (&bv)[16]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 b4 = *reinterpret_cast<const float4 *>(&lbias[wm * 64 + 16 * kq + 4 * j]);
      bv[4 * j] = b4.x;
      bv[4 * j + 1] = b4.y;
      bv[4 * j + 2] = b4.z;
      bv[4 * j + 3] = b4.w;
    }
  };

  // Prologue: the first item's loads go out before anything waits on memory
  // (the in-band scales, and in pass 2 the partial maxima), so that those
  // latencies overlap.
  Cursor lc = first, cc = first;
  if (items > 0) gload(lc);
  const float ws = MODE == kModeF32 ? 1.0f : load_scale(a.ws), xs = MODE == kModeF32 ? 1.0f : load_scale(a.xs);
  const float lo = a.relu ? 0.0f : -INFINITY;
  float s = 1.0f, inv = 1.0f;
  if constexpr (QUANT) {
    s = scale_from_parts(a.parts, a.nparts, red);
    inv = 1.0f / s;
    if (blockIdx.x == 0) write_slot(reinterpret_cast<uint8_t *>(a.out) + a.N * a.OC, s);
  }
  const float t = ws * xs;

  v4i acc[FN][4];
#pragma unroll
  for (int fn = 0; fn < FN; ++fn)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[fn][b] = v4i{0, 0, 0, 0};

  // Pass 1 state: per-channel extremes of the valid accumulators of the
  // current channel block, and the running max|f|.
  int32_t amx[16], amn[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    amx[j] = INT32_MIN;
    amn[j] = INT32_MAX;
  }
  int cur_ob = -1;
  float m = 0.0f;
  float bcur[16];  // bias of the channel block being accumulated
  auto flush = [&]() {
    const float(&bv)[16] = bcur;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (amx[j] >= amn[j]) {  // the lane saw a valid row of this channel
        const float f1 = fmaxf(static_cast<float>(amx[j]) * t + bv[j], lo);
        const float f2 = fmaxf(static_cast<float>(amn[j]) * t + bv[j], lo);
        m = fmaxf(m, fmaxf(fabsf(f1), fabsf(f2)));
      }
      amx[j] = INT32_MIN;
      amn[j] = INT32_MAX;
    }
  };

  for (int it = 0; it < items; ++it) {
    __syncthreads();  // every wave is done reading the previous item from LDS
    lstore();
    __syncthreads();
    if (it + 1 < items) {
      advance(lc);
      gload(lc);
    }
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      v4i af[4], bf[FN];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int r = wm * 64 + 16 * (li >> 2) + 4 * b + (li & 3);
        af[b] = *reinterpret_cast<const v4i *>(&lds[st * LS + swz(r, kq)]);
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int r = wn * WTN + 16 * fn + li;
        bf[fn] = *reinterpret_cast<const v4i *>(&lds[st * LS + LA + swz(r, kq)]);
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[fn][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[b], bf[fn], acc[fn][b], 0, 0, 0);
    }
    const Cursor ec = cc;
    advance(cc);
    if (ec.kc + 1 < kchunks) continue;

    // Epilogue of the tile: lane (li, kq) holds channels og .. og+15 of
    // activation row n.
    const int o0 = ec.ob * TM, n0 = ec.nb * TN;
    const int og = o0 + wm * 64 + 16 * kq;
    if constexpr (MODE == kModeF32) {
      float cs[16];
      lds_bias(cs);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int nl = wn * WTN + 16 * fn + li;
        const int n = n0 + nl;
        const float rs = lrs[nl];
        v4i yv[4];
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            yv[b][r] = __float_as_int(rs * cs[4 * b + r] * static_cast<float>(acc[fn][b][r]));
        const uint32_t row = static_cast<uint32_t>(n) * static_cast<uint32_t>(OC);
        const bool n_ok = n < N;
        if (a.vec) {
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const uint32_t off = n_ok && og + 4 * b < OC ? 4 * (row + og + 4 * b) : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b128(yv[b], ybuf, off, 0, 0);
            if (a.dot) __builtin_amdgcn_raw_buffer_store_b128(acc[fn][b], dbuf, off, 0, 0);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const uint32_t off = n_ok && og + j < OC ? 4 * (row + og + j) : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b32(yv[j >> 2][j & 3], ybuf, off, 0, 0);
            if (a.dot) __builtin_amdgcn_raw_buffer_store_b32(acc[fn][j >> 2][j & 3], dbuf, off, 0, 0);
          }
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[fn][b] = v4i{0, 0, 0, 0};
      }
    } else if constexpr (MODE == kModeMax) {
      if (ec.ob != cur_ob) {
        if (cur_ob >= 0) flush();
        cur_ob = ec.ob;
        lds_bias(bcur);
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        if (n0 + wn * WTN + 16 * fn + li < N) {
#pragma unroll
          for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              amx[4 * b + r] = max(amx[4 * b + r], acc[fn][b][r]);
              amn[4 * b + r] = min(amn[4 * b + r], acc[fn][b][r]);
            }
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[fn][b] = v4i{0, 0, 0, 0};
      }
    } else {
      float bv[16];
      lds_bias(bv);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int n = n0 + wn * WTN + 16 * fn + li;
        const bool n_ok = n < N;
        float v[16];
        uint32_t q[16];  // q in the low byte of each
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) v[4 * b + r] = fmaxf(static_cast<float>(acc[fn][b][r]) * t + bv[4 * b + r], lo);
        quant16(v, s, inv, q);
        const uint32_t row = static_cast<uint32_t>(n) * static_cast<uint32_t>(OC);
        if (a.vec) {
          v4i pk;
#pragma unroll
          for (int b = 0; b < 4; ++b)
            pk[b] = static_cast<int>(pack_low_bytes(q[4 * b], q[4 * b + 1], q[4 * b + 2], q[4 * b + 3]));
          const uint32_t off = n_ok && og < OC ? row + og : kOutOfRange;
          __builtin_amdgcn_raw_buffer_store_b128(pk, obuf, off, 0, 0);
          if (a.dot) {
#pragma unroll
            for (int b = 0; b < 4; ++b)
              __builtin_amdgcn_raw_buffer_store_b128(acc[fn][b], dbuf, off == kOutOfRange ? kOutOfRange : 4 * (off + 4 * b),
                                                     0, 0);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const uint32_t off = n_ok && og + j < OC ? row + og + j : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(q[j]), obuf, off, 0, 0);
            if (a.dot)
              __builtin_amdgcn_raw_buffer_store_b32(acc[fn][j >> 2][j & 3], dbuf, off == kOutOfRange ? kOutOfRange : 4 * off,
                                                    0, 0);
          }
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[fn][b] = v4i{0, 0, 0, 0};
      }
    }
  }
  if constexpr (MODE == kModeMax) {
    if (cur_ob >= 0) flush();
    m = block_max(m, red);
    if (threadIdx.x == 0) a.parts[blockIdx.x] = m;
  }
}

// ---------------------------------------------------------------------------
// W8A8 activation-resident int8-MFMA contraction (the prefill shapes, W8A8
// variant 10).  A workgroup of 8 waves copies its tile of 64 activation rows
// (K bytes each, row pitch K + 16) into LDS once; each wave then streams the
// int8 weights of its 16-row subtiles (wave, wave + 8, ..., G at a time) in
// batches of KST 64-position chunks, the next batch's loads in flight while
// the current one's MFMAs run, with no further barrier.  Weights are loaded
// row-contiguously (lane l: row l/4, bytes 16*(l%4) of the chunk: 4
// consecutive lanes read 64 contiguous bytes) and moved into MFMA lane order
// by ds_bpermute; each weight operand feeds 4 MFMAs (the 4 blocks of 16
// activation rows) whose B operands come from LDS.  Epilogue as the tile
// kernel's F32 mode: y = (aScale * wScale) * (float)acc.

template <int G, int KST, bool VEC4>
__global__ void __launch_bounds__(512)
w8a8_res_kernel(const int8_t *__restrict__ wq, const float *__restrict__ wscale, int OC, int K,
                const int8_t *__restrict__ aq, const float *__restrict__ ascale, int M, float *__restrict__ y,
                int32_t *__restrict__ dot, int tiles_m, int ms) {
  constexpr int WN = 4, BN = 64, W = 8;
  extern __shared__ __attribute__((aligned(16))) int8_t lt[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, kb = lane >> 4;
  const int tile_m = static_cast<int>(blockIdx.x) % tiles_m, tile_n = static_cast<int>(blockIdx.x) / tiles_m;
  const int o_tile = tile_m * ms * 16, n0 = tile_n * BN;
  const int n_here = M - n0 < BN ? M - n0 : BN;
  const int pitch = K + 16;
  const int sub_total = (OC - o_tile + 15) / 16;
  const int present = sub_total < ms ? sub_total : ms;  // 16-row subtiles of this tile
  const int mine = present > wave ? (present - wave + W - 1) / W : 0;
  const int groups = (mine + G - 1) / G;
  const int chunks = K / 64;
  const int batches = (chunks + KST - 1) / KST;
  const __amdgpu_buffer_rsrc_t wbuf = buffer_of(wq, static_cast<uint32_t>(OC) * static_cast<uint32_t>(K));
  const __amdgpu_buffer_rsrc_t abuf = buffer_of(aq + static_cast<int64_t>(n0) * K,
                                                static_cast<uint32_t>(n_here) * static_cast<uint32_t>(K));

  // Activation scales of this lane's rows n0 + 16*n + li (0 past M; never stored).
  float asc[WN];
  {
    const __amdgpu_buffer_rsrc_t sbuf = buffer_of(ascale + n0, static_cast<uint32_t>(4 * n_here));
#pragma unroll
    for (int n = 0; n < WN; ++n)
      asc[n] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(sbuf, static_cast<uint32_t>(4 * (16 * n + li)), 0, 0));
  }

  // The activation tile into LDS, 8 pieces of 16 bytes per thread in flight;
  // rows past M read as zero.
  {
    const int ppr = K / 16;  // pieces per row
    const int pieces = BN * ppr;
    for (int p0 = 0; p0 < pieces; p0 += 512 * 8) {
      v4i t[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int p = p0 + 512 * j + tid;
        const int r = p / ppr, c = p - (p / ppr) * ppr;
        t[j] = __builtin_amdgcn_raw_buffer_load_b128(
            abuf, p < pieces && r < n_here ? static_cast<uint32_t>(r * K + 16 * c) : kOutOfRange, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int p = p0 + 512 * j + tid;
        if (p < pieces) {
          const int r = p / ppr, c = p - (p / ppr) * ppr;
          *reinterpret_cast<v4i *>(lt + r * pitch + 16 * c) = t[j];
        }
      }
    }
  }
  __syncthreads();

  const int perm = 4 * (4 * li + kb);  // ds_bpermute source lane (bytes) of MFMA lane (li, kb)
  const int8_t *lb = lt + li * pitch + 16 * kb;
  const __amdgpu_buffer_rsrc_t cbuf = buffer_of(wscale, static_cast<uint32_t>(4 * OC));
  const uint32_t out_bytes = static_cast<uint32_t>(M) * static_cast<uint32_t>(OC) * 4u;
  const __amdgpu_buffer_rsrc_t ybuf = buffer_of(y, out_bytes);
  const __amdgpu_buffer_rsrc_t dbuf = buffer_of(dot, dot ? out_bytes : 0u);

  for (int grp = 0; grp < groups; ++grp) {
    // Row of this lane's loads in subtile gi of the group (past OC or past
    // the tile: an out-of-range offset, reads 0, never stored).
    uint32_t wrow[G];
    bool wok[G];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const int sub = wave + W * (grp * G + gi);
      const int row = o_tile + 16 * sub + (lane >> 2);
      wok[gi] = sub < present && row < OC;
      wrow[gi] = static_cast<uint32_t>(row) * static_cast<uint32_t>(K) + 16u * static_cast<uint32_t>(lane & 3);
    }
    v4i acc[G][WN];
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
#pragma unroll
      for (int n = 0; n < WN; ++n) acc[gi][n] = v4i{0, 0, 0, 0};
    // The group's loads, permutes and MFMAs for its GS subtiles only (a
    // short last group runs none for the subtiles it lacks).
    auto run = [&](auto gsc) {
      constexpr int GS = decltype(gsc)::value;
      auto load = [&](int bt, v4i (&w)[G][KST]) {
#pragma unroll
        for (int gi = 0; gi < GS; ++gi)
#pragma unroll
          for (int kk = 0; kk < KST; ++kk) {
            const int chunk = bt * KST + kk;
            w[gi][kk] = __builtin_amdgcn_raw_buffer_load_b128(
                wbuf, wok[gi] && chunk < chunks ? wrow[gi] + 64u * static_cast<uint32_t>(chunk) : kOutOfRange, 0, 0);
          }
      };
      // Permutes one chunk ahead of its MFMAs (GS operands at a time), so that
      // only two chunks' worth of permuted registers are live.
      auto compute = [&](int bt, const v4i (&w)[G][KST]) {
        v4i pw[2][G];
#pragma unroll
        for (int gi = 0; gi < GS; ++gi)
#pragma unroll
          for (int e = 0; e < 4; ++e) pw[0][gi][e] = __builtin_amdgcn_ds_bpermute(perm, w[gi][0][e]);
#pragma unroll
        for (int kk = 0; kk < KST; ++kk) {
          if (kk + 1 < KST) {
#pragma unroll
            for (int gi = 0; gi < GS; ++gi)
#pragma unroll
              for (int e = 0; e < 4; ++e) pw[(kk + 1) & 1][gi][e] = __builtin_amdgcn_ds_bpermute(perm, w[gi][kk + 1][e]);
          }
          const int chunk = bt * KST + kk;
          if (chunk >= chunks) continue;  // wave-uniform
#pragma unroll
          for (int n = 0; n < WN; ++n) {
            const v4i b = *reinterpret_cast<const v4i *>(lb + 16 * n * pitch + 64 * chunk);
#pragma unroll
            for (int gi = 0; gi < GS; ++gi)
              acc[gi][n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(pw[kk & 1][gi], b, acc[gi][n], 0, 0, 0);
          }
        }
      };
      v4i wa[G][KST], wb[G][KST];
      load(0, wa);
      for (int bt = 0; bt < batches; bt += 2) {
        load(bt + 1, wb);
        compute(bt, wa);
        if (bt + 1 >= batches) break;
        load(bt + 2, wa);
        compute(bt + 1, wb);
      }
    };
    const int gs = mine - grp * G < G ? mine - grp * G : G;
    if (gs == G) {
      run(std::integral_constant<int, G>{});
    } else {
      switch (gs) {
        case 1: run(std::integral_constant<int, 1>{}); break;
        case 2: if constexpr (G > 2) run(std::integral_constant<int, 2>{}); break;
        case 3: if constexpr (G > 3) run(std::integral_constant<int, 3>{}); break;
        default: break;
      }
    }

    // Lane (li, kb) holds, per subtile gi, weight rows o + r (o = o_tile +
    // 16*sub + 4*kb, r = 0..3) of activation rows n0 + 16*n + li.
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const int sub = wave + W * (grp * G + gi);
      if (sub >= present) continue;  // wave-uniform
      const int o = o_tile + 16 * sub + 4 * kb;
      float cs[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        cs[r] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(cbuf, o + r < OC ? static_cast<uint32_t>(4 * (o + r)) : kOutOfRange, 0, 0));
#pragma unroll
      for (int n = 0; n < WN; ++n) {
        const int m = n0 + 16 * n + li;
        const bool m_ok = m < M;
        const uint32_t row = static_cast<uint32_t>(m_ok ? m : 0) * static_cast<uint32_t>(OC);
        v4i yv;
#pragma unroll
        for (int r = 0; r < 4; ++r) yv[r] = __float_as_int(asc[n] * cs[r] * static_cast<float>(acc[gi][n][r]));
        if constexpr (VEC4) {
          const uint32_t off = m_ok && o < OC ? 4u * (row + static_cast<uint32_t>(o)) : kOutOfRange;
          __builtin_amdgcn_raw_buffer_store_b128(yv, ybuf, off, 0, 0);
          if (dot) __builtin_amdgcn_raw_buffer_store_b128(acc[gi][n], dbuf, off, 0, 0);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t off = m_ok && o + r < OC ? 4u * (row + static_cast<uint32_t>(o + r)) : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b32(yv[r], ybuf, off, 0, 0);
            if (dot) __builtin_amdgcn_raw_buffer_store_b32(acc[gi][n][r], dbuf, off, 0, 0);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Skinny int8 MFMA contraction for few activation rows (the encoder's last
// stages and connector, W8A8 decode): the tile kernel above would have only a
// few dozen tiles there.  A workgroup of W waves owns 16 output channels and
// up to 16 * FN activation rows; its waves take the 64-byte K-steps
// round-robin, SPW steps per batch with the next batch's loads in flight,
// and sum their int32 partial tiles through LDS.  Lane (li, kq) loads row li
// of each operand block at bytes 16 * kq of a step (the MFMA operand order).
// Wave 0 finishes: it holds channels o0 + 4 * kq + r (r = 0..3) of row
// n0 + 16 * fn + li, and applies the same epilogue as the tile kernel (max|f|,
// requantization with the exact division, or the W8A8 dequantization).
// Items (16-channel block, 16*FN-row block) are walked with a grid stride.

template <int W>
__device__ inline float wave_group_max(float v, float *red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < W; ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

template <int W, int FN, int SPW, int MODE>
__global__ void __launch_bounds__(64 * W) i8s_mm_skinny_kernel(I8S_KARGS) {
  I8S_MAT_ARGS();
  __shared__ __attribute__((aligned(16))) v4i part[W][FN][64];
  __shared__ float red[W];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, kq = lane >> 4;
  const int OC = static_cast<int>(a.OC), IC = static_cast<int>(a.IC), N = static_cast<int>(a.N);
  const __amdgpu_buffer_rsrc_t wbuf = buffer_of(a.w, static_cast<uint32_t>(a.OC * a.IC));
  const __amdgpu_buffer_rsrc_t xbuf = buffer_of(a.x, static_cast<uint32_t>(a.N * a.IC));
  const float *cvec = MODE == kModeF32 ? a.cscale : a.bias;
  const __amdgpu_buffer_rsrc_t bbuf = buffer_of(cvec, cvec ? static_cast<uint32_t>(a.OC * 4) : 0u);
  const __amdgpu_buffer_rsrc_t rbuf = buffer_of(a.rscale, MODE == kModeF32 ? static_cast<uint32_t>(a.N * 4) : 0u);

  // Quant mode: the Max pass ran on this same grid and left one maximum per
  // workgroup, kG of them, at the tenth argument (which carries the per-row
  // scales in F32 mode).  This thread's first one is loaded behind the first
  // item's first operand batch and the tensor scale is reduced after that
  // item's K-loop, so that the two memory latencies overlap.
  const __amdgpu_buffer_rsrc_t pbuf = buffer_of(a.rscale, MODE == kModeQuant ? static_cast<uint32_t>(4 * kG) : 0u);
  float s = 1.0f;
  bool have_s = MODE != kModeQuant;
  auto tensor_scale = [&](float pm) {
    for (int i = tid + 64 * W; i < kG; i += 64 * W) pm = fmaxf(pm, a.rscale[i]);
    float r = wave_group_max<W>(pm, red);
    if (r < kAmaxFloor) r = kAmaxFloor;
    s = r / 127.0f;
    int8_t *outp = a.out;  // pinned here so that its address is not computed ahead of the loads
    __asm__ volatile("" : "+s"(outp));
    if (blockIdx.x == 0) write_slot(reinterpret_cast<uint8_t *>(outp) + a.N * a.OC, s);
    have_s = true;
  };

  const int blocks_o = (OC + 15) / 16, blocks_n = (N + 16 * FN - 1) / (16 * FN);
  const int items = blocks_o * blocks_n;
  const int steps = (IC + 63) / 64;
  float m = 0.0f;
  for (int item = blockIdx.x; item < items; item += kG) {
    const int o0 = (item % blocks_o) * 16, n0 = (item / blocks_o) * (16 * FN);
    const bool o_ok = o0 + li < OC;
    // Epilogue constants of this lane (channels o0 + 4*kq + r; rows
    // n0 + 16*fn + li), loaded ahead of the operand stream so that wave 0
    // does not wait on memory before its stores.
    const int oc = o0 + 4 * kq;
    float cv[4], rsv[FN];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      cv[r] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          bbuf, oc + r < OC ? static_cast<uint32_t>(4 * (oc + r)) : kOutOfRange, 0, 0));
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int n = n0 + 16 * fn + li;
      rsv[fn] = MODE == kModeF32 ? __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                                       rbuf, n < N ? static_cast<uint32_t>(4 * n) : kOutOfRange, 0, 0))
                                 : 0.0f;
    }
    const uint32_t wrow = static_cast<uint32_t>(o0 + li) * static_cast<uint32_t>(IC) + 16 * kq;
    uint32_t xrow[FN];
    bool n_ok[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      n_ok[fn] = n0 + 16 * fn + li < N;
      xrow[fn] = static_cast<uint32_t>(n0 + 16 * fn + li) * static_cast<uint32_t>(IC) + 16 * kq;
    }
    // Step slot i of batch g of this wave: K-step wave + W * (SPW * g + i).
    auto load = [&](int g, v4i (&av)[SPW], v4i (&bv)[SPW][FN]) {
#pragma unroll
      for (int i = 0; i < SPW; ++i) {
        const int st = wave + W * (SPW * g + i);
        const bool kok = st < steps && 64 * st + 16 * kq < IC;
        av[i] = __builtin_amdgcn_raw_buffer_load_b128(wbuf, kok && o_ok ? wrow + 64 * st : kOutOfRange, 0, 0);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          bv[i][fn] = __builtin_amdgcn_raw_buffer_load_b128(xbuf, kok && n_ok[fn] ? xrow[fn] + 64 * st : kOutOfRange,
                                                            0, 0);
      }
    };
    v4i acc[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) acc[fn] = v4i{0, 0, 0, 0};
    auto compute = [&](const v4i (&av)[SPW], const v4i (&bv)[SPW][FN]) {
#pragma unroll
      for (int i = 0; i < SPW; ++i)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[fn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[i], bv[i][fn], acc[fn], 0, 0, 0);
    };
    const int mine = steps > wave ? (steps - wave + W - 1) / W : 0;
    const int batches = (mine + SPW - 1) / SPW;
    v4i aa[SPW], ab[SPW], ba[SPW][FN], bb[SPW][FN];
    if (batches > 0) load(0, aa, ba);
    float p0 = 0.0f;  // out of range, and so 0, once the scale is known
    if constexpr (MODE == kModeQuant)
      p0 = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          pbuf, have_s ? kOutOfRange : static_cast<uint32_t>(4 * tid), 0, 0));
    for (int g = 0; g < batches; g += 2) {
      if (g + 1 < batches) load(g + 1, ab, bb);
      compute(aa, ba);
      if (g + 1 >= batches) break;
      if (g + 2 < batches) load(g + 2, aa, ba);
      compute(ab, bb);
    }
    if constexpr (MODE == kModeQuant) {
      if (!have_s) tensor_scale(p0);
    }
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) part[wave][fn][lane] = acc[fn];
    __syncthreads();
    if (wave == 0) {
      // Output descriptors are built here, from pointers the compiler may not
      // hoist, so that the first operand loads wait on no argument outside
      // the preloaded ones.
      int8_t *outp = a.out;
      int32_t *dotp = a.dot;
      float *yp = a.y;
      const uint8_t *wsp = a.ws, *xsp = a.xs;
      int relu = a.relu;
      __asm__ volatile("" : "+s"(outp), "+s"(dotp), "+s"(yp), "+s"(wsp), "+s"(xsp), "+s"(relu));
      const float t = MODE == kModeF32 ? 1.0f : load_scale(wsp) * load_scale(xsp);
      const float lo = relu ? 0.0f : -INFINITY;
      const __amdgpu_buffer_rsrc_t obuf = buffer_of(outp, static_cast<uint32_t>(a.N * a.OC));
      const __amdgpu_buffer_rsrc_t dbuf = buffer_of(dotp, dotp ? static_cast<uint32_t>(a.N * a.OC * 4) : 0u);
      const __amdgpu_buffer_rsrc_t ybuf =
          buffer_of(yp, MODE == kModeF32 ? static_cast<uint32_t>(a.N * a.OC * 4) : 0u);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        v4i tot = part[0][fn][lane];
#pragma unroll
        for (int w = 1; w < W; ++w) tot += part[w][fn][lane];
        acc[fn] = tot;
      }
      // Lane (li, kq): channels o0 + 4*kq + r of row n0 + 16*fn + li.
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int n = n0 + 16 * fn + li;
        const uint32_t row = static_cast<uint32_t>(n) * static_cast<uint32_t>(OC);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ok = n < N && oc + r < OC;
          const uint32_t off = ok ? row + oc + r : kOutOfRange;
          if constexpr (MODE == kModeF32) {
            const float y = rsv[fn] * cv[r] * static_cast<float>(acc[fn][r]);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(y), ybuf, ok ? 4 * off : kOutOfRange, 0, 0);
          } else {
            const float v = fmaxf(static_cast<float>(acc[fn][r]) * t + cv[r], lo);
            if constexpr (MODE == kModeMax) {
              if (ok) m = fmaxf(m, fabsf(v));
            } else {
              __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(quant(v, s)), obuf, off, 0, 0);
            }
          }
          if (dotp && MODE != kModeMax)
            __builtin_amdgcn_raw_buffer_store_b32(acc[fn][r], dbuf, ok ? 4 * off : kOutOfRange, 0, 0);
        }
      }
    }
    __syncthreads();  // part[] is reused by the next item
  }
  if constexpr (MODE == kModeQuant) {
    // A workgroup with no item still reports the scale.
    if (!have_s)
      tensor_scale(__int_as_float(__builtin_amdgcn_raw_buffer_load_b32(pbuf, static_cast<uint32_t>(4 * tid), 0, 0)));
  }
  if constexpr (MODE == kModeMax) {
    m = wave_group_max<W>(m, red);
    if (threadIdx.x == 0) a.parts[blockIdx.x] = m;
  }
}

// ---------------------------------------------------------------------------
// Per-channel W8A8 row quantizers: one workgroup per row (a weight channel or
// an activation row); the row maximum starts at 1e-9.  Weights: s = mx/127,
// q = rint(w / s) (lrintf's ties to even).  Activations: s = mx/127,
// inv = 127/mx, v = x * inv, q = trunc(v + copysign(0.5, v)).

template <bool WEIGHT>
__global__ void __launch_bounds__(kThreads) w8a8_quant_rows_kernel(const float *__restrict__ x, int64_t K,
                                                                   int8_t *__restrict__ q, float *__restrict__ scale) {
  __shared__ float red[4];
  const float *xr = x + blockIdx.x * K;
  int8_t *qr = q + blockIdx.x * K;
  float mx = 1e-9f;
  for (int64_t k = threadIdx.x; k < K; k += kThreads) mx = fmaxf(mx, fabsf(xr[k]));
  mx = block_max(mx, red);
  const float s = mx / 127.0f;
  if (threadIdx.x == 0) scale[blockIdx.x] = s;
  if constexpr (WEIGHT) {
    for (int64_t k = threadIdx.x; k < K; k += kThreads) {
      const float r = fminf(fmaxf(rintf(xr[k] / s), -127.0f), 127.0f);
      qr[k] = static_cast<int8_t>(static_cast<int>(r));
    }
  } else {
    const float inv = 127.0f / mx;
    for (int64_t k = threadIdx.x; k < K; k += kThreads) {
      const float v = xr[k] * inv;
      const float h = v + copysignf(0.5f, v);
      const int qi = static_cast<int>(fminf(fmaxf(h, -127.0f), 127.0f));
      qr[k] = static_cast<int8_t>(qi);
    }
  }
}

// The activation rounding of the kernel above, for one value.
__device__ inline int w8a8_round_act(float x, float inv) {
  const float v = x * inv;
  const float h = v + copysignf(0.5f, v);
  return static_cast<int>(fminf(fmaxf(h, -127.0f), 127.0f));
}

// The activation quantizer with the row held in registers: W waves per row,
// thread t loads the float4s at 4 * (t + 64 W j), j < R (64 W R >= K / 4),
// all before the first use, takes the row maximum with DPP moves (and, for
// W > 1, through LDS) and writes four codes as one 32-bit store.  Same
// arithmetic as w8a8_quant_rows_kernel<false>, so the same codes and scales.
// Needs K % 4 == 0, x 16-byte and q 4-byte aligned.
template <int R, int W>
__global__ void __launch_bounds__(64 * W) w8a8_quant_act_reg_kernel(const float *__restrict__ x, int64_t K,
                                                                    int8_t *__restrict__ q, float *__restrict__ scale) {
  const int t = threadIdx.x;
  const int K4 = static_cast<int>(K >> 2);
  const float4 *xr = reinterpret_cast<const float4 *>(x + blockIdx.x * K);
  uint32_t *qr = reinterpret_cast<uint32_t *>(q + blockIdx.x * K);
  float4 v[R];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int i = t + 64 * W * j;
    v[j] = i < K4 ? xr[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }
  float mx = 1e-9f;
#pragma unroll
  for (int j = 0; j < R; ++j)
    mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
  if constexpr (W == 1) {
    mx = wave_max(mx);
  } else {
    __shared__ float red[W];
    mx = wave_max(mx);
    if ((t & 63) == 0) red[t >> 6] = mx;
    __syncthreads();
    mx = red[0];
#pragma unroll
    for (int w = 1; w < W; ++w) mx = fmaxf(mx, red[w]);
  }
  if (t == 0) scale[blockIdx.x] = mx / 127.0f;
  const float inv = 127.0f / mx;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int i = t + 64 * W * j;
    if (i < K4) {
      const uint32_t b0 = static_cast<uint32_t>(w8a8_round_act(v[j].x, inv)) & 0xFFu;
      const uint32_t b1 = static_cast<uint32_t>(w8a8_round_act(v[j].y, inv)) & 0xFFu;
      const uint32_t b2 = static_cast<uint32_t>(w8a8_round_act(v[j].z, inv)) & 0xFFu;
      const uint32_t b3 = static_cast<uint32_t>(w8a8_round_act(v[j].w, inv)) & 0xFFu;
      qr[i] = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
    }
  }
}

constexpr int kActRegMaxR = 36;          // float4s a thread holds at most
constexpr int64_t kActRegRowsOneWave = 1024;  // rows from which each row gets one wave

template <int R, int W>
void launch_act_reg(const float *x, int64_t M, int64_t K, int8_t *q, float *scale, hipStream_t stream) {
  hipLaunchKernelGGL((w8a8_quant_act_reg_kernel<R, W>), dim3(static_cast<uint32_t>(M)), dim3(64 * W), 0, stream, x,
                     K, q, scale);
}

template <int W>
void launch_act_reg_w(int64_t r, const float *x, int64_t M, int64_t K, int8_t *q, float *scale, hipStream_t stream) {
  if (r <= 2) launch_act_reg<2, W>(x, M, K, q, scale, stream);
  else if (r <= 4) launch_act_reg<4, W>(x, M, K, q, scale, stream);
  else if (r <= 6) launch_act_reg<6, W>(x, M, K, q, scale, stream);
  else if (r <= 9) launch_act_reg<9, W>(x, M, K, q, scale, stream);
  else if (r <= 12) launch_act_reg<12, W>(x, M, K, q, scale, stream);
  else if (r <= 18) launch_act_reg<18, W>(x, M, K, q, scale, stream);
  else if (r <= 24) launch_act_reg<24, W>(x, M, K, q, scale, stream);
  else launch_act_reg<36, W>(x, M, K, q, scale, stream);
}

// Waves per row, as measured on the Qwen2-1.5B row lengths: from 1024 rows
// one wave each fills the chip; fewer rows split each row over four waves,
// and a few long rows (K > 4096, at most 64 rows) over eight.
int act_reg_waves(int64_t M, int64_t K) {
  if (M >= kActRegRowsOneWave) return 1;
  return (K > 4096 && M <= 64) ? 8 : 4;
}

// false where the register quantizer does not take the row (then the
// workgroup-per-row kernel runs).
bool launch_act_reg_fit(const float *x, int64_t M, int64_t K, int8_t *q, float *scale, hipStream_t stream) {
  if (K % 4 != 0 || !aligned(x, 16) || !aligned(q, 4)) return false;
  const int W = act_reg_waves(M, K);
  const int64_t r = (K / 4 + 64 * W - 1) / (64 * W);
  if (r > kActRegMaxR) return false;
  if (W == 1) launch_act_reg_w<1>(r, x, M, K, q, scale, stream);
  else if (W == 4) launch_act_reg_w<4>(r, x, M, K, q, scale, stream);
  else launch_act_reg_w<8>(r, x, M, K, q, scale, stream);
  return true;
}

// ---------------------------------------------------------------------------
// W8A8 decode in one launch: the activation quantizer and an int8 GEMV for
// M <= 4 activation rows (W8A8 variant 11, F32-input entry points only).
//
// Every workgroup quantizes the M rows itself, with the operations of
// w8a8_quant_rows_kernel<false> ("Experiment - int8 W8A8 path (the practical
// default)", Implementation): mx = max(1e-9, max|x|), inv = 127/mx, code =
// w8a8_round_act(x, inv), scale mx/127 -- so the codes and scales are those
// of the two-launch path bit for bit -- into LDS.  It then contracts its
// R = T/L weight rows: L lanes per row, lane j holding the row's 16-byte
// chunks j, j + L, ..., four v_dot4 (int8 x int8 -> int32) per chunk and
// activation row, a sum over the row's L lanes (integer, exact in any
// order), and the epilogue y = (ascale * wscale) * (float)C, the order of
// the page's dequantization.  The activations are loaded before the weights
// (loads retire in order: waiting for x does not wait for the weight
// stream), and every load is unconditional: chunks past K read zeros (their
// products are 0 whatever the LDS bytes they meet), rows past OC read zeros
// and are never stored.  Workgroup 0 also writes the codes and scales where
// the two-launch path's quantizer would.

// Sum over each group of L consecutive lanes (L a power of two up to 64),
// in every lane of the group.
template <int L>
__device__ inline int lanes_sum(int v) {
  static_assert(L >= 1 && L <= 64 && (L & (L - 1)) == 0, "power-of-two lane group");
  if constexpr (L >= 2) v += dpp_move<0xB1>(v);   // quad_perm(1,0,3,2)
  if constexpr (L >= 4) v += dpp_move<0x4E>(v);   // quad_perm(2,3,0,1)
  if constexpr (L >= 8) v += dpp_move<0x141>(v);  // row_half_mirror
  if constexpr (L >= 16) v += dpp_move<0x140>(v); // row_mirror
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

template <int NC, int L, int CPL, int XPT, int T>
__global__ void __launch_bounds__(T) w8a8_gemv_fused_kernel(const int8_t *__restrict__ wq, const float *__restrict__ x,
                                                            int OC, int K, const float *__restrict__ wscale,
                                                            float *__restrict__ y, int32_t *__restrict__ dot,
                                                            int8_t *__restrict__ aq, float *__restrict__ ascale) {
  constexpr int W = T / 64;
  constexpr int R = T / L;  // weight rows per workgroup
  constexpr int kRowBytes = (4 * T * XPT > 16 * L * CPL) ? 4 * T * XPT : 16 * L * CPL;
  __shared__ __attribute__((aligned(16))) int8_t lq[NC][kRowBytes];
  __shared__ float red[NC][W];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rl = tid / L, j = tid % L;
  const int row0 = static_cast<int>(blockIdx.x) * R;
  const int K4 = K >> 2;

  // The activation rows (float4 i of row c at thread i % T, slot i / T).
  const __amdgpu_buffer_rsrc_t xbuf = buffer_of(x, static_cast<uint32_t>(NC * K * 4));
  float4 xv[NC][XPT];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int idx = tid + T * i;
      const v4i t = __builtin_amdgcn_raw_buffer_load_b128(
          xbuf, idx < K4 ? static_cast<uint32_t>(16 * (c * K4 + idx)) : kOutOfRange, 0, 0);
      xv[c][i] = make_float4(__int_as_float(t[0]), __int_as_float(t[1]), __int_as_float(t[2]), __int_as_float(t[3]));
    }
  // This lane's weight chunks and its row's weight scale.
  const __amdgpu_buffer_rsrc_t wbuf =
      buffer_of(wq + static_cast<int64_t>(row0) * K, static_cast<uint32_t>((OC - row0) * K));
  v4i wv[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int ch = j + L * i;
    wv[i] = __builtin_amdgcn_raw_buffer_load_b128(
        wbuf, 16 * ch < K ? static_cast<uint32_t>(rl * K + 16 * ch) : kOutOfRange, 0, 0);
  }
  const __amdgpu_buffer_rsrc_t sbuf = buffer_of(wscale + row0, static_cast<uint32_t>(4 * (OC - row0)));
  const float wsn = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(sbuf, static_cast<uint32_t>(4 * rl), 0, 0));
  __builtin_amdgcn_sched_barrier(0);  // every load is issued before the first use of x

  // Row maxima over the workgroup.
  float mx[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float m = 1e-9f;
#pragma unroll
    for (int i = 0; i < XPT; ++i)
      m = fmaxf(m, fmaxf(fmaxf(fabsf(xv[c][i].x), fabsf(xv[c][i].y)), fmaxf(fabsf(xv[c][i].z), fabsf(xv[c][i].w))));
    m = wave_max(m);
    if (lane == 0) red[c][wave] = m;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float m = red[c][0];
#pragma unroll
    for (int w = 1; w < W; ++w) m = fmaxf(m, red[c][w]);
    mx[c] = m;
  }
  // Codes into LDS (and, from workgroup 0, where the quantizer writes them).
  const bool first = blockIdx.x == 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const float inv = 127.0f / mx[c];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int idx = tid + T * i;
      if (idx < K4) {
        const uint32_t b0 = static_cast<uint32_t>(w8a8_round_act(xv[c][i].x, inv)) & 0xFFu;
        const uint32_t b1 = static_cast<uint32_t>(w8a8_round_act(xv[c][i].y, inv)) & 0xFFu;
        const uint32_t b2 = static_cast<uint32_t>(w8a8_round_act(xv[c][i].z, inv)) & 0xFFu;
        const uint32_t b3 = static_cast<uint32_t>(w8a8_round_act(xv[c][i].w, inv)) & 0xFFu;
        const uint32_t q4 = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
        *reinterpret_cast<uint32_t *>(&lq[c][4 * idx]) = q4;
        if (first) reinterpret_cast<uint32_t *>(aq + static_cast<int64_t>(c) * K)[idx] = q4;
      }
    }
    if (first && tid == 0) ascale[c] = mx[c] / 127.0f;
  }
  __syncthreads();

  // Contraction: four v_dot4 per chunk and activation row.
  int acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = 0;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int ch = j + L * i;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const v4i b = *reinterpret_cast<const v4i *>(&lq[c][16 * ch]);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[c] = __builtin_amdgcn_sdot4(wv[i][e], b[e], acc[c], false);
    }
  }
  const int row = row0 + rl;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int C = lanes_sum<L>(acc[c]);
    if (j == c && row < OC) {
      const float as = mx[c] / 127.0f;
      y[static_cast<int64_t>(c) * OC + row] = (as * wsn) * static_cast<float>(C);
      if (dot) dot[static_cast<int64_t>(c) * OC + row] = C;
    }
  }
}

// ---------------------------------------------------------------------------
// Host side.

constexpr int kVariants = 9;
constexpr int kW8a8Variants = 11;  // the I8_S variants, 10: activation-resident, 11: fused decode (W8A8 only)
constexpr int64_t kW8a8ResMaxLds = 160 * 1024;

// Variant 10 needs K a multiple of 64 and the 64-row activation tile (pitch
// K + 16) within the LDS of a CU.
bool w8a8_res_fits(int64_t K) { return K % 64 == 0 && 64 * (K + 16) <= kW8a8ResMaxLds; }

template <int G, int KST, bool VEC4>
int launch_w8a8_res_inst(int64_t blocks, int64_t lds, const MatArgs &a, int tiles_m, int ms, hipStream_t stream) {
  // Allow the large dynamic LDS once per device for this instantiation
  // (repeating it from racing threads is harmless).
  static std::atomic<uint64_t> attr_done{0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return I2S_EHIP;
  const uint64_t bit = dev < 64 ? (uint64_t{1} << dev) : 0;
  if (!bit || !(attr_done.load(std::memory_order_acquire) & bit)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(&w8a8_res_kernel<G, KST, VEC4>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kW8a8ResMaxLds)) != hipSuccess)
      return I2S_EHIP;
    attr_done.fetch_or(bit, std::memory_order_acq_rel);
  }
  hipLaunchKernelGGL((w8a8_res_kernel<G, KST, VEC4>), dim3(static_cast<unsigned>(blocks)), dim3(512),
                     static_cast<size_t>(lds), stream, static_cast<const int8_t *>(a.w), a.cscale,
                     static_cast<int>(a.OC), static_cast<int>(a.IC), static_cast<const int8_t *>(a.x), a.rscale,
                     static_cast<int>(a.N), a.y, a.dot, tiles_m, ms);
  return hipGetLastError() == hipSuccess ? I2S_OK : I2S_EHIP;
}

// Tiles of 64 activation rows; weight tiles of ms 16-row subtiles, ms chosen
// so that the grid is about one workgroup per compute unit.
int launch_w8a8_res(const MatArgs &a, hipStream_t stream) {
  if (!w8a8_res_fits(a.IC)) return I2S_EKERNEL;
  const int64_t tiles_n = (a.N + 63) / 64;
  const int64_t mt = (a.OC + 15) / 16;
  int64_t per = 256 / tiles_n;
  if (per < 1) per = 1;
  int64_t ms = (mt + per - 1) / per;
  if (ms < 1) ms = 1;
  const int64_t tiles_m = (mt + ms - 1) / ms;
  const int64_t blocks = tiles_m * tiles_n;
  if (blocks > 0x7fffffff || ms > 0x7fffffff) return I2S_ERANGE;
  const int64_t lds = 64 * (a.IC + 16);
  // Groups of 4 subtiles in 2-chunk batches from 4096 output channels
  // (gate 8960 x 1536, M = 512: 18.0 against 20.6 us for groups of 3 in
  // 4-chunk batches; M = 1024: 31.7 against 34.8), groups of 3 below
  // (1536 x 1536: 8.5 against 8.6).
  const int tm = static_cast<int>(tiles_m), msub = static_cast<int>(ms);
  if (a.OC >= 4096) {
    if (a.OC % 4 == 0) return launch_w8a8_res_inst<4, 2, true>(blocks, lds, a, tm, msub, stream);
    return launch_w8a8_res_inst<4, 2, false>(blocks, lds, a, tm, msub, stream);
  }
  if (a.OC % 4 == 0) return launch_w8a8_res_inst<3, 4, true>(blocks, lds, a, tm, msub, stream);
  return launch_w8a8_res_inst<3, 4, false>(blocks, lds, a, tm, msub, stream);
}

// f32 selects the W8A8 epilogue (one pass into a.y); otherwise the two
// passes of mul_mat_add.
template <int TM, int TN, int KS>
int launch_mfma(MatArgs a, bool f32, hipStream_t stream) {
  // A multiple of the channel-block count when possible: each workgroup then
  // keeps one channel block over all of its tiles.
  // The grid stays within what is resident at once (kResidentGroups), so each
  // workgroup's prologue is paid once and its tiles stream through the
  // pipeline.  The larger operand is made XCD-local when the tile counts
  // allow it; otherwise tiles are dealt with a plain grid stride (a multiple
  // of the channel-block count when possible, so that a workgroup keeps one
  // channel block).
  const int64_t tiles_o = (a.OC + TM - 1) / TM, tiles_n = (a.N + TN - 1) / TN;
  const int64_t cap = kResidentGroups;
  const bool x_larger = a.N >= a.OC;  // both operands have IC bytes per row
  int g;
  if (x_larger && tiles_o >= 1 && tiles_n >= kXcds && kXcds * tiles_o <= cap) {
    const int64_t r = std::min((tiles_n + kXcds - 1) / kXcds, cap / (kXcds * tiles_o));
    a.map = kMapXLocal;
    a.rep = static_cast<int>(r);
    g = static_cast<int>(kXcds * tiles_o * r);
  } else if (!x_larger && tiles_n >= 1 && tiles_o >= kXcds && kXcds * tiles_n <= cap) {
    const int64_t r = std::min((tiles_o + kXcds - 1) / kXcds, cap / (kXcds * tiles_n));
    a.map = kMapWLocal;
    a.rep = static_cast<int>(r);
    g = static_cast<int>(kXcds * tiles_n * r);
  } else {
    a.map = kMapStride;
    a.rep = 1;
    g = static_cast<int>(tiles_o * tiles_n < cap ? (tiles_o * tiles_n > 0 ? tiles_o * tiles_n : 1) : cap);
    if (tiles_o >= 1 && tiles_o <= cap) {
      const int64_t per = tiles_n < cap / tiles_o ? tiles_n : cap / tiles_o;
      g = static_cast<int>(tiles_o * (per > 0 ? per : 1));
    }
  }
  a.nparts = g;
  if (f32) {  // W8A8: one pass, F32 out
    hipLaunchKernelGGL((i8s_mm_mfma_kernel<TM, TN, KS, kModeF32>), dim3(g), dim3(kThreads), 0, stream,
                       I8S_KARGS_OF(a, true, g));
    return hip_status();
  }
  hipLaunchKernelGGL((i8s_mm_mfma_kernel<TM, TN, KS, kModeMax>), dim3(g), dim3(kThreads), 0, stream,
                     I8S_KARGS_OF(a, false, g));
  hipLaunchKernelGGL((i8s_mm_mfma_kernel<TM, TN, KS, kModeQuant>), dim3(g), dim3(kThreads), 0, stream,
                     I8S_KARGS_OF(a, false, g));
  return hip_status();
}

template <int FN, int W>
int launch_skinny_fn_w(MatArgs a, bool f32, int64_t items, hipStream_t stream) {
  constexpr int SPW = 2;
  const int g = parts_for(items);
  a.nparts = g;
  if (f32) {
    hipLaunchKernelGGL((i8s_mm_skinny_kernel<W, FN, SPW, kModeF32>), dim3(g), dim3(64 * W), 0, stream,
                       I8S_KARGS_OF(a, true, g));
    return hip_status();
  }
  hipLaunchKernelGGL((i8s_mm_skinny_kernel<W, FN, SPW, kModeMax>), dim3(g), dim3(64 * W), 0, stream,
                     I8S_KARGS_OF(a, false, g));
  hipLaunchKernelGGL((i8s_mm_skinny_kernel<W, FN, SPW, kModeQuant>), dim3(g), dim3(64 * W), 0, stream,
                     I8S_KARGS_OF(a, false, g));
  return hip_status();
}

// Waves per workgroup, measured on MI355X: with at least one item per
// compute unit, 4 waves (gate 8960 x 1536 at one row: 6.2 against 6.9 us);
// with fewer items, 8 waves split each item's K-steps further (down
// 1536 x 8960: 9.1 against 11.8 us with 4).
template <int FN>
int launch_skinny_fn(MatArgs a, bool f32, hipStream_t stream) {
  const int64_t items = ((a.OC + 15) / 16) * ((a.N + 16 * FN - 1) / (16 * FN));
  return items >= kSkinnyFewWavesItems ? launch_skinny_fn_w<FN, 4>(a, f32, items, stream)
                                       : launch_skinny_fn_w<FN, 8>(a, f32, items, stream);
}

// Row blocks of 16, 32 or 64 rows, by N.
int launch_skinny(MatArgs a, bool f32, hipStream_t stream) {
  if (a.N <= 16) return launch_skinny_fn<1>(a, f32, stream);
  if (a.N <= 32) return launch_skinny_fn<2>(a, f32, stream);
  return launch_skinny_fn<4>(a, f32, stream);
}

int launch_plain(MatArgs a, hipStream_t stream) {
  const int g = parts_for((a.N * a.OC + kThreads - 1) / kThreads);
  a.nparts = g;
  hipLaunchKernelGGL(i8s_mm_plain_kernel<false>, dim3(g), dim3(kThreads), 0, stream, I8S_KARGS_OF(a, false, g));
  hipLaunchKernelGGL(i8s_mm_plain_kernel<true>, dim3(g), dim3(kThreads), 0, stream, I8S_KARGS_OF(a, false, g));
  return hip_status();
}

// Tile (channels x rows, 64-byte steps per K chunk): 2 = 128 x 128 x 1, 3 = 64 x 128 x 1,
// 4 = 128 x 64 x 1, 5 = 128 x 64 x 2, 6 = 64 x 128 x 2, 7 = 128 x 64 x 4, 8 = 64 x 64 x 1;
// 9 = the skinny kernel (16 channels x up to 64 rows per workgroup, waves split K).
// The skinny kernel when the tile kernel would have too few tiles: up to 64
// rows, up to 256 rows with fewer than 128 tiles of 128 x 64, or up to 512
// rows with fewer than 64 (measured on the encoder, connector and decoder
// shapes).
bool skinny_wins(int64_t OC, int64_t N) {
  const int64_t tiles = ((OC + 127) / 128) * ((N + 63) / 64);
  return N <= 64 || (N <= 256 && tiles < 128) || (N <= 512 && tiles < 64);
}

int auto_variant(int64_t OC, int64_t IC, int64_t N) {
  if (IC % 16 != 0) return 1;
  if (skinny_wins(OC, N)) return 9;
  if (OC <= 64) return 6;   // 64 x 128 x 2: few channels, many rows
  if (IC <= 64) return 2;   // 128 x 128 x 1
  if (IC <= 128) return 5;  // 128 x 64 x 2
  return 7;                 // 128 x 64 x 4
}

int check_mm(const uint8_t *w, int64_t OC, int64_t IC, const uint8_t *x, int64_t N, const float *bias,
             const uint8_t *out, const int32_t *dot_out, void *workspace, size_t workspace_bytes) {
  if (!w || !x || !out || OC < 0 || IC < 0 || N < 0) return I2S_EINVAL;
  if (!aligned(w, 16) || !aligned(x, 16) || !aligned(out, 16)) return I2S_EINVAL;
  if ((bias && !aligned(bias, 4)) || (dot_out && !aligned(dot_out, 4))) return I2S_EINVAL;
  if (IC > I8S_MAX_IC) return I2S_ERANGE;
  if (OC * IC >= kMaxBytes || N * IC >= kMaxBytes || N * OC >= kMaxBytes / 4) return I2S_ERANGE;
  if (OC > kMaxBytes || N > kMaxBytes) return I2S_ERANGE;  // sizes go to the kernels as 32-bit values
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < kMaxParts * sizeof(float)) return I2S_EWORKSPACE;
  return I2S_OK;
}

}  // namespace

extern "C" size_t i8s_bytes(int64_t n) { return n < 0 ? 0 : static_cast<size_t>(n) + I8S_SCALE_SLOT; }

extern "C" size_t i8s_workspace_bytes(void) { return kMaxParts * sizeof(float); }

extern "C" int i8s_variants(void) { return kVariants; }

extern "C" int i8s_mul_mat_add_variant(int64_t OC, int64_t IC, int64_t N) { return auto_variant(OC, IC, N); }

extern "C" int i8s_quantize(const float *x, int64_t n, uint8_t *out, void *workspace, size_t workspace_bytes,
                            void *stream) {
  if ((!x && n != 0) || !out || n < 0 || !aligned(x, 16) || !aligned(out, 16)) return I2S_EINVAL;
  if (n >= kMaxBytes) return I2S_ERANGE;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < kMaxParts * sizeof(float)) return I2S_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int g = parts_for((n / 16 + kThreads - 1) / kThreads);
  float *parts = static_cast<float *>(workspace);
  hipLaunchKernelGGL(i8s_absmax_kernel, dim3(g), dim3(kThreads), 0, s, x, n, parts);
  hipLaunchKernelGGL(i8s_quantize_kernel, dim3(g), dim3(kThreads), 0, s, x, n, parts, g, out);
  return hip_status();
}

extern "C" int i8s_dequantize(const uint8_t *t, int64_t n, float *y, void *stream) {
  if (!t || (!y && n != 0) || n < 0 || !aligned(t, 16) || !aligned(y, 16)) return I2S_EINVAL;
  if (n >= kMaxBytes / 4) return I2S_ERANGE;
  const int g = parts_for((n / 16 + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(i8s_dequantize_kernel, dim3(g), dim3(kThreads), 0, static_cast<hipStream_t>(stream), t, n, y);
  return hip_status();
}

extern "C" int i8s_mul_mat_add_ex(const uint8_t *w, int64_t OC, int64_t IC, const uint8_t *x, int64_t N,
                                  const float *bias, int relu, uint8_t *out, int32_t *dot_out, int variant,
                                  void *workspace, size_t workspace_bytes, void *stream) {
  const int st = check_mm(w, OC, IC, x, N, bias, out, dot_out, workspace, workspace_bytes);
  if (st != I2S_OK) return st;
  if (variant < 0 || variant > kVariants) return I2S_EKERNEL;
  if (variant == 0) variant = auto_variant(OC, IC, N);
  if (variant >= 2 && IC % 16 != 0) return I2S_EKERNEL;
  MatArgs a = {};  // every field not set below (the W8A8 ones) stays null
  a.w = reinterpret_cast<const int8_t *>(w);
  a.x = reinterpret_cast<const int8_t *>(x);
  a.ws = w + OC * IC;
  a.xs = x + N * IC;
  a.bias = bias;
  a.parts = static_cast<float *>(workspace);
  a.out = reinterpret_cast<int8_t *>(out);
  a.dot = dot_out;
  a.OC = OC;
  a.IC = IC;
  a.N = N;
  a.nparts = 0;
  a.relu = relu ? 1 : 0;
  a.vec = (OC % 16 == 0) && (!dot_out || aligned(dot_out, 16));
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (variant) {
    case 1: return launch_plain(a, s);
    case 9: return launch_skinny(a, false, s);
    case 8: return launch_mfma<64, 64, 1>(a, false, s);
    case 2: return launch_mfma<128, 128, 1>(a, false, s);
    case 3: return launch_mfma<64, 128, 1>(a, false, s);
    case 4: return launch_mfma<128, 64, 1>(a, false, s);
    case 5: return launch_mfma<128, 64, 2>(a, false, s);
    case 6: return launch_mfma<64, 128, 2>(a, false, s);
    default: return launch_mfma<128, 64, 4>(a, false, s);
  }
}

extern "C" int i8s_mul_mat_add(const uint8_t *w, int64_t OC, int64_t IC, const uint8_t *x, int64_t N,
                               const float *bias, uint8_t *out, void *workspace, size_t workspace_bytes, void *stream) {
  return i8s_mul_mat_add_ex(w, OC, IC, x, N, bias, 0, out, nullptr, 0, workspace, workspace_bytes, stream);
}

extern "C" int i8s_mul_mat_add_relu(const uint8_t *w, int64_t OC, int64_t IC, const uint8_t *x, int64_t N,
                                    const float *bias, uint8_t *out, void *workspace, size_t workspace_bytes,
                                    void *stream) {
  return i8s_mul_mat_add_ex(w, OC, IC, x, N, bias, 1, out, nullptr, 0, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
// Per-channel W8A8 (include/w8a8.h).

namespace {

// The skinny kernel for few rows (as for I8_S); otherwise 128 x 64 tiles with
// 4-step K chunks, measured fastest on the Qwen2-1.5B projection shapes.
// Measured on MI355X (the Qwen2 gate, q and k shapes, M 1..1024): the skinny
// kernel while it wins, the activation-resident kernel from 128 rows where K
// fits it (gate 8960 x 1536, M = 512: 22 against 31 us with weights from
// HBM), the tile kernels otherwise.
// W8A8 variant 11: lanes per weight row by K (16 for K <= 2048, 32 to 4096,
// 64 to 9216), activation rows NC = M <= 4.  Measured on MI355X (weights
// from HBM): gate 8960 x 1536 at M = 1 takes 4.14 us with 16 lanes and 256
// threads (4.25-4.50 with 8 or 32 lanes, or 512 threads); the down
// projection 1536 x 8960 4.37 us at M = 1 and 7.9 at M = 4 with 64 lanes and
// 512 threads, against 5.2 and 10.7 with 256 threads and 4.8 and 9.7 with
// 32 lanes.
constexpr int64_t kW8a8FusedMaxM = 4;
constexpr int kW8a8FusedMaxK = 9216;
bool w8a8_fused_fits(int64_t K, int64_t M) { return M >= 1 && M <= kW8a8FusedMaxM && K <= kW8a8FusedMaxK; }

template <int KMAX, int NC, int L, int CPL, int XPT, int T>
int launch_w8a8_fused_cfg(const int8_t *wq, const float *wscale, int64_t OC, int64_t K, const float *x, float *y,
                          int32_t *dot, int8_t *aq, float *as, hipStream_t stream) {
  static_assert(4 * T * XPT >= KMAX && 16 * L * CPL >= KMAX, "the threads hold a row of KMAX values, the lanes its chunks");
  constexpr int R = T / L;
  const int64_t blocks = (OC + R - 1) / R;
  hipLaunchKernelGGL((w8a8_gemv_fused_kernel<NC, L, CPL, XPT, T>), dim3(static_cast<uint32_t>(blocks)), dim3(T), 0,
                     stream, wq, x, static_cast<int>(OC), static_cast<int>(K), wscale, y, dot, aq, as);
  return hip_status();
}

template <int NC>
int launch_w8a8_fused_nc(const int8_t *wq, const float *wscale, int64_t OC, int64_t K, const float *x, float *y,
                         int32_t *dot, int8_t *aq, float *as, hipStream_t stream) {
  if (K <= 1536) {
    // Beyond 256 workgroups of 16 rows some compute units hold two, and the
    // second one's activation loads queue behind the first one's weights.
    // Workgroups of 48 rows (six waves, 8 lanes per row) keep up to 12288
    // rows at one per compute unit: 8960 x 1536 at M = 1 takes 3.85 us
    // instead of 4.16.  Fewer rows keep 16-row workgroups, which fill more
    // of the chip (1536 x 1536: 2.19 us against 2.97).
    if (OC > 8192 && OC <= 12288)
      return launch_w8a8_fused_cfg<1536, NC, 8, 12, 1, 384>(wq, wscale, OC, K, x, y, dot, aq, as, stream);
    return launch_w8a8_fused_cfg<1536, NC, 16, 6, 2, 256>(wq, wscale, OC, K, x, y, dot, aq, as, stream);
  }
  if (K <= 2048) return launch_w8a8_fused_cfg<2048, NC, 16, 8, 2, 256>(wq, wscale, OC, K, x, y, dot, aq, as, stream);
  if (K <= 4096) return launch_w8a8_fused_cfg<4096, NC, 32, 8, 4, 256>(wq, wscale, OC, K, x, y, dot, aq, as, stream);
  return launch_w8a8_fused_cfg<kW8a8FusedMaxK, NC, 64, 9, 5, 512>(wq, wscale, OC, K, x, y, dot, aq, as, stream);
}

int launch_w8a8_fused(const int8_t *wq, const float *wscale, int64_t OC, int64_t K, const float *x, int64_t M,
                      float *y, int32_t *dot, int8_t *aq, float *as, hipStream_t stream) {
  switch (M) {
    case 1: return launch_w8a8_fused_nc<1>(wq, wscale, OC, K, x, y, dot, aq, as, stream);
    case 2: return launch_w8a8_fused_nc<2>(wq, wscale, OC, K, x, y, dot, aq, as, stream);
    case 3: return launch_w8a8_fused_nc<3>(wq, wscale, OC, K, x, y, dot, aq, as, stream);
    default: return launch_w8a8_fused_nc<4>(wq, wscale, OC, K, x, y, dot, aq, as, stream);
  }
}

int w8a8_auto_variant(int64_t OC, int64_t K, int64_t M) {
  if (skinny_wins(OC, M)) return 9;
  if (OC <= 64) return 6;
  if (M >= 128 && w8a8_res_fits(K)) return 10;
  return 7;
}

int check_rows(const void *x, int64_t rows, int64_t K, const void *q, const float *scale) {
  if (!x || !q || !scale || rows < 0 || K < 0) return I2S_EINVAL;
  if (rows * K >= kMaxBytes) return I2S_ERANGE;
  return I2S_OK;
}

}  // namespace

extern "C" size_t w8a8_act_workspace_bytes(int64_t M, int64_t K) {
  if (M < 0 || K < 0) return 0;
  const size_t q = (static_cast<size_t>(M) * static_cast<size_t>(K) + 255) / 256 * 256;
  return q + (static_cast<size_t>(M) * 4 + 255) / 256 * 256;
}

extern "C" int w8a8_quantize_weight(const float *w, int64_t OC, int64_t K, int8_t *wq, float *wscale, void *stream) {
  const int st = check_rows(w, OC, K, wq, wscale);
  if (st != I2S_OK) return st;
  if (OC == 0) return I2S_OK;
  hipLaunchKernelGGL(w8a8_quant_rows_kernel<true>, dim3(static_cast<uint32_t>(OC)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), w, K, wq, wscale);
  return hip_status();
}

extern "C" int w8a8_quantize_act(const float *x, int64_t M, int64_t K, int8_t *q, float *ascale, void *stream) {
  const int st = check_rows(x, M, K, q, ascale);
  if (st != I2S_OK) return st;
  if (M == 0) return I2S_OK;
  if (!launch_act_reg_fit(x, M, K, q, ascale, static_cast<hipStream_t>(stream)))
    hipLaunchKernelGGL(w8a8_quant_rows_kernel<false>, dim3(static_cast<uint32_t>(M)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), x, K, q, ascale);
  return hip_status();
}

// The automatic choice of the F32-input entry points: the fused decode
// kernel for M <= 4 (K % 16 == 0 as the contraction needs), else the
// contraction's own choice after a separate quantizer launch.
int w8a8_mul_mat_auto(int64_t OC, int64_t K, int64_t M) {
  return (w8a8_fused_fits(K, M) && K % 16 == 0) ? 11 : w8a8_auto_variant(OC, K, M);
}

extern "C" int w8a8_mul_mat_variant(int64_t OC, int64_t K, int64_t M) { return w8a8_mul_mat_auto(OC, K, M); }

extern "C" int w8a8_variants(void) { return kW8a8Variants; }

extern "C" int w8a8_matmul(const int8_t *wq, const float *wscale, int64_t OC, int64_t K, const int8_t *aq,
                           const float *ascale, int64_t M, float *y, int32_t *dot_out, int variant, void *stream) {
  if (!wq || !wscale || !aq || !ascale || !y || OC < 0 || K < 0 || M < 0) return I2S_EINVAL;
  if (!aligned(wq, 16) || !aligned(aq, 16) || !aligned(y, 16) || !aligned(wscale, 4) || !aligned(ascale, 4))
    return I2S_EINVAL;
  if (dot_out && !aligned(dot_out, 16)) return I2S_EINVAL;
  if (K == 0 || K % 16 != 0) return I2S_EALIGN;
  if (OC * K >= kMaxBytes || M * K >= kMaxBytes || M * OC >= kMaxBytes / 4) return I2S_ERANGE;
  if (OC > kMaxBytes || M > kMaxBytes) return I2S_ERANGE;  // sizes go to the kernels as 32-bit values
  // variant 11 quantizes F32 rows itself: only the F32-input entry points take it
  if (variant < 0 || variant == 1 || variant == 11 || variant > kW8a8Variants) return I2S_EKERNEL;
  if (variant == 10 && !w8a8_res_fits(K)) return I2S_EKERNEL;
  if (variant == 0) variant = w8a8_auto_variant(OC, K, M);
  if (OC == 0 || M == 0) return I2S_OK;
  MatArgs a = {};
  a.w = wq;
  a.x = aq;
  a.dot = dot_out;
  a.OC = OC;
  a.IC = K;
  a.N = M;
  a.vec = OC % 4 == 0;
  a.cscale = wscale;
  a.rscale = ascale;
  a.y = y;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (variant) {
    case 2: return launch_mfma<128, 128, 1>(a, true, s);
    case 3: return launch_mfma<64, 128, 1>(a, true, s);
    case 4: return launch_mfma<128, 64, 1>(a, true, s);
    case 5: return launch_mfma<128, 64, 2>(a, true, s);
    case 6: return launch_mfma<64, 128, 2>(a, true, s);
    case 7: return launch_mfma<128, 64, 4>(a, true, s);
    case 9: return launch_skinny(a, true, s);
    case 10: return launch_w8a8_res(a, s);
    default: return launch_mfma<64, 64, 1>(a, true, s);
  }
}

extern "C" int w8a8_mul_mat_ex(const int8_t *wq, const float *wscale, int64_t OC, int64_t K, const float *x, int64_t M,
                               void *workspace, size_t workspace_bytes, float *y, int32_t *dot_out, int variant,
                               void *stream) {
  if (!x || !aligned(x, 16)) return I2S_EINVAL;
  if (M < 0 || K < 0) return I2S_EINVAL;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < w8a8_act_workspace_bytes(M, K))
    return I2S_EWORKSPACE;
  int8_t *aq = static_cast<int8_t *>(workspace);
  float *as = reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                        (static_cast<size_t>(M) * static_cast<size_t>(K) + 255) / 256 * 256);
  // Validate the contraction's arguments before launching anything.
  if (!wq || !wscale || !y || OC < 0) return I2S_EINVAL;
  if (!aligned(wq, 16) || !aligned(y, 16) || !aligned(wscale, 4) || (dot_out && !aligned(dot_out, 16)))
    return I2S_EINVAL;
  if (K == 0 || K % 16 != 0) return I2S_EALIGN;
  if (OC * K >= kMaxBytes || M * K >= kMaxBytes || M * OC >= kMaxBytes / 4) return I2S_ERANGE;
  if (OC > kMaxBytes || M > kMaxBytes) return I2S_ERANGE;  // sizes go to the kernels as 32-bit values
  if (variant < 0 || variant == 1 || variant > kW8a8Variants) return I2S_EKERNEL;
  if (variant == 10 && !w8a8_res_fits(K)) return I2S_EKERNEL;
  if (variant == 11 && !w8a8_fused_fits(K, M)) return I2S_EKERNEL;
  if (variant == 0) variant = w8a8_mul_mat_auto(OC, K, M);
  if (variant == 11) {
    if (OC == 0) return w8a8_quantize_act(x, M, K, aq, as, stream);  // nothing to contract; the codes as ever
    return launch_w8a8_fused(wq, wscale, OC, K, x, M, y, dot_out, aq, as, static_cast<hipStream_t>(stream));
  }
  int st = w8a8_quantize_act(x, M, K, aq, as, stream);
  if (st != I2S_OK) return st;
  return w8a8_matmul(wq, wscale, OC, K, aq, as, M, y, dot_out, variant, stream);
}

extern "C" int w8a8_mul_mat(const int8_t *wq, const float *wscale, int64_t OC, int64_t K, const float *x, int64_t M,
                            void *workspace, size_t workspace_bytes, float *y, void *stream) {
  return w8a8_mul_mat_ex(wq, wscale, OC, K, x, M, workspace, workspace_bytes, y, nullptr, 0, stream);
}
