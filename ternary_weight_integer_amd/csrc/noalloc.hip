// i2s_mul_mat_noalloc: the I2_S matmul for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  It is i2s_mul_mat with its activation workspace
// taken from a fixed array in the library's own device memory instead of an
// argument; the kernels, and so every result bit, are i2s_mul_mat's.
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy (I2S_NOALLOC_SCRATCH_BYTES) until the process ends.
// Its host-side name is only a handle for the runtime, not a device address,
// so the device address is looked up once per device with
// hipGetSymbolAddress and that pointer is what the kernels receive.
// Nothing here allocates or frees memory.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <atomic>

#include "i2s.h"

namespace {

constexpr size_t kScratchBytes = I2S_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "the workspace is carved in 256-byte sections");

__device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of `scratch` on each device, looked up on the first call
// made with that device current.  Racing first calls look up the same value.
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];

int scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return I2S_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return I2S_ERANGE;
  void *p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return I2S_EHIP;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return I2S_OK;
}

}  // namespace

extern "C" size_t i2s_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" int i2s_mul_mat_noalloc(const uint8_t *packed, int64_t rows, int64_t K, const float *x, int64_t N,
                                   float *y, int32_t *dot_out, void *stream) {
  // Sizes first, on the host: a bad shape, or one whose workspace exceeds the
  // array, is refused before the device is touched.  The remaining checks
  // (pointers, alignment, ranges) are i2s_mul_mat's.
  if (N < 0 || rows < 0) return I2S_EINVAL;
  if (i2s_packed_bytes(0, K) == 0) return I2S_EALIGN;
  if (N == 0 || rows == 0) return I2S_OK;
  if (i2s_act_workspace_bytes(N, K) > kScratchBytes) return I2S_ESCRATCH;
  void *ws = nullptr;
  const int st = scratch_address(&ws);
  if (st != I2S_OK) return st;
  return i2s_mul_mat(packed, rows, K, x, N, ws, kScratchBytes, y, dot_out, stream);
}
