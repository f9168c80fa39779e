// chimera_kda_fwd_noalloc: chimera_kda_fwd with its workspace in a device array that the
// library owns, for callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The array is a file-scope __device__ object: each GPU the library runs on holds its own copy,
// allocated when the code object loads there and kept until the process ends. In host code its
// name is only a host-side stand-in; the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and only that address is handed to kernels.
// Every call on one GPU shares that GPU's array: calls that overlap on one device race. Nothing
// in it needs to start at zero (every workspace entry is written before it is read).
#include <hip/hip_runtime.h>

#include <atomic>

#include "chimera_mshortconv.h"

namespace {

constexpr size_t kScratchBytes = CHIMERA_KDA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_ptr[kMaxDevices];   // device address per device, once looked up

// The scratch array's device address on the current device. Concurrent first calls store the
// same address.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  void* p = dev >= 0 && dev < kMaxDevices ? scratch_ptr[dev].load(std::memory_order_acquire) : nullptr;
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    if (dev >= 0 && dev < kMaxDevices) scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" chimera_status chimera_kda_fwd_noalloc(const void* q, const void* k, const void* v, int64_t qkv_stride,
                                                  const void* alpha, const void* beta, const float* S0, void* o,
                                                  float* S_final, int64_t B, int64_t T, int64_t H, int64_t dk,
                                                  int64_t dv, chimera_dtype dt, uint32_t flags,
                                                  hipStream_t stream) {
  // Sizes first, on the host: a request whose workspace exceeds the array is refused before any
  // HIP call. Invalid sizes need no workspace and are reported by chimera_kda_fwd.
  const size_t need = chimera_kda_workspace_size(B, T, H, dk, dv, dt, flags);
  if (need > kScratchBytes) return CHIMERA_ERR_WORKSPACE;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (need > 0) {
    if (scratch_address(&ws) != hipSuccess) return CHIMERA_ERR_HIP;
    ws_bytes = kScratchBytes;
  }
  return chimera_kda_fwd(q, k, v, qkv_stride, alpha, beta, S0, o, S_final, B, T, H, dk, dv, dt, flags, ws, ws_bytes,
                         stream);
}
