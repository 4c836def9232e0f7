// noalloc.hip -- qlora_linear_fwd for callers that cannot allocate device
// memory: the same launches, with the workspace taken from a fixed device
// array of this library instead of an argument.
//
// The array lives in the library's code object, one copy per GPU the
// library runs on, held until the process ends.  Its device address on the
// current GPU is looked up once per GPU (hipGetSymbolAddress) and kept; host
// code never passes the array's own name to a launch or a copy, since on the
// host that name is only a stand-in for the device symbol.
//
// The forward writes every workspace word before it reads it, so nothing in
// the array has to start at zero, and stale contents from an earlier call
// are harmless.  Calls that overlap on one GPU (different streams, or host
// threads without ordering) share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "qlora.h"
#include "qlora_kernels.h"

namespace {

constexpr size_t kScratchBytes = QLORA_STATIC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current GPU.
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QLORA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QLORA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QLORA_OK;
}

}  // namespace

extern "C" int qlora_linear_fwd_noalloc(const qlora_nf4_t* q, const uint16_t* X, int64_t M,
                                        const uint16_t* A, const uint16_t* B, int64_t r,
                                        float lora_alpha, uint16_t* Y, float* T_save,
                                        void* stream) {
  int s = qlora::linear_fwd_check(q, X, M, A, B, r, Y, T_save, kScratchBytes);
  if (s == QLORA_ERR_WORKSPACE) return QLORA_ERR_SCRATCH;
  if (s) return s;
  if (M == 0) return QLORA_OK;
  void* ws = nullptr;
  s = scratch_on_current_device(&ws);
  if (s) return s;
  return qlora_linear_fwd(q, X, M, A, B, r, lora_alpha, Y, T_save, ws, kScratchBytes, stream);
}
