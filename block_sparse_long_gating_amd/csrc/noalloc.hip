// Allocation-free decode step: moba_decode_fwd with its workspace in a fixed,
// file-scope device array instead of the library's stream-ordered pool, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight generation loops, harnesses that forbid allocation).
//
// Every GPU the library runs on holds its own copy of `scratch` (kNoAllocBytes)
// until the process ends. Host code never uses the array's name as an address:
// at a device's first call, with that device current, its device address is
// looked up once with hipGetSymbolAddress and kept per device. Calls on one GPU
// share that memory, so calls that overlap on one GPU (on different streams,
// or from different threads without ordering) race; calls ordered on one
// stream do not. The decode kernels write every workspace byte they read in
// the same call, so nothing needs clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/moba.h"
#include "kernels.h"

namespace {

constexpr size_t kNoAllocBytes = static_cast<size_t>(MOBA_NOALLOC_SCRATCH_BYTES);
static_assert(kNoAllocBytes % 256 == 0, "the scratch array is handed out in 256-byte aligned pieces");

static __device__ __align__(256) char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;

struct ScratchState {
  std::once_flag once;
  hipError_t error = hipSuccess;
  char* ptr = nullptr;   // device address of this device's copy of `scratch`
};

ScratchState g_scratch[kMaxDevices];

void lookup(ScratchState* st) {
  void* p = nullptr;
  st->error = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (st->error == hipSuccess && p == nullptr) st->error = hipErrorInvalidSymbol;
  st->ptr = static_cast<char*>(p);
}

}  // namespace

extern "C" int moba_decode_fwd_noalloc(const void* q, const void* k, const void* v, const float* kbar,
                                       int32_t kbar_blocks, void* out, float* lse, int32_t* sel, int64_t N, int32_t H,
                                       int32_t D, int32_t block_size, int32_t topk, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return moba::fail_hip(e);
  if (dev < 0 || dev >= kMaxDevices) return MOBA_ERR_UNSUPPORTED;
  ScratchState* st = &g_scratch[dev];
  std::call_once(st->once, lookup, st);
  if (st->error != hipSuccess) return moba::fail_hip(st->error);
  return moba::decode_with_workspace(q, k, v, kbar, kbar_blocks, out, lse, sel, N, H, D, block_size, topk, stream,
                                     st->ptr, kNoAllocBytes);
}
