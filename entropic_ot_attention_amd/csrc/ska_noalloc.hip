// Forward entry point that allocates nothing: sinkhorn_attn_fwd on a workspace held in a
// file-scope device array of this library instead of one the caller passes.
//
// For callers that cannot allocate device memory around the call (HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).  Each GPU the library runs on holds its own
// copy of the array from module load until the process ends.  The array's address on the
// current device is looked up once per device with hipGetSymbolAddress (in host code the
// array's name is only a host-side stand-in) and kept; kernels receive that address as their
// workspace pointer.  Every call on one GPU shares that GPU's array, so calls that overlap on
// one GPU (different streams, or different host threads without ordering) race.  The forward
// reads no workspace location that the same call has not written first (its fill kernels run
// on the caller's stream where a path needs zeroed duals), so the array is never cleared here.

#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "sinkhorn_attn.h"
#include "ska_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;   // SKA_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == SKA_NOALLOC_SCRATCH_BYTES, "header and library disagree");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch` (looked up on the first call per device).
ska_status scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return ska::set_error(SKA_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return ska::set_error(SKA_ERR_UNSUPPORTED, "device index beyond the scratch table (64 devices)");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return ska::set_error(SKA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") +
                                             hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SKA_OK;
}

}  // namespace

extern "C" ska_status sinkhorn_attn_fwd_noalloc(const ska_problem* p, const void* Q, const void* K,
                                                const void* V, void* O, float* duals,
                                                hipStream_t stream) {
  ska::set_error(SKA_OK, "");
  size_t need = 0;
  const ska_status s = ska_workspace_bytes(p, SKA_OP_FWD, &need);
  if (s != SKA_OK) return s;
  if (need > kScratchBytes)
    return ska::set_error(SKA_ERR_UNSUPPORTED,
                          "sinkhorn_attn_fwd_noalloc: the problem needs " + std::to_string(need) +
                              " workspace bytes, above the library's static scratch of " +
                              std::to_string(kScratchBytes) +
                              " bytes; call sinkhorn_attn_fwd with a caller workspace");
  if (p->bh == 0 || p->L == 0) return SKA_OK;
  void* ws = nullptr;
  const ska_status t = scratch_on_current_device(&ws);
  if (t != SKA_OK) return t;
  return sinkhorn_attn_fwd(p, Q, K, V, O, duals, ws, kScratchBytes, stream);
}
