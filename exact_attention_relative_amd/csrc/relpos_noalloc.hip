// relpos_attn_fwd_noalloc: the forward call for callers that cannot allocate device memory
// (code under graph capture, tight serving loops, harnesses that forbid allocation).  The
// forward's workspace (index maps, bias LUTs, per-row products) lives in a file-scope device
// array instead of a caller buffer; the call allocates nothing and otherwise runs exactly the
// kernels of relpos_attn_fwd.
#include <mutex>

#include "../../include/relpos_attn.h"

#include <hip/hip_runtime.h>

namespace {

// One copy per GPU, held until the process ends.  Host code never uses this name as an address
// (on the host it is only a stand-in): the device address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[RELPOS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};   // device address of `scratch` per device, once known

// The device address of the current device's copy of `scratch` (looked up once per device, with
// that device current), or nullptr on failure.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int relpos_attn_fwd_noalloc(const relpos_desc* desc, const void* q, const void* k,
                                       const void* v, const void* rel_a, const void* rel_b,
                                       const float* bias_a, const float* bias_b, void* o,
                                       float* lse, hipStream_t stream) {
  // size check first, on the host only: nothing is launched for a refused call
  size_t need = 0;
  int st = relpos_attn_workspace_size(desc, 0, &need);
  if (st != RELPOS_OK) return st;
  if (need > (size_t)RELPOS_NOALLOC_SCRATCH_BYTES) return RELPOS_E_WORKSPACE;
  void* ptr = scratch_ptr();
  if (!ptr) return RELPOS_E_LAUNCH;
  return relpos_attn_fwd(desc, q, k, v, rel_a, rel_b, bias_a, bias_b, o, lse, ptr,
                         (size_t)RELPOS_NOALLOC_SCRATCH_BYTES, stream);
}
