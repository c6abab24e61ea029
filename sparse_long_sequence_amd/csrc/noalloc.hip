// noalloc.hip — la_attn_forward_noalloc: band + global attention for callers
// that cannot allocate device memory (code under graph capture, serving loops,
// harnesses that forbid hipMalloc).
//
// The call is la_attn_forward with one difference: its workspace (the global
// rows' key-chunk partials and their arrival counter words) is a fixed array
// in the library's own device memory, `scratch`, instead of a caller buffer.
// Every GPU the library runs on holds one copy of it, of kScratchBytes, from
// the first call on that GPU until the process ends. Nothing in it needs
// clearing between calls: the partials are written before they are read, and
// the counter words carry a token unique to each call (see la_attn_forward).
// All calls on one GPU share the array, so calls that overlap in time on one
// GPU (other streams, other host threads) race and must be serialised by the
// caller.
#include <mutex>
#include <string>

#include "entry.h"
#include "kernels.h"
#include "longattn.h"

namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;  // 32 MiB per GPU
constexpr int kMaxDevices = 64;

// The array's name is a host-side stand-in in host code: its device address
// comes from hipGetSymbolAddress, once per device, and only that address is
// ever handed to a kernel.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

void* g_scratch[kMaxDevices];
hipError_t g_status[kMaxDevices];
std::once_flag g_once[kMaxDevices];

// The current device's copy of `scratch` (its address looked up on the first
// call on that device, with the device current), or null with the reason set
// as the thread's error message.
void* device_scratch() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    la::set_error(LA_EHIP, (std::string("hipGetDevice failed: ") + hipGetErrorString(e)).c_str());
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    la::set_error(LA_EUNSUPPORTED, "device index above 63");
    return nullptr;
  }
  std::call_once(g_once[dev], [dev]() {
    void* p = nullptr;
    g_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch[dev] = g_status[dev] == hipSuccess ? p : nullptr;
  });
  if (g_status[dev] != hipSuccess) {
    la::set_error(LA_EHIP, (std::string("hipGetSymbolAddress failed: ") +
                            hipGetErrorString(g_status[dev])).c_str());
    return nullptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

la_status la_attn_forward_noalloc(const la_dims* dims, const void* q, const void* k,
                                  const void* v, const int32_t* global_idx, int32_t n_global,
                                  int32_t radius, const int32_t* dilation, int32_t causal,
                                  const float* rel_bias, void* out, float* lse,
                                  hipStream_t stream, const la_attn_ext* ext) {
  if (ext && (ext->workspace || ext->workspace_bytes))
    return la::set_error(LA_EINVAL, "la_attn_forward_noalloc takes no workspace (ext->workspace "
                                    "must be NULL and ext->workspace_bytes 0)");
  la::WorkspaceSource src;
  src.fixed_bytes = kScratchBytes;
  src.get = device_scratch;
  return la::attn_forward_ws(dims, q, k, v, global_idx, n_global, radius, dilation, causal,
                             rel_bias, out, lse, stream, ext, src);
}

}  // extern "C"
