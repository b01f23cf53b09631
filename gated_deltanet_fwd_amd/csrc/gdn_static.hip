// The forward entry point that allocates nothing (gdn_fwd_noalloc in include/gdn.h), for callers
// that cannot allocate device memory: code under graph capture, tight serving loops, harnesses
// that forbid hipMalloc. Its workspace is a file-scope device array of fixed size instead of a
// caller's buffer; everything else is gdn_fwd on the caller's stream alone.
//
// Every GPU the library runs on holds its own copy of the array until the process ends. Its
// device address is looked up once per device (hipGetSymbolAddress with that device current) on
// the entry point's first call there; the host-side name of the array is not a device address
// and is never passed to a kernel or a copy. Calls on one GPU share the array and keep the last
// call's contents; the forward writes every workspace word it reads before reading it (chunk
// tables, norms, q.k tiles, status), so nothing needs clearing between calls. Calls that overlap
// on one GPU (two streams, two threads) race on the array.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn.h"
#include "gdn_internal.h"

namespace gdn {
int gdn_fwd_single_stream(const gdn_problem* p, const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const int32_t* cu_seqlens, const float* h0, void* o, float* ht,
                          void* saved, void* workspace, size_t workspace_bytes, void* stream);
int gdn_set_error(int code, const char* msg);
} // namespace gdn

static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices]; // device address of `scratch` on each device, once looked up

// The device address of this device's scratch array (looked up on the first call on the device,
// with it current), or NULL with the error set.
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    gdn::gdn_set_error(GDN_EHIP, "gdn_fwd_noalloc: no current device (or device index beyond 63)");
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      gdn::gdn_set_error(GDN_EHIP, "gdn_fwd_noalloc: hipGetSymbolAddress of the scratch array failed");
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

} // namespace

extern "C" int gdn_fwd_noalloc(const gdn_problem* p, const void* q, const void* k, const void* v, const float* g,
                               const float* beta, const int32_t* cu_seqlens, const float* h0, void* o, float* ht,
                               void* saved, void* stream) {
  const size_t need = gdn_workspace_bytes(p, GDN_OP_FWD);
  if (need == 0) return p ? GDN_EINVAL : gdn::gdn_set_error(GDN_EINVAL, "problem descriptor is NULL");
  if (need > (size_t)GDN_NOALLOC_SCRATCH_BYTES)
    return gdn::gdn_set_error(GDN_EWORKSPACE,
                              "gdn_fwd_noalloc: the problem needs more forward workspace than the fixed scratch "
                              "array holds (GDN_NOALLOC_SCRATCH_BYTES); call gdn_fwd with a workspace instead");
  void* ws = scratch_for_current_device();
  if (!ws) return GDN_EHIP;
  return gdn::gdn_fwd_single_stream(p, q, k, v, g, beta, cu_seqlens, h0, o, ht, saved, ws,
                                    (size_t)GDN_NOALLOC_SCRATCH_BYTES, stream);
}
