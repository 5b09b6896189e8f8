// gdn_chunk_fwd_noalloc: the whole forward with its workspace in a fixed
// device array of the library instead of caller memory, for callers that
// cannot allocate (code under HIP graph capture, tight serving loops, hosts
// that forbid allocation after start-up).
//
// `scratch` is a file-scope device array. In host code its name is only a
// host-side stand-in: passing it to a kernel compiles but faults on the GPU.
// Its device address is taken once per device with hipGetSymbolAddress, with
// that device current, and only that address is ever handed to kernels. Each
// GPU holds its own copy, at its own address, until the process ends.
//
// Every call on one device shares that device's array and leaves the last
// call's intermediates in it. The forward writes every intermediate before it
// reads it (stage 1 fills the fragment blocks, the chunk table and the
// sequence ranking; stage 2 reads only those), so nothing has to start at
// zero. Calls that overlap in time on one device (different streams, or host
// threads racing to enqueue) race on the array: the caller orders them.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn.h"

namespace {

constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

std::mutex g_mutex;
void *g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the current device, taken once per device.
gdn_status scratch_of_current_device(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GDN_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return GDN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GDN_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return GDN_OK;
}

}  // namespace

extern "C" gdn_status gdn_chunk_fwd_noalloc(const gdn_config *cfg, const void *q, const void *k,
                                            const void *v, const float *g, const float *beta,
                                            const float *h0, const int32_t *cu_seqlens,
                                            const int32_t *chunk_indices, void *o, float *hT,
                                            void *stream) {
  size_t need = 0;
  const gdn_status st = gdn_workspace_size(cfg, &need);  // validates cfg
  if (st != GDN_OK) return st;
  if (need > static_cast<size_t>(GDN_NOALLOC_SCRATCH_BYTES)) return GDN_ERR_WORKSPACE;
  void *ws = nullptr;
  const gdn_status sc = scratch_of_current_device(&ws);
  if (sc != GDN_OK) return sc;
  // every other argument is checked here, on the host, before any launch
  return gdn_chunk_fwd(cfg, q, k, v, g, beta, h0, cu_seqlens, chunk_indices, o, hT, ws,
                       static_cast<size_t>(GDN_NOALLOC_SCRATCH_BYTES), stream);
}
