// The allocation-free form of the megabatched step: the workspace is a
// static device array of DION3_STATIC_SCRATCH_BYTES (one copy per GPU the
// library runs on, held until the process ends) instead of caller memory, for
// callers that cannot allocate device memory.  The array's device address is
// looked up once per device with hipGetSymbolAddress and only that address is
// ever handed to kernels or copies: in host code the array's name is a
// host-side stand-in, not a device address.
#include <mutex>

#include "../../include/dion3.h"
#include "dion3_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[DION3_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// The device address of `scratch` on device `dev` (the current device).
dion3_status scratch_of(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return DION3_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return dion3::note_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol);
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return DION3_OK;
}

}  // namespace

extern "C" {

dion3_status dion3_step_megabatch_noalloc(float* const* W, float* const* M, int32_t batch,
                                          int64_t n, int64_t m, int64_t ld, int64_t k, float lr,
                                          float mu, const dion3_ns_cfg* cfg, int32_t* idx_out,
                                          uint16_t* O_out, void* stream) {
  if (!W || !M) return DION3_ERR_ARG;
  size_t need = 0;
  dion3_status st = dion3_workspace_size(batch, n, m, k, &need);
  if (st != DION3_OK) return st;
  if (need > (size_t)DION3_STATIC_SCRATCH_BYTES) return DION3_ERR_WORKSPACE;
  // the stream must belong to the current device, whose copy of the array is used
  int dev = 0, sdev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipStreamGetDevice((hipStream_t)stream, &sdev);
  if (e != hipSuccess) return dion3::note_hip_error(e);
  if (sdev != dev) return DION3_ERR_ARG;
  void* ws = nullptr;
  st = scratch_of(dev, &ws);
  if (st != DION3_OK) return st;
  return dion3_step_megabatch(W, M, batch, n, m, ld, k, lr, mu, cfg, idx_out, O_out, ws,
                              (size_t)DION3_STATIC_SCRATCH_BYTES, stream);
}

}  // extern "C"
