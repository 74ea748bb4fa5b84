// NVFP4 tensor-scale pass with library-owned scratch, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  Same kernels and bits as qf_nvfp4_tensor_scale_grouped; the amax partials
// live in a fixed device array instead of a caller workspace.
//
// Each GPU holds its own copy of `scratch` until the process ends.  Host code never uses
// the array's name as an address: the first call on a device (with that device current)
// looks up the device address with hipGetSymbolAddress and keeps it per device.  Calls that
// overlap on one GPU share the array and race; every call rewrites all partials it reads,
// so nothing needs clearing between calls.
#include <mutex>

#include "qf_kernels.h"

namespace {
// AMAX_GRID partial maxima per group for up to 16 groups: 128 KiB per GPU.
constexpr int NOALLOC_GROUPS = 16;
constexpr size_t NOALLOC_WORDS = (size_t)qf::AMAX_GRID * NOALLOC_GROUPS;
constexpr int MAX_DEVICES = 64;

void* g_scratch_ptr[MAX_DEVICES];
std::mutex g_scratch_mu;
}  // namespace

static __device__ __align__(256) uint32_t scratch[NOALLOC_WORDS];

namespace {
// Device address of this device's `scratch` (looked up once per device), or an error.
hipError_t scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

extern "C" {

size_t qf_noalloc_scratch_bytes(void) { return sizeof(uint32_t) * NOALLOC_WORDS; }

qf_status qf_nvfp4_tensor_scale_grouped_noalloc(const qf_tensor_desc* d, int n, int n_groups, float* d_scales,
                                                uint32_t* d_nonfinite, void* stream) {
  // every argument, and that the partials fit the fixed array, before any HIP call
  const qf_status chk = qf::check_tensor_scale(d, n, n_groups, d_scales);
  if (chk != QF_OK) return chk;
  if (qf_nvfp4_tensor_scale_workspace(d, n) > qf_noalloc_scratch_bytes()) return QF_ERR_WORKSPACE;
  void* ws = nullptr;
  const hipError_t e = scratch_for_current_device(&ws);
  if (e != hipSuccess) return qf::status_of(e);
  return qf_nvfp4_tensor_scale_grouped(d, n, n_groups, d_scales, d_nonfinite, ws, qf_noalloc_scratch_bytes(),
                                       stream);
}

}  // extern "C"
