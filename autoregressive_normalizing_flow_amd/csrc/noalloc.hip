// Allocation-free variant of the fused affine kernel's entry point, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc): the kernel's
// cross-block scratch (per-block partial sums and the ticket counter) lives in
// a static device array of this library instead of a caller buffer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/af.h"
#include "kernels.h"

namespace {

constexpr size_t kScratchBytes = 256 * 1024;
static_assert(kScratchBytes == AF_NOALLOC_SCRATCH_BYTES, "header limit");

// One copy per GPU, held until the process ends.  In host code `scratch`
// names a host-side stand-in: only the per-device address obtained below is
// ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device

// The current device's copy of `scratch`, looked up once per device.
af_status scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return (af_status)af::record_error(AF_ERR_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return (af_status)af::record_error(AF_ERR_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return (af_status)af::record_error(
          AF_ERR_HIP, e != hipSuccess ? hipGetErrorString(e) : "no address for scratch");
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return AF_OK;
}

}  // namespace

extern "C" af_status afk_affine_noalloc(int mode, const float* head, const float* src,
                                        float* dst, int N, int rows_per_sample, int C,
                                        float* res, void* stream) {
  if (mode != 0 && mode != 1)
    return (af_status)af::record_error(AF_ERR_ARG, "mode must be 0 or 1");
  if (!head || !src || !dst || !res)
    return (af_status)af::record_error(AF_ERR_ARG, "NULL argument");
  if (src == dst) return (af_status)af::record_error(AF_ERR_ARG, "src and dst may not alias");
  if (N < 1 || rows_per_sample < 1 || C < 1 || C > 256)
    return (af_status)af::record_error(AF_ERR_ARG, "bad sizes");
  const size_t need = afk_affine_partials_bytes(N, rows_per_sample, C);
  if (need > kScratchBytes)
    return (af_status)af::record_error(
        AF_ERR_WORKSPACE, "afk_affine_noalloc: N x partial groups exceed the static scratch of "
                          "AF_NOALLOC_SCRATCH_BYTES (256 KiB)");
  void* base = nullptr;
  if (af_status s = scratch_of_current_device(&base)) return s;
  hipStream_t st = (hipStream_t)stream;
  char* pb = (char*)base;
  unsigned* counter = (unsigned*)(pb + need - 256);
  // the array keeps the last call's contents: the ticket counter must start
  // at zero (a fill kernel, so that the call can be captured into a graph)
  hipError_t e = af::launch_fill_u32(counter, 0u, 1, st);
  if (e != hipSuccess) return (af_status)af::record_error(AF_ERR_HIP, hipGetErrorString(e));
  af::AffineArgs aa{head, nullptr, 1, mode == 0 ? src : nullptr,
                    mode == 0 ? dst : const_cast<float*>(src), mode == 1 ? dst : nullptr,
                    N, rows_per_sample, C, rows_per_sample, 0, 0, (float*)pb, res, counter,
                    nullptr};
  e = af::launch_affine(mode, aa, st);
  if (e != hipSuccess) return (af_status)af::record_error(AF_ERR_HIP, hipGetErrorString(e));
  return AF_OK;
}
