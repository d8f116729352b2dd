// unfused_det_decode_noalloc: the N-launch detection-decode tail staged
// through a device array that belongs to the library instead of a workspace
// the caller allocates. It is for callers that cannot allocate device memory
// around a call: code under HIP graph capture, serving loops that must not
// call the allocator, harnesses that forbid it. The kernels are those of
// unfused_det_decode; nothing here allocates or frees device memory.
#include <cstdio>
#include <mutex>

#include "internal.h"

namespace {

// 16 MiB: the 3-level 80/40/20 YOLO head (3 anchors x 85 channels, fp16)
// stages 2 x 25,200 x 85 x 2 = 8,568,000 bytes per image.
constexpr size_t kScratchBytes = (size_t)16 << 20;

// One copy per GPU, held until the process ends. Host code never passes this
// name to a kernel or a copy: on the host it is only a stand-in for the
// symbol. scratch_ptr() returns the device address to use.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The device address of `scratch` on the current device, looked up once per
// device with that device current.
int scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return np::set_error(NP_EDEVICE, "no HIP device available for the scratch array");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      char msg[256];
      snprintf(msg, sizeof msg, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
               hipGetErrorString(e));
      return np::set_error(NP_ELAUNCH, msg);
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return NP_OK;
}

}  // namespace

extern "C" int unfused_det_decode_noalloc(const void* const* level_logits, int n_levels,
                                          const int32_t* H, const int32_t* W,
                                          const float* strides, const float* anchors_wh,
                                          int n_anchors, int n_ch, int batch, np_dtype in_dt,
                                          float* out, hipStream_t stream) {
  int rc = np::validate_det_call(level_logits, n_levels, H, W, strides, anchors_wh, n_anchors,
                                 n_ch, batch, in_dt, out);
  if (rc) return rc;
  int64_t rows = 0;
  for (int l = 0; l < n_levels; ++l) rows += (int64_t)n_anchors * H[l] * W[l];
  const int64_t need = 2 * (int64_t)batch * rows * n_ch * np::dt_size(in_dt);
  if (need > (int64_t)kScratchBytes) {
    char msg[256];
    snprintf(msg, sizeof msg,
             "unfused_det_decode_noalloc: the call stages %lld bytes, more than its %zu-byte "
             "scratch array (use unfused_det_decode with a workspace)",
             (long long)need, kScratchBytes);
    return np::set_error(NP_EINVAL, msg);
  }
  if ((rc = np::check_device_call())) return rc;
  void* ws = nullptr;
  if ((rc = scratch_ptr(&ws))) return rc;
  return unfused_det_decode(level_logits, n_levels, H, W, strides, anchors_wh, n_anchors, n_ch,
                            batch, in_dt, out, ws, kScratchBytes, stream);
}
