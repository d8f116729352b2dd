// Fused residual add + RMSNorm (TeleTron write-up, 2kiu.com/news/5927820,
// sections 3.3 and 4.2: per-row local reduction, then elementwise scaling, fp32
// accumulation, one block per row, vector loads of 8 elements).
//
// Register path: one workgroup of WAVES wave64s per row; each thread holds VPT
// 16-byte vectors of the row in registers between the two phases, so x and r
// are read once and h and out written once (non-temporal stores: the outputs
// are not read again by this kernel):
//   h = round(x + r) -> store h; sum of h^2 in fp32 per thread -> wave64 DPP
//   reduction -> one LDS slot per wave -> every thread adds the WAVES partials
//   in a fixed order -> rstd = 1/sqrt(mean + eps) -> out = h * rstd * w.
// Generic path (unaligned pointers, odd or very long rows): the same per-row
// block, element by element, in two passes.
#include "device.h"
#include "internal.h"

namespace np {
namespace {

template <typename T, int VPT, int WAVES, bool HAS_R, bool HAS_W, bool HAS_H>
__global__ __launch_bounds__(64 * WAVES) void rms_vec(const T* x, const T* r, const T* w, T* h,
                                                      T* out, int cols, float eps) {
  constexpr int N = Vec<T>::N;
  constexpr int THREADS = 64 * WAVES;
  __shared__ float part[WAVES];
  const int64_t off = (int64_t)blockIdx.x * cols;
  const int nvec = cols / N;
  float hv[VPT][N];
  float wv[VPT][N];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int vi = threadIdx.x + j * THREADS;
    if (vi < nvec) {
      load_vec<T>(x + off + vi * N, hv[j]);
      if (HAS_R) {
        float rv[N];
        load_vec<T>(r + off + vi * N, rv);
#pragma unroll
        for (int e = 0; e < N; ++e) hv[j][e] += rv[e];
      }
      if (HAS_W) {
        load_vec<T>(w + vi * N, wv[j]);
      } else {
#pragma unroll
        for (int e = 0; e < N; ++e) wv[j][e] = 1.0f;
      }
    } else {
#pragma unroll
      for (int e = 0; e < N; ++e) hv[j][e] = wv[j][e] = 0.0f;
    }
  }
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int vi = threadIdx.x + j * THREADS;
#pragma unroll
    for (int e = 0; e < N; ++e) {
      hv[j][e] = round_via<T>(hv[j][e]);  // the stored h is what the norm sees
      ss += hv[j][e] * hv[j][e];
    }
    if (HAS_H && vi < nvec) store_vec_nt<T>(h + off + vi * N, hv[j]);
  }
  const float tot = block_sum<WAVES>(ss, part);
  const float rstd = 1.0f / sqrtf(tot / (float)cols + eps);
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int vi = threadIdx.x + j * THREADS;
    if (vi < nvec) {
      float o[N];
#pragma unroll
      for (int e = 0; e < N; ++e) o[e] = hv[j][e] * rstd * wv[j][e];
      store_vec_nt<T>(out + off + vi * N, o);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void rms_generic(const T* x, const T* r, const T* w, T* h,
                                                   T* out, int cols, float eps) {
  __shared__ float part[4];
  const int64_t off = (int64_t)blockIdx.x * cols;
  float ss = 0.0f;
  for (int j = threadIdx.x; j < cols; j += 256) {
    float s = to_f(x[off + j]);
    if (r) s += to_f(r[off + j]);
    const float hr = round_via<T>(s);
    if (h) h[off + j] = from_f<T>(hr);
    ss += hr * hr;
  }
  const float tot = block_sum<4>(ss, part);
  const float rstd = 1.0f / sqrtf(tot / (float)cols + eps);
  for (int j = threadIdx.x; j < cols; j += 256) {
    float hr;
    if (h) {
      hr = to_f(h[off + j]);  // written by this thread in pass 1
    } else {
      float s = to_f(x[off + j]);
      if (r) s += to_f(r[off + j]);
      hr = round_via<T>(s);
    }
    const float wj = w ? to_f(w[j]) : 1.0f;
    out[off + j] = from_f<T>(hr * rstd * wj);
  }
}

template <typename T, int VPT, int WAVES, bool HAS_R, bool HAS_W, bool HAS_H>
void launch_vec3(const void* x, const void* r, const void* w, void* h, void* out, int64_t rows,
                 int cols, float eps, hipStream_t s) {
  hipLaunchKernelGGL((rms_vec<T, VPT, WAVES, HAS_R, HAS_W, HAS_H>), dim3((unsigned)rows),
                     dim3(64 * WAVES), 0, s, static_cast<const T*>(x), static_cast<const T*>(r),
                     static_cast<const T*>(w), static_cast<T*>(h), static_cast<T*>(out), cols,
                     eps);
}

template <typename T, int VPT, int WAVES>
void launch_vec(const void* x, const void* r, const void* w, void* h, void* out, int64_t rows,
                int cols, float eps, hipStream_t s) {
  const int key = (r ? 4 : 0) | (w ? 2 : 0) | (h ? 1 : 0);
#define NP_RMS_CASE(K, R, W, H) \
  case K: launch_vec3<T, VPT, WAVES, R, W, H>(x, r, w, h, out, rows, cols, eps, s); break;
  switch (key) {
    NP_RMS_CASE(7, true, true, true)
    NP_RMS_CASE(6, true, true, false)
    NP_RMS_CASE(5, true, false, true)
    NP_RMS_CASE(4, true, false, false)
    NP_RMS_CASE(3, false, true, true)
    NP_RMS_CASE(2, false, true, false)
    NP_RMS_CASE(1, false, false, true)
    default: launch_vec3<T, VPT, WAVES, false, false, false>(x, r, w, h, out, rows, cols, eps, s);
  }
#undef NP_RMS_CASE
}

template <typename T>
hipError_t launch_t(const void* x, const void* r, const void* w, void* h, void* out,
                    int64_t rows, int64_t cols, float eps, bool vec, hipStream_t s) {
  constexpr int N = Vec<T>::N;
  const int64_t nvec = cols / N;
  // rows of up to 256 vectors: 4 waves, one vector per thread; longer rows: 8
  // waves with 1, 2 or 4 vectors per thread (measured at [16384, 4096] bf16:
  // 8 waves x 1 vector 73.3 / 87.7 us warm / cold against 74.6 / 88.6 us for
  // 4 waves x 2 vectors)
  if (vec && cols % N == 0 && nvec <= 512 * 4) {
    if (nvec <= 256)
      launch_vec<T, 1, 4>(x, r, w, h, out, rows, (int)cols, eps, s);
    else if (nvec <= 512)
      launch_vec<T, 1, 8>(x, r, w, h, out, rows, (int)cols, eps, s);
    else if (nvec <= 1024)
      launch_vec<T, 2, 8>(x, r, w, h, out, rows, (int)cols, eps, s);
    else
      launch_vec<T, 4, 8>(x, r, w, h, out, rows, (int)cols, eps, s);
  } else {
    hipLaunchKernelGGL((rms_generic<T>), dim3((unsigned)rows), dim3(256), 0, s,
                       static_cast<const T*>(x), static_cast<const T*>(r),
                       static_cast<const T*>(w), static_cast<T*>(h), static_cast<T*>(out),
                       (int)cols, eps);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_add_rmsnorm(const void* x, const void* r, const void* w, void* h, void* out,
                              int64_t rows, int64_t cols, float eps, int dt, bool vec,
                              hipStream_t s) {
  switch (dt) {
    case NP_F32: return launch_t<float>(x, r, w, h, out, rows, cols, eps, vec, s);
    case NP_F16: return launch_t<_Float16>(x, r, w, h, out, rows, cols, eps, vec, s);
    default: return launch_t<__bf16>(x, r, w, h, out, rows, cols, eps, vec, s);
  }
}

}  // namespace np
