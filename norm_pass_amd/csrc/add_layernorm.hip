// Fused residual add + LayerNorm (DeepJIT write-up, hotelren.com/news/5350627,
// section 4.3: one block per row, the row's mean and variance, normalise,
// affine gamma / beta -- instead of separate mean, variance and normalise
// kernels that each read and write the whole tensor).
//
// Same register structure as the RMSNorm kernel: one workgroup of 4 wave64s
// per row, the row held in registers (VPT 16-byte vectors per thread), so x
// and r are read once and h and out written once. The variance is taken in a
// second pass over the registers, mean((h - mu)^2), rather than the page's
// E[h^2] - mu^2, which cancels catastrophically when |mu| >> sigma. Each
// statistic is a wave64 DPP sum plus one LDS slot per wave (two LDS arrays, so
// the second reduction cannot overwrite partials still being read).
#include "device.h"
#include "internal.h"

namespace np {
namespace {

template <typename T, int VPT, int WAVES, bool HAS_R, bool HAS_G, bool HAS_B, bool HAS_H>
__global__ __launch_bounds__(64 * WAVES) void ln_vec(const T* x, const T* r, const T* g,
                                                     const T* b, T* h, T* out, int cols,
                                                     float eps) {
  constexpr int N = Vec<T>::N;
  constexpr int THREADS = 64 * WAVES;
  __shared__ float part_mu[WAVES], part_var[WAVES];
  const int64_t off = (int64_t)blockIdx.x * cols;
  const int nvec = cols / N;
  float hv[VPT][N];
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
    } else {
#pragma unroll
      for (int e = 0; e < N; ++e) hv[j][e] = 0.0f;
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int vi = threadIdx.x + j * THREADS;
#pragma unroll
    for (int e = 0; e < N; ++e) {
      hv[j][e] = round_via<T>(hv[j][e]);  // the stored h is what the norm sees
      s += hv[j][e];
    }
    if (HAS_H && vi < nvec) store_vec_nt<T>(h + off + vi * N, hv[j]);
  }
  const float mu = block_sum<WAVES>(s, part_mu) / (float)cols;
  float sq = 0.0f;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int vi = threadIdx.x + j * THREADS;
#pragma unroll
    for (int e = 0; e < N; ++e) {
      hv[j][e] -= mu;
      if (vi < nvec) sq += hv[j][e] * hv[j][e];
    }
  }
  const float rstd = 1.0f / sqrtf(block_sum<WAVES>(sq, part_var) / (float)cols + eps);
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int vi = threadIdx.x + j * THREADS;
    if (vi < nvec) {
      float gv[N], bv[N], o[N];
      if (HAS_G) load_vec<T>(g + vi * N, gv);
      if (HAS_B) load_vec<T>(b + vi * N, bv);
#pragma unroll
      for (int e = 0; e < N; ++e) {
        const float y = hv[j][e] * rstd;
        o[e] = HAS_G ? (HAS_B ? fmaf(y, gv[e], bv[e]) : y * gv[e]) : (HAS_B ? y + bv[e] : y);
      }
      store_vec_nt<T>(out + off + vi * N, o);
    }
  }
}

// Any alignment / row length: element by element, three passes over the row.
template <typename T>
__global__ __launch_bounds__(256) void ln_generic(const T* x, const T* r, const T* g,
                                                  const T* b, T* h, T* out, int cols,
                                                  float eps) {
  __shared__ float part_mu[4], part_var[4];
  const int64_t off = (int64_t)blockIdx.x * cols;
  auto hval = [&](int j) {
    float v = to_f(x[off + j]);
    if (r) v += to_f(r[off + j]);
    return round_via<T>(v);
  };
  float s = 0.0f;
  for (int j = threadIdx.x; j < cols; j += 256) {
    const float hj = hval(j);
    if (h) h[off + j] = from_f<T>(hj);
    s += hj;
  }
  const float mu = block_sum<4>(s, part_mu) / (float)cols;
  float sq = 0.0f;
  // h_out may alias x: once stored, read h back rather than recomputing x + r
  for (int j = threadIdx.x; j < cols; j += 256) {
    const float d = (h ? to_f(h[off + j]) : hval(j)) - mu;
    sq += d * d;
  }
  const float rstd = 1.0f / sqrtf(block_sum<4>(sq, part_var) / (float)cols + eps);
  for (int j = threadIdx.x; j < cols; j += 256) {
    const float y = ((h ? to_f(h[off + j]) : hval(j)) - mu) * rstd;
    const float gj = g ? to_f(g[j]) : 1.0f;
    const float bj = b ? to_f(b[j]) : 0.0f;
    out[off + j] = from_f<T>(fmaf(y, gj, bj));
  }
}

template <typename T, int VPT, int WAVES, bool HAS_R, bool HAS_G, bool HAS_B, bool HAS_H>
void launch5(const void* x, const void* r, const void* g, const void* b, void* h, void* out,
             int64_t rows, int cols, float eps, hipStream_t s) {
  hipLaunchKernelGGL((ln_vec<T, VPT, WAVES, HAS_R, HAS_G, HAS_B, HAS_H>), dim3((unsigned)rows),
                     dim3(64 * WAVES), 0, s, static_cast<const T*>(x), static_cast<const T*>(r),
                     static_cast<const T*>(g), static_cast<const T*>(b), static_cast<T*>(h),
                     static_cast<T*>(out), cols, eps);
}

template <typename T, int VPT, int WAVES>
void launch_flags(const void* x, const void* r, const void* g, const void* b, void* h, void* out,
                  int64_t rows, int cols, float eps, hipStream_t s) {
  const int key = (r ? 8 : 0) | (g ? 4 : 0) | (b ? 2 : 0) | (h ? 1 : 0);
  switch (key) {
#define NP_LN_CASE(K, R, G, B, H) \
  case K: launch5<T, VPT, WAVES, R, G, B, H>(x, r, g, b, h, out, rows, cols, eps, s); break;
    NP_LN_CASE(15, true, true, true, true)
    NP_LN_CASE(14, true, true, true, false)
    NP_LN_CASE(13, true, true, false, true)
    NP_LN_CASE(12, true, true, false, false)
    NP_LN_CASE(11, true, false, true, true)
    NP_LN_CASE(10, true, false, true, false)
    NP_LN_CASE(9, true, false, false, true)
    NP_LN_CASE(8, true, false, false, false)
    NP_LN_CASE(7, false, true, true, true)
    NP_LN_CASE(6, false, true, true, false)
    NP_LN_CASE(5, false, true, false, true)
    NP_LN_CASE(4, false, true, false, false)
    NP_LN_CASE(3, false, false, true, true)
    NP_LN_CASE(2, false, false, true, false)
    NP_LN_CASE(1, false, false, false, true)
    NP_LN_CASE(0, false, false, false, false)
#undef NP_LN_CASE
  }
}

template <typename T>
hipError_t launch_t(const void* x, const void* r, const void* g, const void* b, void* h,
                    void* out, int64_t rows, int64_t cols, float eps, bool vec, hipStream_t s) {
  constexpr int N = Vec<T>::N;
  const int64_t nvec = cols / N;
  // the row-length policy of the RMSNorm kernel: 4 waves up to 256 vectors,
  // then 8 waves with 1, 2 or 4 vectors per thread
  if (vec && cols % N == 0 && nvec <= 512 * 4) {
    const int c = (int)cols;
    if (nvec <= 256)
      launch_flags<T, 1, 4>(x, r, g, b, h, out, rows, c, eps, s);
    else if (nvec <= 512)
      launch_flags<T, 1, 8>(x, r, g, b, h, out, rows, c, eps, s);
    else if (nvec <= 1024)
      launch_flags<T, 2, 8>(x, r, g, b, h, out, rows, c, eps, s);
    else
      launch_flags<T, 4, 8>(x, r, g, b, h, out, rows, c, eps, s);
  } else {
    hipLaunchKernelGGL((ln_generic<T>), dim3((unsigned)rows), dim3(256), 0, s,
                       static_cast<const T*>(x), static_cast<const T*>(r),
                       static_cast<const T*>(g), static_cast<const T*>(b), static_cast<T*>(h),
                       static_cast<T*>(out), (int)cols, eps);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_add_layernorm(const void* x, const void* r, const void* g, const void* b,
                                void* h, void* out, int64_t rows, int64_t cols, float eps, int dt,
                                bool vec, hipStream_t s) {
  switch (dt) {
    case NP_F32: return launch_t<float>(x, r, g, b, h, out, rows, cols, eps, vec, s);
    case NP_F16: return launch_t<_Float16>(x, r, g, b, h, out, rows, cols, eps, vec, s);
    default: return launch_t<__bf16>(x, r, g, b, h, out, rows, cols, eps, vec, s);
  }
}

}  // namespace np
