// Fused QKV split + rotate-half RoPE + Q scale (TeleTron write-up,
// 2kiu.com/news/5927820, section 3.1: multi-head split, rotary position
// encoding and scaling after the QKV projection, as one fused group).
//
// Input: packed rows [T, 3, H, D]; outputs head-major [H, T, D]. A thread owns
// one token t and one 16-byte chunk j of the first half of a head vector (the
// matching chunk of the second half is its rotation partner). It evaluates the
// chunk's E angles theta = fp32(pos) * inv_i and their sine/cosine once, then
// walks over all H heads of Q (or K) reusing them: a token's 64 angles serve
// all 48 rotated head vectors. Blocks are (token tile) x (q, k, v); V blocks
// are plain 16-byte copies into the head-major layout. Reads and writes are
// full 128-byte lines: 8 lanes cover one 256-byte head vector.
#include "device.h"
#include "internal.h"

namespace np {
namespace {

constexpr int kBlock = 256;

template <typename T, int HU>
__global__ __launch_bounds__(kBlock) void rope_vec(RopeArgs a) {
  constexpr int E = Vec<T>::N;
  const int half = a.D / 2;
  const int P = half / E;            // chunks per half head vector (divides kBlock)
  const int TB = kBlock / P;         // tokens per block
  const int j = threadIdx.x % P;
  const int64_t t = (int64_t)blockIdx.x * TB + threadIdx.x / P;
  const int s = blockIdx.y;          // 0 = q, 1 = k, 2 = v
  if (t >= a.T) return;
  const T* src = static_cast<const T*>(a.qkv) + (t * 3 + s) * (int64_t)a.H * a.D;
  T* dst = static_cast<T*>(s == 0 ? a.q : s == 1 ? a.k : a.v) + t * a.D;
  const int64_t hstride = a.T * a.D;  // distance between heads in the output
  const int lo = j * E;
  const int hi = half + j * E;
  if (s == 2) {
    for (int h = 0; h < a.H; ++h) {
      const u32x4 x0 = load_raw(src + (int64_t)h * a.D + lo);
      const u32x4 x1 = load_raw(src + (int64_t)h * a.D + hi);
      store_raw(dst + h * hstride + lo, x0);
      store_raw(dst + h * hstride + hi, x1);
    }
    return;
  }
  const float p = a.pos ? (float)a.pos[t] : (float)t;
  float cs[E], sn[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float theta = p * a.inv[lo + e];  // one fp32 multiply
    sincosf(theta, &sn[e], &cs[e]);
  }
  const float sc = s == 0 ? a.q_scale : 1.0f;
  int h = 0;
  for (; h + HU <= a.H; h += HU) {
    float u[HU][E], w[HU][E];
#pragma unroll
    for (int k = 0; k < HU; ++k) {
      load_vec<T>(src + (int64_t)(h + k) * a.D + lo, u[k]);
      load_vec<T>(src + (int64_t)(h + k) * a.D + hi, w[k]);
    }
#pragma unroll
    for (int k = 0; k < HU; ++k) {
      float o1[E], o2[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        o1[e] = (u[k][e] * cs[e] - w[k][e] * sn[e]) * sc;
        o2[e] = (w[k][e] * cs[e] + u[k][e] * sn[e]) * sc;
      }
      store_vec<T>(dst + (h + k) * hstride + lo, o1);
      store_vec<T>(dst + (h + k) * hstride + hi, o2);
    }
  }
  for (; h < a.H; ++h) {
    float u[E], w[E], o1[E], o2[E];
    load_vec<T>(src + (int64_t)h * a.D + lo, u);
    load_vec<T>(src + (int64_t)h * a.D + hi, w);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      o1[e] = (u[e] * cs[e] - w[e] * sn[e]) * sc;
      o2[e] = (w[e] * cs[e] + u[e] * sn[e]) * sc;
    }
    store_vec<T>(dst + h * hstride + lo, o1);
    store_vec<T>(dst + h * hstride + hi, o2);
  }
}

// Any layout / alignment: one thread per (token, s, head, pair index).
template <typename T>
__global__ __launch_bounds__(kBlock) void rope_scalar(RopeArgs a) {
  const int half = a.D / 2;
  const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int64_t total = a.T * 3 * a.H * half;
  if (gid >= total) return;
  const int i = (int)(gid % half);
  int64_t rest = gid / half;
  const int h = (int)(rest % a.H);
  rest /= a.H;
  const int s = (int)(rest % 3);
  const int64_t t = rest / 3;
  const T* src = static_cast<const T*>(a.qkv) + ((t * 3 + s) * a.H + h) * (int64_t)a.D;
  T* dst = static_cast<T*>(s == 0 ? a.q : s == 1 ? a.k : a.v) + ((int64_t)h * a.T + t) * a.D;
  if (s == 2) {
    dst[i] = src[i];
    dst[i + half] = src[i + half];
    return;
  }
  const float p = a.pos ? (float)a.pos[t] : (float)t;
  const float theta = p * a.inv[i];
  float sn, cs;
  sincosf(theta, &sn, &cs);
  const float sc = s == 0 ? a.q_scale : 1.0f;
  const float u = to_f(src[i]);
  const float w = to_f(src[i + half]);
  dst[i] = from_f<T>((u * cs - w * sn) * sc);
  dst[i + half] = from_f<T>((w * cs + u * sn) * sc);
}

template <typename T>
hipError_t launch_t(const RopeArgs& a, bool vec, hipStream_t s) {
  constexpr int E = Vec<T>::N;
  const int half = a.D / 2;
  const int P = half / E;
  if (vec && half % E == 0 && P > 0 && kBlock % P == 0) {
    const int TB = kBlock / P;
    const unsigned gx = (unsigned)((a.T + TB - 1) / TB);
    hipLaunchKernelGGL((rope_vec<T, 4>), dim3(gx, 3), dim3(kBlock), 0, s, a);
  } else {
    const int64_t total = a.T * 3 * a.H * (int64_t)half;
    hipLaunchKernelGGL((rope_scalar<T>), dim3((unsigned)((total + kBlock - 1) / kBlock)),
                       dim3(kBlock), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qkv_rope(const RopeArgs& a, int dt, bool vec, hipStream_t s) {
  switch (dt) {
    case NP_F32: return launch_t<float>(a, vec, s);
    case NP_F16: return launch_t<_Float16>(a, vec, s);
    default: return launch_t<__bf16>(a, vec, s);
  }
}

}  // namespace np
