// Fused QKV split + rotate-half RoPE + Q scale (TeleTron write-up,
// 2kiu.com/news/5927820, section 3.1: multi-head split, rotary position
// encoding and scaling after the QKV projection, as one fused group).
//
// Main path (head vectors of exactly 16 chunks of 16 bytes, e.g. D = 128 in
// bf16): one workgroup per token streams the token's packed row [3, H, D]
// front to back, one 16-byte chunk per lane, so reads are fully sequential. A
// head vector then sits in one 16-lane DPP row and the rotation partner of
// chunk j (j +- 8, the other half) is fetched from the neighbouring lane with
// row_ror:8 instead of being loaded again. The token's D/2 angles and their
// sine/cosine are computed once into LDS (also pre-multiplied by q_scale for
// Q, so Q costs no extra multiply) and shared by all 2H rotated vectors.
// Writes are whole 256-byte head vectors into the head-major outputs, with the
// non-temporal hint (nothing reads them back here).
//
// Other layouts: packed rows [T, 3, H, D]; outputs head-major [H, T, D]. A thread owns
// one token t and one 16-byte chunk j of the first half of a head vector (the
// matching chunk of the second half is its rotation partner). It evaluates the
// chunk's E angles theta = fp32(pos) * inv_i and their sine/cosine once, then
// walks over all H heads of Q (or K) reusing them: a token's 64 angles serve
// all 48 rotated head vectors. Blocks are (token tile) x (q, k, v); V blocks
// are plain 16-byte copies into the head-major layout. Reads and writes are
// full 128-byte lines: 8 lanes cover one 256-byte head vector.
#include <algorithm>

#include "device.h"
#include "internal.h"

namespace np {

namespace {

constexpr int kBlock = 256;
// Threads per token workgroup. At H = 24, D = 128 bf16 a token is 1152 chunks:
// 768 threads take two passes (the second half full). Measured on MI355X,
// 16384 tokens, warm / cold: 384 threads 100-103 / 107-108 us; 640-896
// threads 100-101 / 100-101 us; 288 threads 104-105 / 109 us.
#ifndef NP_ROPE_TOK_BLOCK
#define NP_ROPE_TOK_BLOCK 768
#endif
constexpr int kTokBlock = NP_ROPE_TOK_BLOCK;

template <typename T, int NC>
__global__ __launch_bounds__(kTokBlock) void rope_tok(RopeArgs a) {
  using RT = rope_math_t<T>;
  constexpr int E = Vec<T>::N;  // elements per 16-byte chunk; D == 16 * E here
  constexpr int HALF = 8 * E;
  // cos / sin of the token's angles, plain (K) and multiplied by q_scale (Q)
  static_assert(HALF <= kTokBlock, "one angle per thread at most");
  __shared__ RT tab[4][HALF];
  const int64_t t = a.t0 + blockIdx.x;
  // the angle inputs, then the row's loads, then the angle table: waits count
  // loads in issue order, so the table is computed while the row is in flight
  const int ia = threadIdx.x;  // this thread's angle, if any
  const float p = a.pos ? (float)a.pos[t] : (float)t;
  const float inv = ia < HALF ? a.inv[ia] : 0.0f;
  const int total = 3 * a.H * 16;  // chunks in the token's packed row
  const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const T*>(a.qkv)) + t * total;
  u32x4 raw[NC];
#pragma unroll
  for (int q = 0; q < NC; ++q) {
    const int c = threadIdx.x + q * kTokBlock;
    raw[q] = load_raw(src + (c < total ? c : 0));
  }
  if (ia < HALF) {
    RT sv, cv;
    rope_sincos(p * inv, &sv, &cv);  // theta = fp32(pos) * inv_i: one fp32 multiply
    tab[0][ia] = cv;
    tab[1][ia] = sv;
    tab[2][ia] = cv * (RT)a.q_scale;
    tab[3][ia] = sv * (RT)a.q_scale;
  }
  __syncthreads();
  const int l16 = threadIdx.x & 15;
  const bool second = l16 >= 8;
  const int f0 = (l16 & 7) * E;
  const float inv_h = 1.0f / (float)a.H;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = threadIdx.x + i * kTokBlock;
    const int hv = c >> 4;  // head vector within the token: s * H + h
    // s = hv / H, exact: (hv + 0.5) / H is at least 0.5 / H away from an integer
    const int s = (int)(((float)hv + 0.5f) * inv_h);
    const int h = hv - s * a.H;
    u32x4 res = raw[i];
    // the DPP partner read needs every lane of the row: all lanes take part,
    // V lanes keep their raw chunk (the branch is wave-uniform when H % 4 == 0)
    T e_in[E];
    __builtin_memcpy(e_in, &raw[i], 16);
    float x[E], pr[E];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = to_f(e_in[e]);
#pragma unroll
    for (int e = 0; e < E; ++e) pr[e] = dpp_f<0x128>(x[e]);  // row_ror:8 -> partner half
    if (s < 2) {
      const RT* cs = tab[s == 0 ? 2 : 0] + f0;
      const RT* sn = tab[s == 0 ? 3 : 1] + f0;
      T e_out[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const RT xe = x[e], pe = pr[e];
        e_out[e] = from_f<T>((float)(second ? xe * cs[e] + pe * sn[e] : xe * cs[e] - pe * sn[e]));
      }
      __builtin_memcpy(&res, e_out, 16);
    }
    if (c < total) {
      T* dst = static_cast<T*>(s == 0 ? a.q : s == 1 ? a.k : a.v);
      store_raw_nt(reinterpret_cast<u32x4*>(dst) + ((int64_t)h * a.T + t) * 16 + l16, res);
    }
  }
}

template <typename T, int HU>
__global__ __launch_bounds__(kBlock) void rope_vec(RopeArgs a) {
  constexpr int E = Vec<T>::N;
  const int half = a.D / 2;
  const int P = half / E;            // chunks per half head vector (divides kBlock)
  const int TB = kBlock / P;         // tokens per block
  const int j = threadIdx.x % P;
  const int64_t t = a.t0 + (int64_t)blockIdx.x * TB + threadIdx.x / P;
  const int s = blockIdx.y;          // 0 = q, 1 = k, 2 = v
  if (t >= a.t_end) return;
  const T* src = static_cast<const T*>(a.qkv) + (t * 3 + s) * (int64_t)a.H * a.D;
  T* dst = static_cast<T*>(s == 0 ? a.q : s == 1 ? a.k : a.v) + t * a.D;
  const int64_t hstride = a.T * a.D;  // distance between heads in the output
  const int lo = j * E;
  const int hi = half + j * E;
  if (s == 2) {
    for (int h = 0; h < a.H; ++h) {
      const u32x4 x0 = load_raw(src + (int64_t)h * a.D + lo);
      const u32x4 x1 = load_raw(src + (int64_t)h * a.D + hi);
      store_raw_nt(dst + h * hstride + lo, x0);
      store_raw_nt(dst + h * hstride + hi, x1);
    }
    return;
  }
  using RT = rope_math_t<T>;
  const float p = a.pos ? (float)a.pos[t] : (float)t;
  RT cs[E], sn[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float theta = p * a.inv[lo + e];  // one fp32 multiply
    rope_sincos(theta, &sn[e], &cs[e]);
  }
  const RT sc = s == 0 ? (RT)a.q_scale : (RT)1;
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
        const RT ue = u[k][e], we = w[k][e];
        o1[e] = (float)((ue * cs[e] - we * sn[e]) * sc);
        o2[e] = (float)((we * cs[e] + ue * sn[e]) * sc);
      }
      store_vec_nt<T>(dst + (h + k) * hstride + lo, o1);
      store_vec_nt<T>(dst + (h + k) * hstride + hi, o2);
    }
  }
  for (; h < a.H; ++h) {
    float u[E], w[E], o1[E], o2[E];
    load_vec<T>(src + (int64_t)h * a.D + lo, u);
    load_vec<T>(src + (int64_t)h * a.D + hi, w);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const RT ue = u[e], we = w[e];
      o1[e] = (float)((ue * cs[e] - we * sn[e]) * sc);
      o2[e] = (float)((we * cs[e] + ue * sn[e]) * sc);
    }
    store_vec_nt<T>(dst + h * hstride + lo, o1);
    store_vec_nt<T>(dst + h * hstride + hi, o2);
  }
}

// Any layout / alignment: one thread per (token, s, head, pair index).
template <typename T>
__global__ __launch_bounds__(kBlock) void rope_scalar(RopeArgs a) {
  const int half = a.D / 2;
  const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int64_t total = (a.t_end - a.t0) * 3 * a.H * half;
  if (gid >= total) return;
  const int i = (int)(gid % half);
  int64_t rest = gid / half;
  const int h = (int)(rest % a.H);
  rest /= a.H;
  const int s = (int)(rest % 3);
  const int64_t t = a.t0 + rest / 3;
  const T* src = static_cast<const T*>(a.qkv) + ((t * 3 + s) * a.H + h) * (int64_t)a.D;
  T* dst = static_cast<T*>(s == 0 ? a.q : s == 1 ? a.k : a.v) + ((int64_t)h * a.T + t) * a.D;
  if (s == 2) {
    dst[i] = src[i];
    dst[i + half] = src[i + half];
    return;
  }
  using RT = rope_math_t<T>;
  const float p = a.pos ? (float)a.pos[t] : (float)t;
  const float theta = p * a.inv[i];
  RT sn, cs;
  rope_sincos(theta, &sn, &cs);
  const RT sc = s == 0 ? (RT)a.q_scale : (RT)1;
  const RT u = to_f(src[i]);
  const RT w = to_f(src[i + half]);
  dst[i] = from_f<T>((float)((u * cs - w * sn) * sc));
  dst[i + half] = from_f<T>((float)((w * cs + u * sn) * sc));
}

template <typename T, int NC>
void launch_tok(const RopeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((rope_tok<T, NC>), dim3((unsigned)(a.t_end - a.t0)), dim3(kTokBlock), 0, s,
                     a);
}

// A dispatch grid counts at most 2^32 work-items, so long calls are split into
// launches over token ranges [t0, t_end) (the kernels index q, k, v with the
// whole call's T). Token launches: 2^21 tokens x 768 threads < 2^31 items.
constexpr int64_t kTokChunk = (int64_t)1 << 21;
constexpr int64_t kMaxItems = (int64_t)1 << 31;

template <typename T>
hipError_t launch_t(const RopeArgs& a0, bool vec, hipStream_t s) {
  constexpr int E = Vec<T>::N;
  const int half = a0.D / 2;
  const int P = half / E;
  const int nc = (3 * a0.H * 16 + kTokBlock - 1) / kTokBlock;
  const int path = (vec && a0.D == 16 * E && nc <= 8) ? 0
                   : (vec && half % E == 0 && P > 0 && kBlock % P == 0) ? 1 : 2;
  // scalar path: one thread per (token, q/k/v, head, pair)
  const int64_t chunk = path < 2 ? kTokChunk
                                 : std::max<int64_t>(1, kMaxItems / (3 * (int64_t)a0.H * half));
  for (int64_t t0 = 0; t0 < a0.T; t0 += chunk) {
    RopeArgs a = a0;
    a.t0 = t0;
    a.t_end = std::min(a0.T, t0 + chunk);
    if (path == 0) {
      switch (nc) {
        case 1: launch_tok<T, 1>(a, s); break;
        case 2: launch_tok<T, 2>(a, s); break;
        case 3: launch_tok<T, 3>(a, s); break;
        case 4: launch_tok<T, 4>(a, s); break;
        case 5: launch_tok<T, 5>(a, s); break;
        case 6: launch_tok<T, 6>(a, s); break;
        case 7: launch_tok<T, 7>(a, s); break;
        default: launch_tok<T, 8>(a, s); break;
      }
    } else if (path == 1) {
      const int TB = kBlock / P;
      const unsigned gx = (unsigned)((a.t_end - a.t0 + TB - 1) / TB);
      hipLaunchKernelGGL((rope_vec<T, 4>), dim3(gx, 3), dim3(kBlock), 0, s, a);
    } else {
      const int64_t total = (a.t_end - a.t0) * 3 * a.H * (int64_t)half;
      hipLaunchKernelGGL((rope_scalar<T>), dim3((unsigned)((total + kBlock - 1) / kBlock)),
                         dim3(kBlock), 0, s, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
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
