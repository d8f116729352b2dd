// RMSNorm + linear + scale on the matrix cores (TeleTron write-up, section
// 4.2: the row's RMS factor is computed inside the linear layer's kernel and
// applied to its accumulation, so no normalised tensor is written or re-read).
//
//   out[m, n] = scale * (rstd_m * sum_k a_mk Wt[n, k] + bias_n)
//   a_mk = x_mk * w_k rounded to T,  rstd_m = 1 / sqrt(mean_k x_mk^2 + eps)
//
// rstd_m is constant along k, so it factors out of the dot product: the kernel
// runs the GEMM of a = x * w and, from the same x tiles while they pass
// through registers on their way to LDS, accumulates each row's sum of
// squares; the epilogue scales the accumulator by rstd. x is read exactly as
// a plain GEMM reads its A operand; there is no separate norm pass.
//
// Tiles: 128 x 128 outputs per 256-thread workgroup, K in steps of 64 (a
// partial last step reads zeros); each wave owns 64 x 64 outputs as 2 x 2
// blocks of v_mfma_f32_32x32x16 (bf16 or f16 inputs, fp32 accumulation).
// Operand layout of that instruction: lane l supplies A[l % 32][8 (l / 32) ..
// + 8] and B[8 (l / 32) .. + 8][l % 32] (16 contiguous bytes of a K-contiguous
// row each); accumulator register j of lane l is C[8 (j / 4) + 4 (l / 32) +
// j % 4][l % 32]. The next K step's global loads are issued before the current
// step's MFMAs, so they are in flight while the matrix cores run.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"
#include "internal.h"

namespace np {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename T>
struct Mfma;
template <>
struct Mfma<__bf16> {
  typedef __bf16 v8 __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ f32x16 run(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Mfma<_Float16> {
  typedef _Float16 v8 __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ f32x16 run(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int PITCH = BK + 8;  // elements; 144-byte LDS rows keep 8 lanes' 16-byte reads in distinct banks
constexpr int NTHR = 256;

// NORM: accumulate sum of squares and scale by rstd (fused form); otherwise a
// plain GEMM with bias (the unfused form's linear layer). HAS_W: multiply the
// A operand by the norm weight on its way to LDS.
template <typename T, bool NORM, bool HAS_W, bool HAS_B>
__global__ __launch_bounds__(NTHR) void rms_linear_mfma(const T* __restrict__ x,
                                                        const T* __restrict__ w,
                                                        const T* __restrict__ Wt,
                                                        const T* __restrict__ bias,
                                                        T* __restrict__ out, int M, int N, int K,
                                                        float eps, float scale) {
  typedef typename Mfma<T>::v8 v8;
  __shared__ __attribute__((aligned(16))) T As[BM * PITCH];
  __shared__ __attribute__((aligned(16))) T Bs[BN * PITCH];
  __shared__ float rstd_s[BM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  // staging map: vector i of this thread is row tid / 8 + 32 i, k chunk tid % 8
  const int srow = tid >> 3, kc = (tid & 7) * 8;
  const T* xrow[4];
  const T* brow[4];
  bool mval[4], nval[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gm = m0 + srow + 32 * i, gn = n0 + srow + 32 * i;
    mval[i] = gm < M;
    nval[i] = gn < N;
    xrow[i] = x + (int64_t)(mval[i] ? gm : M - 1) * K;  // clamped: always a valid row
    brow[i] = Wt + (int64_t)(nval[i] ? gn : N - 1) * K;
  }
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 xa[4], xb[4], wa = zero;
  auto load_step = [&](int k0) {
    const int gk = k0 + kc;
    const bool kval = gk < K;  // K % 8 == 0: a vector is wholly inside or outside
    const int lk = kval ? gk : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 va = load_raw(xrow[i] + lk);
      const u32x4 vb = load_raw(brow[i] + lk);
      xa[i] = (kval && mval[i]) ? va : zero;
      xb[i] = (kval && nval[i]) ? vb : zero;
    }
    if (HAS_W) wa = load_raw(w + lk);
  };
  float ss[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  auto store_step = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 av = xa[i];
      if (NORM || HAS_W) {
        T e[8], wv[8];
        __builtin_memcpy(e, &xa[i], 16);
        if (HAS_W) __builtin_memcpy(wv, &wa, 16);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float f = to_f(e[j]);
          if (NORM) ss[i] = __builtin_fmaf(f, f, ss[i]);
          if (HAS_W) e[j] = from_f<T>(f * to_f(wv[j]));  // exact product, one rounding to T
        }
        if (HAS_W) __builtin_memcpy(&av, e, 16);
      }
      *reinterpret_cast<u32x4*>(&As[(srow + 32 * i) * PITCH + kc]) = av;
      *reinterpret_cast<u32x4*>(&Bs[(srow + 32 * i) * PITCH + kc]) = xb[i];
    }
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int ksteps = (K + BK - 1) / BK;
  load_step(0);
  const int arow = wm * 64 + (lane & 31), brw = wn * 64 + (lane & 31), kl = (lane >> 5) * 8;
  for (int t = 0; t < ksteps; ++t) {
    __syncthreads();  // the previous step's MFMA operands have been read
    store_step();
    __syncthreads();
    if (t + 1 < ksteps) load_step((t + 1) * BK);  // in flight during the MFMAs below
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      v8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const u32x4 ra = *reinterpret_cast<const u32x4*>(&As[(arow + 32 * i) * PITCH + ks * 16 + kl]);
        const u32x4 rb = *reinterpret_cast<const u32x4*>(&Bs[(brw + 32 * i) * PITCH + ks * 16 + kl]);
        __builtin_memcpy(&a[i], &ra, 16);
        __builtin_memcpy(&b[i], &rb, 16);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = Mfma<T>::run(a[i], b[j], acc[i][j]);
    }
  }
  // rstd per row: the 8 lanes that staged a row hold its partial sums
  if (NORM) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = ss[i];
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      v += __shfl_xor(v, 4);
      if ((tid & 7) == 0) rstd_s[srow + 32 * i] = 1.0f / sqrtf(v / (float)K + eps);
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int gn = n0 + wn * 64 + j * 32 + (lane & 31);
    if (gn >= N) continue;
    const float bv = HAS_B ? to_f(bias[gn]) : 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int gm = m0 + row;
        if (gm < M) {
          const float rs = NORM ? rstd_s[row] : 1.0f;
          out[(int64_t)gm * N + gn] = from_f<T>(scale * __builtin_fmaf(rs, acc[i][j][r], bv));
        }
      }
    }
  }
}

template <typename T, bool NORM>
hipError_t launch_t(const void* x, const void* w, const void* Wt, const void* b, void* out,
                    int M, int N, int K, float eps, float scale, hipStream_t s) {
  const dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
  const T* xp = static_cast<const T*>(x);
  const T* wp = static_cast<const T*>(w);
  const T* Wp = static_cast<const T*>(Wt);
  const T* bp = static_cast<const T*>(b);
  T* op = static_cast<T*>(out);
#define NP_RL(HW, HB)                                                                          \
  hipLaunchKernelGGL((rms_linear_mfma<T, NORM, HW, HB>), grid, dim3(NTHR), 0, s, xp, wp, Wp, bp, \
                     op, M, N, K, eps, scale)
  if (w && b) NP_RL(true, true);
  else if (w) NP_RL(true, false);
  else if (b) NP_RL(false, true);
  else NP_RL(false, false);
#undef NP_RL
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm_linear(const void* x, const void* w, const void* Wt, const void* b,
                                 void* out, int M, int N, int K, float eps, float scale, int dt,
                                 bool norm, hipStream_t s) {
  if (dt == NP_BF16)
    return norm ? launch_t<__bf16, true>(x, w, Wt, b, out, M, N, K, eps, scale, s)
                : launch_t<__bf16, false>(x, nullptr, Wt, b, out, M, N, K, eps, scale, s);
  if (dt == NP_F16)
    return norm ? launch_t<_Float16, true>(x, w, Wt, b, out, M, N, K, eps, scale, s)
                : launch_t<_Float16, false>(x, nullptr, Wt, b, out, M, N, K, eps, scale, s);
  return hipErrorInvalidValue;
}

}  // namespace np
