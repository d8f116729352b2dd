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
// Tiles: 256 x 256 outputs per 512-thread workgroup (one per CU: the two LDS
// stages take 144 KiB of gfx950's 160 KiB; two waves per SIMD, so one wave's
// MFMAs run while the other waits on LDS or stages data), K in steps of 64 (a
// partial last step reads zeros); each wave owns 128 x 64 outputs as 4 x 2
// blocks of v_mfma_f32_32x32x16 (bf16 or f16 inputs, fp32 accumulation).
// Operand layout of that instruction: lane l supplies A[l % 32][8 (l / 32) ..
// + 8] and B[8 (l / 32) .. + 8][l % 32] (16 contiguous bytes of a K-contiguous
// row each); accumulator register j of lane l is C[8 (j / 4) + 4 (l / 32) +
// j % 4][l % 32]. The loads of K step s + 2 are issued before the MFMAs of
// step s, so they are in flight while the matrix cores run; the epilogue
// rounds the tile into LDS and writes 16-byte rows.
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

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int PITCH = BK + 8;  // elements: 144-byte LDS rows keep 8 lanes' 16-byte reads in distinct banks
constexpr int NTHR = 512;      // 8 waves (2 per SIMD), each 128 x 64 outputs = 4 x 2 MFMA blocks
constexpr int WN = 4;          // waves along N (2 along M)
constexpr int FM = 4, FN = 2;  // 32 x 32 MFMA blocks per wave along M and N
constexpr int SV = BM * BK / 8 / NTHR;  // 16-byte staging vectors per thread and operand
constexpr int SROWS = NTHR / 8;         // rows staged per pass
constexpr int STAGE = (BM + BN) * PITCH;  // elements per LDS stage (A then B)
constexpr int CPITCH = BN + 8;            // elements per row of the epilogue's output tile
constexpr int SMEM = 2 * STAGE * 2;       // bytes: two stages (147,456); the output tile reuses them
static_assert(BM * CPITCH * 2 <= SMEM, "epilogue tile must fit in the stage buffers");
static_assert(2 * 32 * FM == BM && WN * 32 * FN == BN && SV * SROWS == BM, "tile / wave layout");
constexpr int GROUP_M = 4;  // tiles of 4 row blocks x all column blocks are taken together

// Workgroups are dispatched round robin to the 8 XCDs (each with its own L2):
// give XCD x a contiguous run of tiles so that the workgroups sharing an L2 also
// share A and B panels.
__device__ __forceinline__ int xcd_tile(int bid, int nb) {
  const int x = bid & 7, j = bid >> 3;
  const int per = nb >> 3, rem = nb & 7;
  return x * per + min(x, rem) + j;
}

// NORM: accumulate sum of squares and scale by rstd (fused form); otherwise a
// plain GEMM with bias (the unfused form's linear layer). HAS_W: multiply the
// A operand by the norm weight on its way to LDS.
template <typename T, bool NORM, bool HAS_W, bool HAS_B>
__global__ __launch_bounds__(NTHR) void rms_linear_mfma(const T* __restrict__ x,
                                                           const T* __restrict__ w,
                                                           const T* __restrict__ Wt,
                                                           const T* __restrict__ bias,
                                                           T* __restrict__ out, int M, int N,
                                                           int K, float eps, float scale,
                                                           int tiles_m, int tiles_n, int vec_out) {
  typedef typename Mfma<T>::v8 v8;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  __shared__ float rstd_s[BM];
  T* const lds = reinterpret_cast<T*>(smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  // output tile of this workgroup
  const int t = xcd_tile(blockIdx.x, tiles_m * tiles_n);
  const int per_group = GROUP_M * tiles_n;
  const int g = t / per_group, within = t - g * per_group;
  const int gsz = min(GROUP_M, tiles_m - g * GROUP_M);
  const int m0 = (g * GROUP_M + within % gsz) * BM, n0 = (within / gsz) * BN;
  // staging map: vector i of this thread is row srow + SROWS i, k chunk kc
  const int srow = tid >> 3, kc = (tid & 7) * 8;
  unsigned mval = 0, nval = 0;  // bit i: row srow + SROWS i is inside M / N
#pragma unroll
  for (int i = 0; i < SV; ++i) {
    mval |= (unsigned)(m0 + srow + SROWS * i < M) << i;
    nval |= (unsigned)(n0 + srow + SROWS * i < N) << i;
  }
  u32x4 xa[SV], xb[SV], wa = {0u, 0u, 0u, 0u};
  auto load_step = [&](int k0) {
    const int gk = k0 + kc;
    const bool kval = gk < K;  // K % 8 == 0: a vector is wholly inside or outside
    const int lk = kval ? gk : 0;
    // every load is issued unconditionally from a clamped (in-bounds) address
    // and masked afterwards: a branch around a load would serialise them
#pragma unroll
    for (int i = 0; i < SV; ++i) {
      const int gm = min(m0 + srow + SROWS * i, M - 1), gn = min(n0 + srow + SROWS * i, N - 1);
      xa[i] = load_raw(x + (int64_t)gm * K + lk);
      xb[i] = load_raw(Wt + (int64_t)gn * K + lk);
    }
#pragma unroll
    for (int i = 0; i < SV; ++i) {
      xa[i] &= (uint32_t)(-(int32_t)(kval && ((mval >> i) & 1)));
      xb[i] &= (uint32_t)(-(int32_t)(kval && ((nval >> i) & 1)));
    }
    if (HAS_W) wa = load_raw(w + lk);
  };
  float ss[SV];
#pragma unroll
  for (int i = 0; i < SV; ++i) ss[i] = 0.0f;
  auto store_step = [&](int buf) {
    T* As = lds + buf * STAGE;
    T* Bs = As + BM * PITCH;
    T wv[8];
    if (HAS_W) __builtin_memcpy(wv, &wa, 16);
#pragma unroll
    for (int i = 0; i < SV; ++i) {
      u32x4 av = xa[i];
      if (NORM || HAS_W) {
        T e[8];
        __builtin_memcpy(e, &xa[i], 16);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float f = to_f(e[j]);
          if (NORM) ss[i] = __builtin_fmaf(f, f, ss[i]);
          if (HAS_W) e[j] = from_f<T>(f * to_f(wv[j]));  // exact product, one rounding to T
        }
        if (HAS_W) __builtin_memcpy(&av, e, 16);
      }
      *reinterpret_cast<u32x4*>(&As[(srow + SROWS * i) * PITCH + kc]) = av;
      *reinterpret_cast<u32x4*>(&Bs[(srow + SROWS * i) * PITCH + kc]) = xb[i];
    }
  };
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  const int arow = wm * 32 * FM + (lane & 31), brw = wn * 32 * FN + (lane & 31);
  const int kl = (lane >> 5) * 8;
  auto compute = [&](int buf) {
    const T* As = lds + buf * STAGE;
    const T* Bs = As + BM * PITCH;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      v8 a[FM], b[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const u32x4 ra = *reinterpret_cast<const u32x4*>(&As[(arow + 32 * i) * PITCH + ks * 16 + kl]);
        __builtin_memcpy(&a[i], &ra, 16);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const u32x4 rb = *reinterpret_cast<const u32x4*>(&Bs[(brw + 32 * j) * PITCH + ks * 16 + kl]);
        __builtin_memcpy(&b[j], &rb, 16);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = Mfma<T>::run(a[i], b[j], acc[i][j]);
    }
  };

  // two LDS stages: step s computes from stage s & 1 while the loads of step
  // s + 1 (issued a step earlier) land in registers and then in the other stage
  // Step s: stage the registers of step s + 1 into the free LDS stage, issue
  // the global loads of step s + 2 into the same registers, then run step s's
  // MFMAs, so the loads have a whole step of MFMAs to land. The loop body has
  // no branch, so the compiler can interleave the staging with the
  // asynchronous MFMAs; loads past the end of K read clamped addresses and
  // are masked to zero.
  const int ksteps = (K + BK - 1) / BK;
  load_step(0);
  store_step(0);
  load_step(BK);
  __syncthreads();
  for (int s = 0; s + 1 < ksteps; ++s) {
    store_step((s + 1) & 1);
    load_step((s + 2) * BK);
    compute(s & 1);
    __syncthreads();
  }
  compute((ksteps - 1) & 1);
  __syncthreads();
  // rstd per row: the 8 lanes that staged a row hold its partial sums
  if (NORM) {
#pragma unroll
    for (int i = 0; i < SV; ++i) {
      float v = ss[i];
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      v += __shfl_xor(v, 4);
      if ((tid & 7) == 0) rstd_s[srow + SROWS * i] = 1.0f / sqrtf(v / (float)K + eps);
    }
    __syncthreads();
  }
  // epilogue: rstd, bias, scale in fp32, rounded to T into an LDS tile, then
  // written out as 16-byte rows
  T* const cs = lds;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int col = wn * 32 * FN + j * 32 + (lane & 31);
    const float bv = (HAS_B && n0 + col < N) ? to_f(bias[n0 + col]) : 0.0f;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 32 * FM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const float rs = NORM ? rstd_s[row] : 1.0f;
        cs[row * CPITCH + col] = from_f<T>(scale * __builtin_fmaf(rs, acc[i][j][r], bv));
      }
    }
  }
  __syncthreads();
#pragma unroll 4
  for (int i = 0; i < BM * BN / 8 / NTHR; ++i) {
    const int v = tid + NTHR * i;
    const int row = v >> 5, cv = (v & 31) * 8;
    const int gm = m0 + row, gn = n0 + cv;
    if (gm >= M) continue;
    T* dst = out + (int64_t)gm * N + gn;
    if (vec_out && gn + 8 <= N) {
      store_raw_nt(dst, *reinterpret_cast<const u32x4*>(&cs[row * CPITCH + cv]));
    } else {
      for (int e = 0; e < 8 && gn + e < N; ++e) dst[e] = cs[row * CPITCH + cv + e];
    }
  }
}

template <typename T, bool NORM>
hipError_t launch_t(const void* x, const void* w, const void* Wt, const void* b, void* out,
                    int M, int N, int K, float eps, float scale, hipStream_t s) {
  const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
  const dim3 grid(tm * tn);
  const int vec_out = (N % 8 == 0 && ((uintptr_t)out & 15) == 0) ? 1 : 0;
  const T* xp = static_cast<const T*>(x);
  const T* wp = static_cast<const T*>(w);
  const T* Wp = static_cast<const T*>(Wt);
  const T* bp = static_cast<const T*>(b);
  T* op = static_cast<T*>(out);
#define NP_RL(HW, HB)                                                                          \
  hipLaunchKernelGGL((rms_linear_mfma<T, NORM, HW, HB>), grid, dim3(NTHR), 0, s, xp, wp, Wp, bp, \
                     op, M, N, K, eps, scale, tm, tn, vec_out)
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
