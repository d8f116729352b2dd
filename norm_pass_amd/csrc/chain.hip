// Fused elementwise chain: one kernel, one read of every input, one write.
//
// DeepJIT write-up (hotelren.com/news/5350627), sections 4.1 and 4.2: an
// elementwise chain welded into one kernel, then the 16-byte vector form with a
// scalar tail. Here the op list travels in the kernel arguments (a generic
// interpreter: the op kind is wave-uniform, so each op is one scalar branch
// followed by straight-line vector work on the thread's elements), every
// thread handles U groups of G elements with dwordx4 loads and stores, and the
// running value stays in fp32 registers; it is rounded only at cast ops and at
// the final store.
#include <type_traits>

#include "device.h"
#include "internal.h"

namespace np {
namespace {

constexpr int kBlock = 256;
constexpr int64_t kMinVecGroups = 65536;

__device__ __forceinline__ float relu_f(float v) { return v > 0.0f ? v : 0.0f; }

// Apply a unary op of the chain to one value.
template <bool FAST>
__device__ __forceinline__ float unary(int kind, float c, float v) {
  switch (kind) {
    case NP_ADD_C: return v + c;
    case NP_MUL_C:
    case NP_SCALE: return v * c;
    case NP_RELU: return relu_f(v);
    case NP_SIGMOID: return chain_sigmoid<FAST>(v);
    case NP_EXP: return chain_exp<FAST>(v);
    case NP_TANH: return chain_tanh<FAST>(v);
    case NP_CAST_F16: return round_via<_Float16>(v);
    case NP_CAST_BF16: return round_via<__bf16>(v);
    default: return v;
  }
}

template <typename T, int G>
__device__ __forceinline__ void load_group(const T* p, float (&v)[G]) {
  constexpr int N = Vec<T>::N;
  static_assert(G % N == 0, "group must be whole 16-byte vectors");
#pragma unroll
  for (int j = 0; j < G / N; ++j) {
    float t[N];
    load_vec<T>(p + j * N, t);
#pragma unroll
    for (int i = 0; i < N; ++i) v[j * N + i] = t[i];
  }
}

template <typename T, int G>
__device__ __forceinline__ void store_group(T* p, const float (&v)[G]) {
  constexpr int N = Vec<T>::N;
  static_assert(G % N == 0, "group must be whole 16-byte vectors");
#pragma unroll
  for (int j = 0; j < G / N; ++j) {
    float t[N];
#pragma unroll
    for (int i = 0; i < N; ++i) t[i] = v[j * N + i];
    store_vec_nt<T>(p + j * N, t);
  }
}

// Run the op list over a block of values (K values per input).
template <bool FAST, int NIN, int K>
__device__ __forceinline__ void run_ops(const ChainArgs& a, const float (&x)[NIN][K],
                                        float (&v)[K]) {
  for (int o = 0; o < a.n_ops; ++o) {
    const int kind = a.kind[o];
    const int arg = a.arg[o];
    const float c = a.c[o];
    if (kind == NP_LOAD || kind == NP_ADD_IN || kind == NP_MUL_IN) {
#pragma unroll
      for (int j = 0; j < NIN; ++j) {
        if (j == arg) {
#pragma unroll
          for (int e = 0; e < K; ++e) {
            v[e] = kind == NP_LOAD ? x[j][e] : kind == NP_ADD_IN ? v[e] + x[j][e] : v[e] * x[j][e];
          }
        }
      }
    } else {
      switch (kind) {
#define NP_CASE(KIND)                                          \
  case KIND:                                                   \
    _Pragma("unroll") for (int e = 0; e < K; ++e) v[e] = unary<FAST>(KIND, c, v[e]); \
    break;
        NP_CASE(NP_ADD_C)
        NP_CASE(NP_MUL_C)
        NP_CASE(NP_SCALE)
        NP_CASE(NP_RELU)
        NP_CASE(NP_SIGMOID)
        NP_CASE(NP_EXP)
        NP_CASE(NP_TANH)
        NP_CASE(NP_CAST_F16)
        NP_CASE(NP_CAST_BF16)
#undef NP_CASE
        default: break;
      }
    }
  }
}

template <typename Tout>
constexpr bool fast_math_for() {
  return std::is_same_v<Tout, _Float16>;  // fp16 output
}

// Vector kernel: thread handles U groups of G elements; the < G leftover
// elements at the end are handled one per thread by the first threads.
template <typename Tin, typename Tout, int NIN, int U, int G>
__global__ __launch_bounds__(kBlock) void chain_vec(ChainArgs a) {
  constexpr bool FAST = fast_math_for<Tout>();
  const int64_t ngroups = a.n / G;
  const int64_t base = (int64_t)blockIdx.x * kBlock * U + threadIdx.x;
  float x[NIN][U * G];
  float v[U * G];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t g = base + (int64_t)u * kBlock;
    if (g < ngroups) {
#pragma unroll
      for (int j = 0; j < NIN; ++j) {
        float t[G];
        load_group<Tin, G>(static_cast<const Tin*>(a.in[j]) + g * G, t);
#pragma unroll
        for (int e = 0; e < G; ++e) x[j][u * G + e] = t[e];
      }
    } else {
#pragma unroll
      for (int j = 0; j < NIN; ++j)
#pragma unroll
        for (int e = 0; e < G; ++e) x[j][u * G + e] = 0.0f;
    }
  }
  run_ops<FAST, NIN, U * G>(a, x, v);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t g = base + (int64_t)u * kBlock;
    if (g < ngroups) {
      float t[G];
#pragma unroll
      for (int e = 0; e < G; ++e) t[e] = v[u * G + e];
      store_group<Tout, G>(static_cast<Tout*>(a.out) + g * G, t);
    }
  }
  // scalar tail
  const int64_t tail0 = ngroups * G;
  const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (gid < a.n - tail0) {
    const int64_t i = tail0 + gid;
    float xs[NIN][1];
    float vs[1];
#pragma unroll
    for (int j = 0; j < NIN; ++j) xs[j][0] = to_f(static_cast<const Tin*>(a.in[j])[i]);
    run_ops<FAST, NIN, 1>(a, xs, vs);
    static_cast<Tout*>(a.out)[i] = from_f<Tout>(vs[0]);
  }
}

// Scalar kernel (any alignment): one element per thread.
template <typename Tin, typename Tout, int NIN>
__global__ __launch_bounds__(kBlock) void chain_scalar(ChainArgs a) {
  constexpr bool FAST = fast_math_for<Tout>();
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i >= a.n) return;
  float xs[NIN][1];
  float vs[1];
#pragma unroll
  for (int j = 0; j < NIN; ++j) xs[j][0] = to_f(static_cast<const Tin*>(a.in[j])[i]);
  run_ops<FAST, NIN, 1>(a, xs, vs);
  static_cast<Tout*>(a.out)[i] = from_f<Tout>(vs[0]);
}

template <typename Tin, typename Tout, int NIN>
hipError_t launch_typed(const ChainArgs& a, bool vec, hipStream_t s) {
  constexpr int G = (sizeof(Tin) == 2 || sizeof(Tout) == 2) ? 8 : 4;
  // below 64 Ki vector groups the chip is better filled by one element per thread
  if (vec && a.n / G >= kMinVecGroups) {
    constexpr int U = 1;
    const int64_t ngroups = a.n / G;
    int64_t blocks = (ngroups + (int64_t)kBlock * U - 1) / ((int64_t)kBlock * U);
    if (blocks < 1) blocks = 1;  // the tail still needs threads
    hipLaunchKernelGGL((chain_vec<Tin, Tout, NIN, U, G>), dim3((unsigned)blocks), dim3(kBlock), 0,
                       s, a);
  } else {
    const int64_t blocks = (a.n + kBlock - 1) / kBlock;
    hipLaunchKernelGGL((chain_scalar<Tin, Tout, NIN>), dim3((unsigned)blocks), dim3(kBlock), 0, s,
                       a);
  }
  return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t launch_nin(const ChainArgs& a, int n_inputs, bool vec, hipStream_t s) {
  switch (n_inputs) {
    case 1: return launch_typed<Tin, Tout, 1>(a, vec, s);
    case 2: return launch_typed<Tin, Tout, 2>(a, vec, s);
    case 3: return launch_typed<Tin, Tout, 3>(a, vec, s);
    default: return launch_typed<Tin, Tout, 4>(a, vec, s);
  }
}

template <typename Tin>
hipError_t launch_out(const ChainArgs& a, int out_dt, int n_inputs, bool vec, hipStream_t s) {
  switch (out_dt) {
    case NP_F32: return launch_nin<Tin, float>(a, n_inputs, vec, s);
    case NP_F16: return launch_nin<Tin, _Float16>(a, n_inputs, vec, s);
    default: return launch_nin<Tin, __bf16>(a, n_inputs, vec, s);
  }
}

}  // namespace

hipError_t launch_chain(const ChainArgs& a, int in_dt, int out_dt, int n_inputs, bool vec,
                        hipStream_t s) {
  switch (in_dt) {
    case NP_F32: return launch_out<float>(a, out_dt, n_inputs, vec, s);
    case NP_F16: return launch_out<_Float16>(a, out_dt, n_inputs, vec, s);
    default: return launch_out<__bf16>(a, out_dt, n_inputs, vec, s);
  }
}

}  // namespace np
