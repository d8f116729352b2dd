// Single-operator kernels for the N-launch baseline: each launch reads its
// operands from HBM and stores its result in the storage type, the way a chain
// of framework operators runs (DeepJIT write-up, hotelren.com/news/5350627,
// section 1.1: every small kernel reads the tensor and writes it back; NaiveRT
// write-up, zhaixingw.cn/coding/291.html: K calls each paying the launch cost).
// They are written with the same care as the fused kernels (16-byte accesses
// where the layout allows, fp32 math), so the comparison isolates what fusion
// removes: launches and intermediate round trips.
#include "device.h"
#include "internal.h"

namespace np {
namespace {

constexpr int kBlock = 256;

__device__ __forceinline__ float unary_op(int kind, float c, float v) {
  switch (kind) {
    case NP_ADD_C: return v + c;
    case NP_MUL_C:
    case NP_SCALE: return v * c;
    case NP_RELU: return v > 0.0f ? v : 0.0f;
    case NP_SIGMOID: return sigmoid_f(v);
    case NP_EXP: return expf(v);
    case NP_TANH: return tanhf(v);
    case NP_CAST_F16: return round_via<_Float16>(v);
    case NP_CAST_BF16: return round_via<__bf16>(v);
    case U_SQUARE: return v * v;
    case U_RSQRT_EPS: return 1.0f / sqrtf(v + c);
    default: return v;  // U_COPY
  }
}

__device__ __forceinline__ float binary_op(int kind, float a, float b) {
  return kind == NP_MUL_IN ? a * b : a + b;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

template <typename T>
__global__ __launch_bounds__(kBlock) void unary_kernel(int kind, float c, const T* in, T* out,
                                                       int64_t n, bool vec) {
  constexpr int N = Vec<T>::N;
  const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (vec) {
    const int64_t nv = n / N;
    if (gid < nv) {
      float v[N];
      load_vec<T>(in + gid * N, v);
#pragma unroll
      for (int e = 0; e < N; ++e) v[e] = unary_op(kind, c, v[e]);
      store_vec_nt<T>(out + gid * N, v);
    }
    const int64_t i = nv * N + gid;
    if (gid < n - nv * N) out[i] = from_f<T>(unary_op(kind, c, to_f(in[i])));
  } else if (gid < n) {
    out[gid] = from_f<T>(unary_op(kind, c, to_f(in[gid])));
  }
}

template <typename T>
__global__ __launch_bounds__(kBlock) void binary_kernel(int kind, const T* a, const T* b, T* out,
                                                        int64_t n, bool vec) {
  constexpr int N = Vec<T>::N;
  const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (vec) {
    const int64_t nv = n / N;
    if (gid < nv) {
      float va[N], vb[N];
      load_vec<T>(a + gid * N, va);
      load_vec<T>(b + gid * N, vb);
#pragma unroll
      for (int e = 0; e < N; ++e) va[e] = binary_op(kind, va[e], vb[e]);
      store_vec_nt<T>(out + gid * N, va);
    }
    const int64_t i = nv * N + gid;
    if (gid < n - nv * N) out[i] = from_f<T>(binary_op(kind, to_f(a[i]), to_f(b[i])));
  } else if (gid < n) {
    out[gid] = from_f<T>(binary_op(kind, to_f(a[gid]), to_f(b[gid])));
  }
}

int64_t blocks_for(int64_t work) {
  int64_t b = (work + kBlock - 1) / kBlock;
  return b < 1 ? 1 : b;
}

// row mean of [rows, cols] -> [rows], fp32 accumulation, one block per row
template <typename T>
__global__ __launch_bounds__(kBlock) void row_mean_kernel(const T* in, T* out, int cols) {
  __shared__ float part[4];
  const int64_t off = (int64_t)blockIdx.x * cols;
  float s = 0.0f;
  for (int j = threadIdx.x; j < cols; j += kBlock) s += to_f(in[off + j]);
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float tot = (part[0] + part[1]) + (part[2] + part[3]);
    out[blockIdx.x] = from_f<T>(tot / (float)cols);
  }
}

// out[i, j] = in[i, j] (op) s[i]  (ROW = true)   or   in[i, j] (op) s[j]  (ROW = false),
// op = multiply / add / subtract
enum BcastOp { B_MUL = 0, B_ADD = 1, B_SUB = 2 };

template <int OP>
__device__ __forceinline__ float bop(float a, float b) {
  return OP == B_MUL ? a * b : OP == B_ADD ? a + b : a - b;
}

template <typename T, bool ROW, int OP>
__global__ __launch_bounds__(kBlock) void bcast_kernel(const T* in, const T* s, T* out,
                                                       int64_t rows, int64_t cols, bool vec) {
  constexpr int N = Vec<T>::N;
  const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (vec) {  // cols % N == 0
    const int64_t nv = rows * cols / N;
    if (gid >= nv) return;
    const int64_t e0 = gid * N;
    const int64_t i = e0 / cols;
    const int64_t j = e0 - i * cols;
    float v[N];
    load_vec<T>(in + e0, v);
    if (ROW) {
      const float f = to_f(s[i]);
#pragma unroll
      for (int e = 0; e < N; ++e) v[e] = bop<OP>(v[e], f);
    } else {
      float w[N];
      load_vec<T>(s + j, w);
#pragma unroll
      for (int e = 0; e < N; ++e) v[e] = bop<OP>(v[e], w[e]);
    }
    store_vec_nt<T>(out + e0, v);
  } else {
    if (gid >= rows * cols) return;
    const int64_t i = gid / cols;
    const int64_t j = gid - i * cols;
    out[gid] = from_f<T>(bop<OP>(to_f(in[gid]), to_f(s[ROW ? i : j])));
  }
}

// qkv [T, 3, H, D] -> q, k, v [H, T, D]; one thread per 16-byte chunk
template <typename T>
__global__ __launch_bounds__(kBlock) void qkv_split_kernel(const T* qkv, T* q, T* k, T* v,
                                                           int64_t T_, int H, int D, bool vec) {
  const int N = vec ? Vec<T>::N : 1;
  const int cpr = D / N;  // chunks per head vector
  const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int64_t total = T_ * 3 * H * cpr;
  if (gid >= total) return;
  const int c = (int)(gid % cpr);
  int64_t rest = gid / cpr;
  const int h = (int)(rest % H);
  rest /= H;
  const int s = (int)(rest % 3);
  const int64_t t = rest / 3;
  const T* src = qkv + ((t * 3 + s) * H + h) * (int64_t)D + c * N;
  T* dst = (s == 0 ? q : s == 1 ? k : v) + ((int64_t)h * T_ + t) * D + c * N;
  if (vec)
    store_raw_nt(dst, load_raw(src));
  else
    *dst = *src;
}

// in-place RoPE on a head-major [H, T, D] tensor: thread = (token, chunk),
// angles computed once per thread and reused over the H heads
template <typename T, bool VEC>
__global__ __launch_bounds__(kBlock) void rope_inplace_kernel(T* x, int64_t T_, int H, int D,
                                                              const int32_t* pos, RopeArgs inv) {
  const int half = D / 2;
  constexpr int E = VEC ? Vec<T>::N : 1;
  const int P = half / E;
  const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (gid >= T_ * P) return;
  const int64_t t = gid / P;
  const int j = (int)(gid % P);
  // fp64 rotation for fp32 data (rope_math_t): one rounding of the rotated value
  using RT = rope_math_t<T>;
  const float p = pos ? (float)pos[t] : (float)t;
  constexpr int EM = Vec<T>::N;
  RT cs[E], sn[E];
#pragma unroll
  for (int e = 0; e < E; ++e) rope_sincos(p * inv.inv[j * E + e], &sn[e], &cs[e]);
  for (int h = 0; h < H; ++h) {
    T* row = x + ((int64_t)h * T_ + t) * D;
    if constexpr (VEC) {
      float u[EM], w[EM];
      load_vec<T>(row + j * E, u);
      load_vec<T>(row + half + j * E, w);
      float o1[EM], o2[EM];
#pragma unroll
      for (int e = 0; e < EM; ++e) {
        const RT ue = u[e], we = w[e];
        o1[e] = (float)(ue * cs[e] - we * sn[e]);
        o2[e] = (float)(we * cs[e] + ue * sn[e]);
      }
      store_vec_nt<T>(row + j * E, o1);
      store_vec_nt<T>(row + half + j * E, o2);
    } else {
      const RT u = to_f(row[j]);
      const RT w = to_f(row[half + j]);
      row[j] = from_f<T>((float)(u * cs[0] - w * sn[0]));
      row[half + j] = from_f<T>((float)(w * cs[0] + u * sn[0]));
    }
  }
}

// NCHW level [b, A*C, H, W] -> rows [b, A, H*W, C]; thread per output element
template <typename T>
__global__ __launch_bounds__(kBlock) void det_permute_kernel(const T* in, T* out, int batch, int A,
                                                             int C, int HW) {
  const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int64_t total = (int64_t)batch * A * HW * C;
  if (gid >= total) return;
  const int k = (int)(gid % C);
  int64_t rest = gid / C;
  const int cell = (int)(rest % HW);
  rest /= HW;  // = b * A + a
  out[gid] = in[(rest * C + k) * HW + cell];
}

// in-place op on channels [k0, k1) of rows [b, A, H*W, C]
struct AnchorTable {
  float wh[16 * 2];  // anchors of this level: (w, h) per anchor
};
template <typename T>
__global__ __launch_bounds__(kBlock) void det_range_kernel(T* rows, int batch, int A, int C,
                                                           int H, int W, int k0, int k1, int op,
                                                           float c, AnchorTable an) {
  const int nk = k1 - k0;
  const int64_t HW = (int64_t)H * W;
  const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int64_t total = (int64_t)batch * A * HW * nk;
  if (gid >= total) return;
  const int k = k0 + (int)(gid % nk);
  const int64_t row = gid / nk;
  const int64_t idx = row * C + k;
  float v = to_f(rows[idx]);
  switch (op) {
    case D_SIGMOID: v = sigmoid_f(v); break;
    case D_EXP: v = expf(v); break;
    case D_MUL_ANCHOR: {
      const int a = (int)((row / HW) % A);
      v *= an.wh[a * 2 + (k - 2)];
      break;
    }
    case D_ADD_GRID: {
      const int cell = (int)(row % HW);
      v += (float)(k == 0 ? cell % W : cell / W);
      break;
    }
    default: v *= c; break;
  }
  rows[idx] = from_f<T>(v);
}

// concat levels [b, R_l, C] -> [b, sum R_l, C]; thread per output element
struct ConcatArgs {
  const void* part[8];
  int64_t rows[8];
  int64_t start[9];
  int n;
};
template <typename T>
__global__ __launch_bounds__(kBlock) void det_concat_kernel(ConcatArgs a, T* out, int batch,
                                                            int64_t total_rows, int C) {
  const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (gid >= (int64_t)batch * total_rows * C) return;
  const int k = (int)(gid % C);
  const int64_t r = (gid / C) % total_rows;
  const int64_t b = gid / (C * total_rows);
  int l = 0;
  while (l + 1 < a.n && r >= a.start[l + 1]) ++l;
  const T* src = static_cast<const T*>(a.part[l]);
  out[gid] = src[(b * a.rows[l] + (r - a.start[l])) * C + k];
}

template <typename T>
__global__ __launch_bounds__(kBlock) void cast_f32_kernel(const T* in, float* out, int64_t n) {
  const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (gid < n) out[gid] = to_f(in[gid]);
}

__global__ void empty_kernel() {}

template <typename F>
hipError_t by_dt(int dt, F&& f) {
  switch (dt) {
    case NP_F32: return f(float{});
    case NP_F16: return f(_Float16{});
    default: return f(__bf16{});
  }
}

}  // namespace

hipError_t launch_unary(int kind, float c, const void* in, void* out, int64_t n, int dt,
                        hipStream_t s) {
  return by_dt(dt, [&](auto tag) {
    using T = decltype(tag);
    const bool vec = aligned16(in) && aligned16(out);
    const int64_t work = vec ? n / Vec<T>::N : n;
    hipLaunchKernelGGL(unary_kernel<T>, dim3((unsigned)blocks_for(work)), dim3(kBlock), 0, s,
                       kind, c, static_cast<const T*>(in), static_cast<T*>(out), n, vec);
    return hipGetLastError();
  });
}

hipError_t launch_binary(int kind, const void* a, const void* b, void* out, int64_t n, int dt,
                         hipStream_t s) {
  return by_dt(dt, [&](auto tag) {
    using T = decltype(tag);
    const bool vec = aligned16(a) && aligned16(b) && aligned16(out);
    const int64_t work = vec ? n / Vec<T>::N : n;
    hipLaunchKernelGGL(binary_kernel<T>, dim3((unsigned)blocks_for(work)), dim3(kBlock), 0, s,
                       kind, static_cast<const T*>(a), static_cast<const T*>(b),
                       static_cast<T*>(out), n, vec);
    return hipGetLastError();
  });
}

hipError_t launch_row_mean(const void* in, void* out, int64_t rows, int64_t cols, int dt,
                           hipStream_t s) {
  return by_dt(dt, [&](auto tag) {
    using T = decltype(tag);
    hipLaunchKernelGGL(row_mean_kernel<T>, dim3((unsigned)rows), dim3(kBlock), 0, s,
                       static_cast<const T*>(in), static_cast<T*>(out), (int)cols);
    return hipGetLastError();
  });
}

template <bool ROW, int OP>
hipError_t bcast(const void* in, const void* sc, void* out, int64_t rows, int64_t cols, int dt,
                 hipStream_t s) {
  return by_dt(dt, [&](auto tag) {
    using T = decltype(tag);
    const bool vec = aligned16(in) && aligned16(out) && cols % Vec<T>::N == 0 &&
                     (ROW || aligned16(sc));
    const int64_t work = vec ? rows * cols / Vec<T>::N : rows * cols;
    hipLaunchKernelGGL((bcast_kernel<T, ROW, OP>), dim3((unsigned)blocks_for(work)),
                       dim3(kBlock), 0, s, static_cast<const T*>(in),
                       static_cast<const T*>(sc), static_cast<T*>(out), rows, cols, vec);
    return hipGetLastError();
  });
}

hipError_t launch_row_scale(const void* in, const void* rs, void* out, int64_t rows,
                            int64_t cols, int dt, hipStream_t s) {
  return bcast<true, B_MUL>(in, rs, out, rows, cols, dt, s);
}

hipError_t launch_col_scale(const void* in, const void* w, void* out, int64_t rows,
                            int64_t cols, int dt, hipStream_t s) {
  return bcast<false, B_MUL>(in, w, out, rows, cols, dt, s);
}

hipError_t launch_row_sub(const void* in, const void* m, void* out, int64_t rows, int64_t cols,
                          int dt, hipStream_t s) {
  return bcast<true, B_SUB>(in, m, out, rows, cols, dt, s);
}

hipError_t launch_col_add(const void* in, const void* b, void* out, int64_t rows, int64_t cols,
                          int dt, hipStream_t s) {
  return bcast<false, B_ADD>(in, b, out, rows, cols, dt, s);
}

hipError_t launch_qkv_split(const void* qkv, void* q, void* k, void* v, int64_t T_, int H, int D,
                            int dt, hipStream_t s) {
  return by_dt(dt, [&](auto tag) {
    using T = decltype(tag);
    const bool vec = aligned16(qkv) && aligned16(q) && aligned16(k) && aligned16(v) &&
                     D % Vec<T>::N == 0;
    const int64_t work = T_ * 3 * H * (int64_t)(vec ? D / Vec<T>::N : D);
    hipLaunchKernelGGL(qkv_split_kernel<T>, dim3((unsigned)blocks_for(work)), dim3(kBlock), 0, s,
                       static_cast<const T*>(qkv), static_cast<T*>(q), static_cast<T*>(k),
                       static_cast<T*>(v), T_, H, D, vec);
    return hipGetLastError();
  });
}

hipError_t launch_rope_inplace(void* x, int64_t T_, int H, int D, const int32_t* pos,
                               const float* inv, int dt, hipStream_t s) {
  RopeArgs table{};
  for (int i = 0; i < D / 2; ++i) table.inv[i] = inv[i];
  return by_dt(dt, [&](auto tag) {
    using T = decltype(tag);
    const bool vec = aligned16(x) && (D / 2) % Vec<T>::N == 0;
    const int64_t work = T_ * (int64_t)(vec ? D / 2 / Vec<T>::N : D / 2);
    if (vec)
      hipLaunchKernelGGL((rope_inplace_kernel<T, true>), dim3((unsigned)blocks_for(work)),
                         dim3(kBlock), 0, s, static_cast<T*>(x), T_, H, D, pos, table);
    else
      hipLaunchKernelGGL((rope_inplace_kernel<T, false>), dim3((unsigned)blocks_for(work)),
                         dim3(kBlock), 0, s, static_cast<T*>(x), T_, H, D, pos, table);
    return hipGetLastError();
  });
}

hipError_t launch_det_permute(const void* in, void* rows_out, int batch, int A, int C, int H,
                              int W, int dt, hipStream_t s) {
  return by_dt(dt, [&](auto tag) {
    using T = decltype(tag);
    const int64_t total = (int64_t)batch * A * C * H * W;
    hipLaunchKernelGGL(det_permute_kernel<T>, dim3((unsigned)blocks_for(total)), dim3(kBlock), 0,
                       s, static_cast<const T*>(in), static_cast<T*>(rows_out), batch, A, C,
                       H * W);
    return hipGetLastError();
  });
}

hipError_t launch_det_range_op(void* rows, int batch, int A, int C, int H, int W, int k0, int k1,
                               int op, float c, const float* anchors_a2, int dt, hipStream_t s) {
  AnchorTable an{};
  for (int i = 0; i < A * 2 && i < 32; ++i) an.wh[i] = anchors_a2[i];
  return by_dt(dt, [&](auto tag) {
    using T = decltype(tag);
    const int64_t total = (int64_t)batch * A * H * W * (k1 - k0);
    hipLaunchKernelGGL(det_range_kernel<T>, dim3((unsigned)blocks_for(total)), dim3(kBlock), 0, s,
                       static_cast<T*>(rows), batch, A, C, H, W, k0, k1, op, c, an);
    return hipGetLastError();
  });
}

hipError_t launch_det_concat(const void* const* parts, const int64_t* part_rows, int n_parts,
                             void* out, int batch, int64_t total_rows, int C, int dt,
                             hipStream_t s) {
  ConcatArgs a{};
  a.n = n_parts;
  a.start[0] = 0;
  for (int l = 0; l < n_parts; ++l) {
    a.part[l] = parts[l];
    a.rows[l] = part_rows[l];
    a.start[l + 1] = a.start[l] + part_rows[l];
  }
  return by_dt(dt, [&](auto tag) {
    using T = decltype(tag);
    const int64_t total = (int64_t)batch * total_rows * C;
    hipLaunchKernelGGL(det_concat_kernel<T>, dim3((unsigned)blocks_for(total)), dim3(kBlock), 0, s,
                       a, static_cast<T*>(out), batch, total_rows, C);
    return hipGetLastError();
  });
}

hipError_t launch_cast_to_f32(const void* in, float* out, int64_t n, int dt, hipStream_t s) {
  return by_dt(dt, [&](auto tag) {
    using T = decltype(tag);
    hipLaunchKernelGGL(cast_f32_kernel<T>, dim3((unsigned)blocks_for(n)), dim3(kBlock), 0, s,
                       static_cast<const T*>(in), out, n);
    return hipGetLastError();
  });
}

hipError_t launch_empty(hipStream_t s) {
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, s);
  return hipGetLastError();
}

}  // namespace np
