// C ABI of the fused-chain library: argument validation, dispatch to the
// kernels, error reporting. Validation is pure host code that runs before any
// HIP call, so a rejected call touches no device. Conventions follow the C-ABI
// operator contract of the page "CUDA算子与AI运行时" (gtnt.cn/news/145880),
// sections 4.1 and 4.3: raw pointers and sizes in, an int status out, the
// caller's stream, no synchronisation inside, no exceptions across the ABI.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>

#include "internal.h"
#include "rtc.h"

namespace {


thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return NP_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(NP_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
}

bool valid_dt(int dt) { return dt == NP_F32 || dt == NP_F16 || dt == NP_BF16; }

// A dispatch grid counts at most 2^32 work-items. The fused calls split long
// inputs into launches of at most these many elements or rows (each a
// multiple of 16 elements, so a 16-byte aligned buffer stays aligned at every
// launch's start); the unfused baselines, one thread per element, take at most
// kUnfusedMax elements per call.
constexpr int64_t kChainChunk = (int64_t)1 << 30;  // elements per chain launch
constexpr int64_t kRowChunk = (int64_t)1 << 22;    // rows per norm launch (<= 512 threads each)
constexpr int64_t kUnfusedMax = (int64_t)1 << 31;
constexpr int64_t kUnfusedRowMax = (int64_t)1 << 23;  // rows of 256-thread row reductions
bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Per-device gfx950 check, done once per device and cached.
std::mutex g_dev_mu;
int g_dev_state[64];  // 0 unknown, 1 gfx950, -1 rejected

int check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= 64) {
    return fail(NP_EDEVICE, "no HIP device available (%s)", hipGetErrorString(e));
  }
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_dev_state[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(NP_EDEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    g_dev_state[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    if (g_dev_state[dev] < 0)
      return fail(NP_EDEVICE, "device %d is %s, this library is built for gfx950", dev,
                  prop.gcnArchName);
  }
  if (g_dev_state[dev] < 0) return fail(NP_EDEVICE, "device %d is not gfx950", dev);
  return NP_OK;
}

int validate_chain(const np_op* ops, int n_ops, const void* const* inputs, int n_inputs,
                   int in_dt, const void* out, int out_dt, int64_t n) {
  if (!ops) return fail(NP_EINVAL, "ops is NULL");
  if (n_ops < 1 || n_ops > NP_MAX_OPS)
    return fail(NP_EINVAL, "n_ops = %d, must be 1..%d", n_ops, NP_MAX_OPS);
  if (n_inputs < 1 || n_inputs > NP_MAX_INPUTS)
    return fail(NP_EINVAL, "n_inputs = %d, must be 1..%d", n_inputs, NP_MAX_INPUTS);
  if (!valid_dt(in_dt) || !valid_dt(out_dt)) return fail(NP_EINVAL, "unknown dtype");
  if (n < 0) return fail(NP_EINVAL, "n = %lld < 0", (long long)n);
  if (n >= ((int64_t)1 << 40))  // beyond any device's memory; keeps grid sizes below 2^31
    return fail(NP_EINVAL, "n = %lld is not below 2^40", (long long)n);
  if (ops[0].kind != NP_LOAD) return fail(NP_EINVAL, "ops[0] must be NP_LOAD");
  for (int i = 0; i < n_ops; ++i) {
    const int k = ops[i].kind;
    if (k < NP_LOAD || k > NP_CAST_BF16) return fail(NP_EINVAL, "ops[%d]: unknown kind %d", i, k);
    if ((k == NP_LOAD || k == NP_ADD_IN || k == NP_MUL_IN) &&
        (ops[i].arg < 0 || ops[i].arg >= n_inputs))
      return fail(NP_EINVAL, "ops[%d]: input index %d out of range", i, ops[i].arg);
  }
  if (n == 0) return NP_OK;
  if (!inputs) return fail(NP_EINVAL, "inputs is NULL");
  for (int j = 0; j < n_inputs; ++j)
    if (!inputs[j]) return fail(NP_EINVAL, "inputs[%d] is NULL", j);
  if (!out) return fail(NP_EINVAL, "out is NULL");
  return NP_OK;
}

np::ChainArgs chain_args(const np_op* ops, int n_ops, const void* const* inputs, int n_inputs,
                         void* out, int64_t n) {
  np::ChainArgs a{};
  a.n_ops = n_ops;
  for (int i = 0; i < n_ops; ++i) {
    a.kind[i] = ops[i].kind;
    a.arg[i] = ops[i].arg;
    a.c[i] = ops[i].c;
  }
  for (int j = 0; j < n_inputs; ++j) a.in[j] = inputs[j];
  a.out = out;
  a.n = n;
  return a;
}

int validate_det(const void* const* lv, int n_levels, const int32_t* H, const int32_t* W,
                 const float* strides, const float* anchors, int n_anchors, int n_ch, int batch,
                 int in_dt, const float* out) {
  if (!lv || !H || !W || !strides || !anchors || !out) return fail(NP_EINVAL, "NULL argument");
  if (n_levels < 1 || n_levels > 8) return fail(NP_EINVAL, "n_levels = %d, must be 1..8", n_levels);
  if (n_anchors < 1 || n_anchors > 16)
    return fail(NP_EINVAL, "n_anchors = %d, must be 1..16", n_anchors);
  if (n_ch < 5 || n_ch > 1024) return fail(NP_EINVAL, "n_ch = %d, must be 5..1024", n_ch);
  if (batch < 1) return fail(NP_EINVAL, "batch = %d < 1", batch);
  if (!valid_dt(in_dt)) return fail(NP_EINVAL, "unknown dtype");
  int64_t rows = 0;
  for (int l = 0; l < n_levels; ++l) {
    if (!lv[l]) return fail(NP_EINVAL, "level_logits[%d] is NULL", l);
    if (H[l] < 1 || W[l] < 1 || (int64_t)H[l] * W[l] > (1 << 22))
      return fail(NP_EINVAL, "level %d: bad H x W = %d x %d", l, H[l], W[l]);
    if (!std::isfinite(strides[l])) return fail(NP_EINVAL, "level %d: stride not finite", l);
    rows += (int64_t)n_anchors * H[l] * W[l];
  }
  if ((int64_t)batch * rows * n_ch >= (int64_t)1 << 40) return fail(NP_EINVAL, "output too large");
  return NP_OK;
}

int validate_norm(const void* x, const void* out, const void* h, int64_t rows, int64_t cols,
                  float eps, int dt) {
  if (!x || !out) return fail(NP_EINVAL, "x or out is NULL");
  if (!valid_dt(dt)) return fail(NP_EINVAL, "unknown dtype");
  if (rows < 0 || rows >= ((int64_t)1 << 31)) return fail(NP_EINVAL, "rows = %lld out of range", (long long)rows);
  if (cols < 1 || cols > ((int64_t)1 << 24)) return fail(NP_EINVAL, "cols = %lld out of range", (long long)cols);
  if (!(eps > 0.0f) || !std::isfinite(eps)) return fail(NP_EINVAL, "eps must be finite and > 0");
  if (h && h == out) return fail(NP_EINVAL, "h_out and out must differ");
  return NP_OK;
}

int validate_rope(const void* qkv, const void* q, const void* k, const void* v, int64_t T,
                  int n_heads, int head_dim, float base, float q_scale, int dt) {
  if (!qkv || !q || !k || !v) return fail(NP_EINVAL, "NULL buffer");
  if (!valid_dt(dt)) return fail(NP_EINVAL, "unknown dtype");
  if (T < 0 || T >= ((int64_t)1 << 31)) return fail(NP_EINVAL, "T out of range");
  if (n_heads < 1 || n_heads > 4096) return fail(NP_EINVAL, "n_heads = %d out of range", n_heads);
  if (head_dim < 2 || head_dim > 512 || (head_dim & 1))
    return fail(NP_EINVAL, "head_dim = %d: must be even and <= 512", head_dim);
  if (!(base > 0.0f) || !std::isfinite(base)) return fail(NP_EINVAL, "base must be > 0");
  if (!std::isfinite(q_scale)) return fail(NP_EINVAL, "q_scale not finite");
  if (qkv == q || qkv == k || qkv == v || q == k || q == v || k == v)
    return fail(NP_EINVAL, "qkv, q, k, v must not alias");
  return NP_OK;
}

// fp32(base^(-2i/head_dim)), evaluated in double and rounded once
void inv_freq(float base, int head_dim, float* inv) {
  for (int i = 0; i < head_dim / 2; ++i)
    inv[i] = (float)std::pow((double)base, -2.0 * (double)i / (double)head_dim);
}

int fill_det_args(np::DetArgs& a, const void* const* lv, int n_levels, const int32_t* H,
                  const int32_t* W, const float* strides, const float* anchors, int n_anchors,
                  int n_ch, int batch, float* out) {
  a = np::DetArgs{};
  np::DetHeader& h = a.h;
  h.n_levels = n_levels;
  h.n_anchors = n_anchors;
  h.n_ch = n_ch;
  h.batch = batch;
  h.out = out;
  const int tp = np::det_tile_cells(n_ch);
  h.tile_cells = tp;
  int64_t row = 0;
  int64_t tiles_total = 0;
  h.tile_start[0] = 0;
  for (int l = 0; l < n_levels; ++l) {
    np::DetLevel& L = a.lv[l];
    L.in = lv[l];
    L.hw = H[l] * W[l];
    L.w = W[l];
    L.stride = strides[l];
    L.inv_w = 1.0f / (float)W[l];
    for (int j = 0; j < n_anchors * 2; ++j) L.anchor[j] = anchors[l * n_anchors * 2 + j];
    L.row_off = row;
    const int64_t hw = (int64_t)H[l] * W[l];
    row += n_anchors * hw;
    h.tiles[l] = (int32_t)((hw + tp - 1) / tp);
    tiles_total += (int64_t)batch * n_anchors * h.tiles[l];
    // one 256-thread workgroup per tile: fewer than 2^31 work-items per launch
    if (tiles_total >= ((int64_t)1 << 23))
      return fail(NP_EINVAL, "output too large for one launch (%lld tiles of %d cells, limit 2^23)",
                  (long long)tiles_total, tp);
    h.tile_start[l + 1] = (int32_t)tiles_total;
  }
  h.total_rows = row;
  return NP_OK;
}


// ---- layout: batched transpose [B, R, S, E] -> [B, S, R, E] ----------------

enum TrKernel { TR_TILE = 1, TR_SMALL = 2, TR_ITEMS = 3 };

struct TrPlan {
  int kernel = 0;
  int item = 1;      // bytes per load / store item
  bool vec = false;  // 16-byte vectors on both sides
  int64_t B = 0, R = 0, S = 0, Ei = 0;  // shape in items (Ei items per unit)
  int64_t per_chunk = 1;                 // matrices per block (TR_SMALL)
  bool diagonal = false;                 // diagonal tile order (TR_TILE)
};

int pow2_item(uint64_t v) {  // largest power of two <= 16 dividing v
  int w = 16;
  while (w > 1 && (v % (uint64_t)w) != 0) w >>= 1;
  return w;
}

int validate_transpose(const void* in, const void* out, int64_t B, int64_t R, int64_t S,
                       int64_t E, int elem_bytes, int64_t* total) {
  if (B < 0 || R < 0 || S < 0 || E < 0)
    return fail(NP_EINVAL, "negative size (B=%lld R=%lld S=%lld E=%lld)", (long long)B,
                (long long)R, (long long)S, (long long)E);
  if (elem_bytes < 1 || elem_bytes > 16)
    return fail(NP_EINVAL, "elem_bytes = %d, must be 1..16", elem_bytes);
  const int64_t lim = (int64_t)1 << 31;
  if (R >= lim || S >= lim || E >= lim || B >= ((int64_t)1 << 40))
    return fail(NP_EINVAL, "size out of range (R, S, E < 2^31, B < 2^40)");
  // total bytes <= 2^46 (64 TiB): checked one factor at a time
  long double t = (long double)B * R * S * E * elem_bytes;
  if (t > (long double)((int64_t)1 << 46)) return fail(NP_EINVAL, "tensor larger than 2^46 bytes");
  *total = B * R * S * E * elem_bytes;
  if (*total == 0) return NP_OK;
  if (!in || !out) return fail(NP_EINVAL, "NULL buffer");
  const uintptr_t a = (uintptr_t)in, b = (uintptr_t)out;
  if (a < b + (uint64_t)*total && b < a + (uint64_t)*total)
    return fail(NP_EINVAL, "in and out overlap (a transpose cannot run in place)");
  return NP_OK;
}

TrPlan plan_transpose(const void* in, const void* out, int64_t B, int64_t R, int64_t S, int64_t E,
                      int elem_bytes, bool naive) {
  TrPlan p;
  const uint64_t u = (uint64_t)E * elem_bytes;  // unit bytes
  const uint64_t addr = (uint64_t)(uintptr_t)in | (uint64_t)(uintptr_t)out;
  if (!naive && (R == 1 || S == 1)) {  // no axis to swap: a contiguous copy
    const uint64_t total = (uint64_t)B * R * S * u;
    p.item = pow2_item(total | addr);
    p.kernel = TR_ITEMS;
    p.B = (int64_t)(total / p.item);
    p.R = p.S = p.Ei = 1;
    return p;
  }
  p.item = pow2_item((naive ? (uint64_t)elem_bytes : u) | addr);
  p.B = B;
  p.R = R;
  p.S = S;
  p.Ei = (int64_t)(u / p.item);
  if (naive) {
    p.kernel = TR_ITEMS;
    return p;
  }
  const uint64_t mat = (uint64_t)R * S * u;
  if (mat <= np::kSmallChunkBytes) {
    p.kernel = TR_SMALL;
    const uint64_t k_max = np::kSmallChunkBytes / mat;
    uint64_t g = 16;
    while (g > 1 && (mat * (16 / g)) % 16 != 0) g >>= 1;  // g = gcd(mat, 16)
    const uint64_t step = 16 / g;                          // matrices per 16-byte multiple
    if (k_max >= step && (addr & 15) == 0) {
      p.per_chunk = (int64_t)(k_max / step * step);
      p.vec = true;
    } else {
      p.per_chunk = (int64_t)k_max;
    }
    return p;
  }
  if ((uint64_t)p.item == u) {
    p.kernel = TR_TILE;
    p.vec = (addr & 15) == 0 && (S * (int64_t)u) % 16 == 0 && (R * (int64_t)u) % 16 == 0;
    // A row pitch that is a power of two of >= 4 KiB maps the rows of one tile
    // column onto the same memory channels; the diagonal order spreads them.
    auto pow2_pitch = [](int64_t b) { return b >= 4096 && (b & (b - 1)) == 0; };
    p.diagonal = pow2_pitch(S * (int64_t)u) || pow2_pitch(R * (int64_t)u);
    return p;
  }
  p.kernel = TR_ITEMS;
  return p;
}

int run_transpose(const void* in, void* out, int64_t B, int64_t R, int64_t S, int64_t E,
                  int elem_bytes, bool naive, hipStream_t stream, const char* who) {
  int64_t total = 0;
  int rc = validate_transpose(in, out, B, R, S, E, elem_bytes, &total);
  if (rc) return rc;
  if (total == 0) return ok();
  const TrPlan p = plan_transpose(in, out, B, R, S, E, elem_bytes, naive);
  const int64_t lim = ((int64_t)1 << 31) - 1;
  const int64_t mat_items = p.R * p.S * p.Ei;
  if (p.kernel == TR_ITEMS && mat_items > lim)
    return fail(NP_EINVAL, "%s: one [R, S] matrix holds %lld items of %d bytes (limit 2^31 - 1)",
                who, (long long)mat_items, p.item);
  if ((rc = check_device())) return rc;
  const uint8_t* src = static_cast<const uint8_t*>(in);
  uint8_t* dst = static_cast<uint8_t*>(out);
  const int64_t mat_bytes = mat_items * p.item;
  hipError_t e = hipSuccess;
  if (p.kernel == TR_TILE) {
    const int64_t T = np::tile_side(p.item);
    const int64_t n_rt = (p.R + T - 1) / T, n_st = (p.S + T - 1) / T;
    const int64_t per_b = n_rt * n_st;
    if (per_b > lim) return fail(NP_EINVAL, "%s: too many tiles per matrix", who);
    np::TileArgs a{};
    a.R = (uint32_t)p.R;
    a.S = (uint32_t)p.S;
    a.tiles_per_b = np::make_fastdiv((uint32_t)per_b);
    a.n_rt = np::make_fastdiv((uint32_t)n_rt);
    a.n_st = np::make_fastdiv((uint32_t)n_st);
    a.diagonal = p.diagonal ? 1u : 0u;
    const int64_t b_step = std::max<int64_t>(1, lim / per_b);
    for (int64_t b0 = 0; b0 < p.B && e == hipSuccess; b0 += b_step) {
      const int64_t nb = std::min(b_step, p.B - b0);
      e = np::launch_tr_tile(src + b0 * mat_bytes, dst + b0 * mat_bytes, a,
                             (uint32_t)(nb * per_b), p.item, p.vec, stream);
    }
  } else if (p.kernel == TR_SMALL) {
    np::SmallArgs a{};
    a.R = (uint32_t)p.R;
    a.S = (uint32_t)p.S;
    a.per_chunk = (uint32_t)p.per_chunk;
    a.mat_items = np::make_fastdiv((uint32_t)mat_items);
    a.re = np::make_fastdiv((uint32_t)(p.R * p.Ei));
    a.e = np::make_fastdiv((uint32_t)p.Ei);
    const int64_t b_step = lim / p.per_chunk * p.per_chunk;  // keeps 32-bit block math
    for (int64_t b0 = 0; b0 < p.B && e == hipSuccess; b0 += b_step) {
      const int64_t nb = std::min(b_step, p.B - b0);
      a.B = (uint32_t)nb;
      e = np::launch_tr_small(src + b0 * mat_bytes, dst + b0 * mat_bytes, a,
                              (uint32_t)((nb + p.per_chunk - 1) / p.per_chunk), p.item, p.vec,
                              stream);
    }
  } else {
    np::ItemArgs a{};
    a.e = np::make_fastdiv((uint32_t)p.Ei);
    a.r = np::make_fastdiv((uint32_t)p.R);
    a.s = np::make_fastdiv((uint32_t)p.S);
    // whole matrices per launch, fewer than 2^31 items
    const int64_t b_step = std::max<int64_t>(1, lim / mat_items);
    for (int64_t b0 = 0; b0 < p.B && e == hipSuccess; b0 += b_step) {
      const int64_t nb = std::min(b_step, p.B - b0);
      a.n_items = (uint32_t)(nb * mat_items);
      e = np::launch_tr_items(src + b0 * mat_bytes, dst + b0 * mat_bytes, a, p.item, !naive,
                              stream);
    }
  }
  if (e != hipSuccess) return hip_fail(e, who);
  return ok();
}

int validate_rms_linear(const void* x, const void* w, const void* Wt, const void* b,
                        const void* out, int64_t M, int64_t N, int64_t K, float eps, float scale,
                        int dt) {
  if (dt != NP_BF16 && dt != NP_F16)
    return fail(NP_EINVAL, "rmsnorm_linear takes fp16 or bf16 (the matrix-core operand types)");
  if (M < 0 || M >= ((int64_t)1 << 31)) return fail(NP_EINVAL, "M = %lld out of range", (long long)M);
  if (N < 1 || N >= ((int64_t)1 << 31)) return fail(NP_EINVAL, "N = %lld out of range", (long long)N);
  if (K < 8 || K >= ((int64_t)1 << 31) || K % 8 != 0)
    return fail(NP_EINVAL, "K = %lld must be a multiple of 8, >= 8", (long long)K);
  if (((M + 255) / 256) * ((N + 255) / 256) >= ((int64_t)1 << 31))
    return fail(NP_EINVAL, "M x N needs more than 2^31 output tiles of 256 x 256");
  if (!(eps > 0.0f) || !std::isfinite(eps)) return fail(NP_EINVAL, "eps must be finite and > 0");
  if (!std::isfinite(scale)) return fail(NP_EINVAL, "scale must be finite");
  if (M == 0) return NP_OK;  // nothing to compute: no buffer is touched
  if (!x || !Wt || !out) return fail(NP_EINVAL, "NULL x, Wt or out");
  if (!aligned16(x) || !aligned16(Wt) || (w && !aligned16(w)))
    return fail(NP_EINVAL, "x, Wt and w_norm must be 16-byte aligned");
  const uint64_t es = 2, o = (uint64_t)(uintptr_t)out, ob = (uint64_t)M * N * es;
  auto overlaps = [&](const void* p, uint64_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    return p && a < o + ob && o < a + bytes;
  };
  if ((overlaps(x, (uint64_t)M * K * es) || overlaps(Wt, (uint64_t)N * K * es) ||
                overlaps(w, (uint64_t)K * es) || overlaps(b, (uint64_t)N * es)))
    return fail(NP_EINVAL, "out overlaps an input");
  return NP_OK;
}

int shuffle_shape(int64_t N, int64_t C, int64_t H, int64_t W, int64_t groups, int layout,
                  int64_t* B, int64_t* R, int64_t* S, int64_t* E) {
  if (N < 0 || C < 0 || H < 0 || W < 0)
    return fail(NP_EINVAL, "negative size (N=%lld C=%lld H=%lld W=%lld)", (long long)N,
                (long long)C, (long long)H, (long long)W);
  if (groups < 1 || (C % groups) != 0)
    return fail(NP_EINVAL, "groups = %lld must be >= 1 and divide C = %lld", (long long)groups,
                (long long)C);
  if (layout != NP_NCHW && layout != NP_NHWC) return fail(NP_EINVAL, "unknown layout %d", layout);
  if (H > ((int64_t)1 << 31) || W > ((int64_t)1 << 31) || N > ((int64_t)1 << 40))
    return fail(NP_EINVAL, "size out of range");
  *R = groups;
  *S = C / groups;
  if (layout == NP_NCHW) {
    *B = N;
    *E = H * W;
  } else {
    *B = N * H * W;
    *E = 1;
  }
  return NP_OK;
}

}  // namespace

namespace np {

int validate_det_call(const void* const* lv, int n_levels, const int32_t* H, const int32_t* W,
                      const float* strides, const float* anchors, int n_anchors, int n_ch,
                      int batch, int in_dt, const float* out) {
  return validate_det(lv, n_levels, H, W, strides, anchors, n_anchors, n_ch, batch, in_dt, out);
}

int set_error(int code, const char* msg) { return fail(code, "%s", msg); }

int check_device_call() { return check_device(); }

}  // namespace np

extern "C" {

int np_init(int device) {
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess || device < 0 || device >= n)
    return fail(NP_EDEVICE, "device %d not available (%d devices)", device, n);
  e = hipSetDevice(device);
  if (e != hipSuccess) return fail(NP_EDEVICE, "hipSetDevice: %s", hipGetErrorString(e));
  int rc = check_device();
  return rc == NP_OK ? ok() : rc;
}

const char* np_last_error(void) { return g_err.c_str(); }

int np_version(void) { return NP_VERSION; }

void np_shutdown(void) { np::rtc_clear(); }

int fuse_chain(const np_op* ops, int n_ops, const void* const* inputs, int n_inputs,
               np_dtype in_dt, void* out, np_dtype out_dt, int64_t n, hipStream_t stream) {
  int rc = validate_chain(ops, n_ops, inputs, n_inputs, in_dt, out, out_dt, n);
  if (rc) return rc;
  if (n == 0) return ok();
  if ((rc = check_device())) return rc;
  bool vec = aligned16(out);
  for (int j = 0; j < n_inputs; ++j) vec = vec && aligned16(inputs[j]);
  const np::ChainArgs all = chain_args(ops, n_ops, inputs, n_inputs, out, n);
  for (int64_t base = 0; base < n; base += kChainChunk) {
    np::ChainArgs a = all;
    a.n = std::min(kChainChunk, n - base);
    for (int j = 0; j < n_inputs; ++j)
      a.in[j] = static_cast<const char*>(inputs[j]) + base * np::dt_size(in_dt);
    a.out = static_cast<char*>(out) + base * np::dt_size(out_dt);
    hipError_t e;
    if (vec && np::rtc_launch(a, n_inputs, in_dt, out_dt, stream, &e)) {
      if (e != hipSuccess) return hip_fail(e, "fuse_chain (specialised)");
      continue;
    }
    e = np::launch_chain(a, in_dt, out_dt, n_inputs, vec, stream);
    if (e != hipSuccess) return hip_fail(e, "fuse_chain");
  }
  return ok();
}

int fuse_chain_prepare(const np_op* ops, int n_ops, int n_inputs, np_dtype in_dt,
                       np_dtype out_dt, int64_t n_or_0) {
  static const void* dummy[NP_MAX_INPUTS] = {&g_dev_state, &g_dev_state, &g_dev_state,
                                              &g_dev_state};
  int rc = validate_chain(ops, n_ops, dummy, n_inputs, in_dt, &g_dev_state, out_dt, n_or_0);
  if (rc) return rc;
  const char* dis = std::getenv("NP_DISABLE_RTC");
  if (dis && std::strcmp(dis, "1") == 0) return ok();
  if ((rc = check_device())) return rc;
  std::string log;
  np::ChainArgs a = chain_args(ops, n_ops, dummy, n_inputs, nullptr, n_or_0);
  rc = np::rtc_prepare(a, n_inputs, in_dt, out_dt, &log);
  if (rc == NP_ECOMPILE) return fail(NP_ECOMPILE, "runtime compile failed: %s", log.c_str());
  if (rc) return fail(rc, "%s", log.c_str());
  return ok();
}

int fuse_det_decode(const void* const* level_logits, int n_levels, const int32_t* H,
                    const int32_t* W, const float* strides, const float* anchors_wh,
                    int n_anchors, int n_ch, int batch, np_dtype in_dt, float* out,
                    hipStream_t stream) {
  int rc = validate_det(level_logits, n_levels, H, W, strides, anchors_wh, n_anchors, n_ch, batch,
                        in_dt, out);
  if (rc) return rc;
  np::DetArgs a;
  if ((rc = fill_det_args(a, level_logits, n_levels, H, W, strides, anchors_wh, n_anchors, n_ch,
                          batch, out)))
    return rc;
  if ((rc = check_device())) return rc;
  const int N = 16 / np::dt_size(in_dt);
  bool vec = true;
  for (int l = 0; l < n_levels; ++l)
    vec = vec && aligned16(level_logits[l]) && ((int64_t)H[l] * W[l]) % N == 0;
  hipError_t e = np::launch_det_decode(a, in_dt, vec, stream);
  if (e != hipSuccess) return hip_fail(e, "fuse_det_decode");
  return ok();
}

int fuse_add_rmsnorm(const void* x, const void* r, const void* w, void* h_out, void* out,
                     int64_t rows, int64_t cols, float eps, np_dtype dt, hipStream_t stream) {
  int rc = validate_norm(x, out, h_out, rows, cols, eps, dt);
  if (rc) return rc;
  if (rows == 0) return ok();
  if ((rc = check_device())) return rc;
  const bool vec = aligned16(x) && aligned16(out) && (!r || aligned16(r)) &&
                   (!w || aligned16(w)) && (!h_out || aligned16(h_out));
  const int64_t es = np::dt_size(dt);
  for (int64_t r0 = 0; r0 < rows; r0 += kRowChunk) {
    const int64_t off = r0 * cols * es;
    auto at = [&](const void* p) { return p ? static_cast<const char*>(p) + off : nullptr; };
    hipError_t e = np::launch_add_rmsnorm(at(x), at(r), w, const_cast<char*>(at(h_out)),
                                          const_cast<char*>(at(out)),
                                          std::min(kRowChunk, rows - r0), cols, eps, dt, vec,
                                          stream);
    if (e != hipSuccess) return hip_fail(e, "fuse_add_rmsnorm");
  }
  return ok();
}

int fuse_add_layernorm(const void* x, const void* r, const void* gamma, const void* beta,
                       void* h_out, void* out, int64_t rows, int64_t cols, float eps, np_dtype dt,
                       hipStream_t stream) {
  int rc = validate_norm(x, out, h_out, rows, cols, eps, dt);
  if (rc) return rc;
  if (rows == 0) return ok();
  if ((rc = check_device())) return rc;
  const bool vec = aligned16(x) && aligned16(out) && (!r || aligned16(r)) &&
                   (!gamma || aligned16(gamma)) && (!beta || aligned16(beta)) &&
                   (!h_out || aligned16(h_out));
  const int64_t es = np::dt_size(dt);
  for (int64_t r0 = 0; r0 < rows; r0 += kRowChunk) {
    const int64_t off = r0 * cols * es;
    auto at = [&](const void* p) { return p ? static_cast<const char*>(p) + off : nullptr; };
    hipError_t e = np::launch_add_layernorm(at(x), at(r), gamma, beta,
                                            const_cast<char*>(at(h_out)),
                                            const_cast<char*>(at(out)),
                                            std::min(kRowChunk, rows - r0), cols, eps, dt, vec,
                                            stream);
    if (e != hipSuccess) return hip_fail(e, "fuse_add_layernorm");
  }
  return ok();
}

int fuse_qkv_rope(const void* qkv, void* q, void* k, void* v, int64_t T, int n_heads,
                  int head_dim, const int32_t* positions, float base, float q_scale,
                  np_dtype dt, hipStream_t stream) {
  int rc = validate_rope(qkv, q, k, v, T, n_heads, head_dim, base, q_scale, dt);
  if (rc) return rc;
  if (T == 0) return ok();
  if ((rc = check_device())) return rc;
  np::RopeArgs a{};
  a.qkv = qkv;
  a.q = q;
  a.k = k;
  a.v = v;
  a.pos = positions;
  a.T = T;
  a.t0 = 0;
  a.t_end = T;
  a.H = n_heads;
  a.D = head_dim;
  a.q_scale = q_scale;
  inv_freq(base, head_dim, a.inv);
  const bool vec = aligned16(qkv) && aligned16(q) && aligned16(k) && aligned16(v);
  hipError_t e = np::launch_qkv_rope(a, dt, vec, stream);
  if (e != hipSuccess) return hip_fail(e, "fuse_qkv_rope");
  return ok();
}

int unfused_chain(const np_op* ops, int n_ops, const void* const* inputs, int n_inputs,
                  np_dtype in_dt, void* out, np_dtype out_dt, int64_t n, hipStream_t stream) {
  int rc = validate_chain(ops, n_ops, inputs, n_inputs, in_dt, out, out_dt, n);
  if (rc) return rc;
  if (in_dt != out_dt) return fail(NP_EINVAL, "unfused_chain needs in_dt == out_dt");
  if (n >= kUnfusedMax)
    return fail(NP_EINVAL, "n = %lld: the unfused baseline takes fewer than 2^31 elements",
                (long long)n);
  if (n == 0) return ok();
  for (int j = 0; j < n_inputs; ++j) {
    if (inputs[j] != out) continue;
    // the first launch reads this input and overwrites it with its result, so
    // it may alias out only if no later op reads it again
    if (j != ops[0].arg) return fail(NP_EINVAL, "out may alias only the first loaded input");
    for (int i = 1; i < n_ops; ++i)
      if ((ops[i].kind == NP_LOAD || ops[i].kind == NP_ADD_IN || ops[i].kind == NP_MUL_IN) &&
          ops[i].arg == j)
        return fail(NP_EINVAL, "out aliases input %d, which op %d reads after the first launch",
                    j, i);
  }
  if ((rc = check_device())) return rc;
  const void* cur = inputs[ops[0].arg];
  hipError_t e = hipSuccess;
  if (n_ops == 1) e = np::launch_unary(np::U_COPY, 0.0f, cur, out, n, out_dt, stream);
  for (int i = 1; i < n_ops && e == hipSuccess; ++i) {
    const np_op& o = ops[i];
    if (o.kind == NP_LOAD) {
      e = np::launch_unary(np::U_COPY, 0.0f, inputs[o.arg], out, n, out_dt, stream);
    } else if (o.kind == NP_ADD_IN || o.kind == NP_MUL_IN) {
      e = np::launch_binary(o.kind, cur, inputs[o.arg], out, n, out_dt, stream);
    } else {
      e = np::launch_unary(o.kind, o.c, cur, out, n, out_dt, stream);
    }
    cur = out;
  }
  if (e != hipSuccess) return hip_fail(e, "unfused_chain");
  return ok();
}

int unfused_det_decode(const void* const* level_logits, int n_levels, const int32_t* H,
                       const int32_t* W, const float* strides, const float* anchors_wh,
                       int n_anchors, int n_ch, int batch, np_dtype in_dt, float* out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc = validate_det(level_logits, n_levels, H, W, strides, anchors_wh, n_anchors, n_ch, batch,
                        in_dt, out);
  if (rc) return rc;
  int64_t rows = 0;
  for (int l = 0; l < n_levels; ++l) rows += (int64_t)n_anchors * H[l] * W[l];
  const int64_t es = np::dt_size(in_dt);
  if ((int64_t)batch * rows * n_ch >= kUnfusedMax)
    return fail(NP_EINVAL, "the unfused baseline takes fewer than 2^31 output elements");
  const int64_t need = 2 * (int64_t)batch * rows * n_ch * es;
  if (!workspace || (int64_t)workspace_bytes < need)
    return fail(NP_EINVAL, "workspace needs %lld bytes", (long long)need);
  if ((rc = check_device())) return rc;
  char* ws = static_cast<char*>(workspace);
  char* cat = ws + (int64_t)batch * rows * n_ch * es;  // second half: concatenated rows
  const void* parts[8];
  int64_t part_rows[8];
  int64_t off = 0;
  hipError_t e = hipSuccess;
  for (int l = 0; l < n_levels && e == hipSuccess; ++l) {
    void* lv = ws + off * n_ch * es;
    const int h = H[l], w = W[l], A = n_anchors, C = n_ch;
    const float* an = anchors_wh + (size_t)l * n_anchors * 2;
    e = np::launch_det_permute(level_logits[l], lv, batch, A, C, h, w, in_dt, stream);
    if (e == hipSuccess) e = np::launch_det_range_op(lv, batch, A, C, h, w, 0, 2, np::D_SIGMOID, 0, an, in_dt, stream);
    if (e == hipSuccess) e = np::launch_det_range_op(lv, batch, A, C, h, w, 4, C, np::D_SIGMOID, 0, an, in_dt, stream);
    if (e == hipSuccess) e = np::launch_det_range_op(lv, batch, A, C, h, w, 2, 4, np::D_EXP, 0, an, in_dt, stream);
    if (e == hipSuccess) e = np::launch_det_range_op(lv, batch, A, C, h, w, 2, 4, np::D_MUL_ANCHOR, 0, an, in_dt, stream);
    if (e == hipSuccess) e = np::launch_det_range_op(lv, batch, A, C, h, w, 0, 2, np::D_ADD_GRID, 0, an, in_dt, stream);
    if (e == hipSuccess) e = np::launch_det_range_op(lv, batch, A, C, h, w, 0, 2, np::D_MUL_C, strides[l], an, in_dt, stream);
    parts[l] = lv;
    part_rows[l] = (int64_t)A * h * w;
    off += (int64_t)batch * A * h * w;
  }
  if (e == hipSuccess)
    e = np::launch_det_concat(parts, part_rows, n_levels, cat, batch, rows, n_ch, in_dt, stream);
  if (e == hipSuccess) e = np::launch_cast_to_f32(cat, out, (int64_t)batch * rows * n_ch, in_dt, stream);
  if (e != hipSuccess) return hip_fail(e, "unfused_det_decode");
  return ok();
}

int unfused_add_rmsnorm(const void* x, const void* r, const void* w, void* h_out, void* out,
                        int64_t rows, int64_t cols, float eps, np_dtype dt, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  int rc = validate_norm(x, out, h_out, rows, cols, eps, dt);
  if (rc) return rc;
  const int64_t es = np::dt_size(dt);
  const int64_t need = (rows * cols + 2 * rows + (h_out ? 0 : rows * cols)) * es;
  if (rows * cols >= kUnfusedMax || rows >= kUnfusedRowMax)
    return fail(NP_EINVAL, "the unfused baseline takes fewer than 2^31 elements and 2^23 rows");
  if (rows == 0) return ok();
  if (!workspace || (int64_t)workspace_bytes < need)
    return fail(NP_EINVAL, "workspace needs %lld bytes", (long long)need);
  if ((rc = check_device())) return rc;
  char* ws = static_cast<char*>(workspace);
  void* sq = ws;
  void* ms = ws + rows * cols * es;
  void* rs = ws + (rows * cols + rows) * es;
  void* h = h_out ? h_out : ws + (rows * cols + 2 * rows) * es;
  const int64_t n = rows * cols;
  hipError_t e = r ? np::launch_binary(NP_ADD_IN, x, r, h, n, dt, stream)
                   : np::launch_unary(np::U_COPY, 0.0f, x, h, n, dt, stream);
  if (e == hipSuccess) e = np::launch_unary(np::U_SQUARE, 0.0f, h, sq, n, dt, stream);
  if (e == hipSuccess) e = np::launch_row_mean(sq, ms, rows, cols, dt, stream);
  if (e == hipSuccess) e = np::launch_unary(np::U_RSQRT_EPS, eps, ms, rs, rows, dt, stream);
  if (e == hipSuccess) e = np::launch_row_scale(h, rs, out, rows, cols, dt, stream);
  if (e == hipSuccess && w) e = np::launch_col_scale(out, w, out, rows, cols, dt, stream);
  if (e != hipSuccess) return hip_fail(e, "unfused_add_rmsnorm");
  return ok();
}

int unfused_add_layernorm(const void* x, const void* r, const void* gamma, const void* beta,
                          void* h_out, void* out, int64_t rows, int64_t cols, float eps,
                          np_dtype dt, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  int rc = validate_norm(x, out, h_out, rows, cols, eps, dt);
  if (rc) return rc;
  const int64_t es = np::dt_size(dt);
  const int64_t need = (rows * cols + 3 * rows + (h_out ? 0 : rows * cols)) * es;
  if (rows * cols >= kUnfusedMax || rows >= kUnfusedRowMax)
    return fail(NP_EINVAL, "the unfused baseline takes fewer than 2^31 elements and 2^23 rows");
  if (rows == 0) return ok();
  if (!workspace || (int64_t)workspace_bytes < need)
    return fail(NP_EINVAL, "workspace needs %lld bytes", (long long)need);
  if ((rc = check_device())) return rc;
  char* ws = static_cast<char*>(workspace);
  const int64_t n = rows * cols;
  void* d = ws;                              // h - mean
  void* mu = ws + n * es;                    // [rows] mean
  void* var = ws + (n + rows) * es;          // [rows] variance
  void* rs = ws + (n + 2 * rows) * es;       // [rows] 1/sqrt(var + eps)
  void* h = h_out ? h_out : ws + (n + 3 * rows) * es;
  // add; row mean; subtract; square (into out, overwritten later); row mean;
  // +eps and 1/sqrt; times rstd; times gamma; plus beta
  hipError_t e = r ? np::launch_binary(NP_ADD_IN, x, r, h, n, dt, stream)
                   : np::launch_unary(np::U_COPY, 0.0f, x, h, n, dt, stream);
  if (e == hipSuccess) e = np::launch_row_mean(h, mu, rows, cols, dt, stream);
  if (e == hipSuccess) e = np::launch_row_sub(h, mu, d, rows, cols, dt, stream);
  if (e == hipSuccess) e = np::launch_unary(np::U_SQUARE, 0.0f, d, out, n, dt, stream);
  if (e == hipSuccess) e = np::launch_row_mean(out, var, rows, cols, dt, stream);
  if (e == hipSuccess) e = np::launch_unary(np::U_RSQRT_EPS, eps, var, rs, rows, dt, stream);
  if (e == hipSuccess) e = np::launch_row_scale(d, rs, out, rows, cols, dt, stream);
  if (e == hipSuccess && gamma) e = np::launch_col_scale(out, gamma, out, rows, cols, dt, stream);
  if (e == hipSuccess && beta) e = np::launch_col_add(out, beta, out, rows, cols, dt, stream);
  if (e != hipSuccess) return hip_fail(e, "unfused_add_layernorm");
  return ok();
}

int unfused_qkv_rope(const void* qkv, void* q, void* k, void* v, int64_t T, int n_heads,
                     int head_dim, const int32_t* positions, float base, float q_scale,
                     np_dtype dt, hipStream_t stream) {
  int rc = validate_rope(qkv, q, k, v, T, n_heads, head_dim, base, q_scale, dt);
  if (rc) return rc;
  if (T * 3 * n_heads * head_dim >= kUnfusedMax)
    return fail(NP_EINVAL, "the unfused baseline takes fewer than 2^31 elements");
  if (T == 0) return ok();
  if ((rc = check_device())) return rc;
  float inv[256];
  inv_freq(base, head_dim, inv);
  hipError_t e = np::launch_qkv_split(qkv, q, k, v, T, n_heads, head_dim, dt, stream);
  if (e == hipSuccess) e = np::launch_rope_inplace(q, T, n_heads, head_dim, positions, inv, dt, stream);
  if (e == hipSuccess) e = np::launch_rope_inplace(k, T, n_heads, head_dim, positions, inv, dt, stream);
  if (e == hipSuccess)
    e = np::launch_unary(NP_MUL_C, q_scale, q, q, T * n_heads * (int64_t)head_dim, dt, stream);
  if (e != hipSuccess) return hip_fail(e, "unfused_qkv_rope");
  return ok();
}

int np_empty_launches(int count, hipStream_t stream) {
  if (count < 0) return fail(NP_EINVAL, "count < 0");
  int rc = check_device();
  if (rc) return rc;
  for (int i = 0; i < count; ++i) {
    hipError_t e = np::launch_empty(stream);
    if (e != hipSuccess) return hip_fail(e, "np_empty_launches");
  }
  return ok();
}

int fuse_transpose021(const void* in, void* out, int64_t B, int64_t R, int64_t S, int64_t E,
                      int elem_bytes, hipStream_t stream) {
  return run_transpose(in, out, B, R, S, E, elem_bytes, false, stream, "fuse_transpose021");
}

int naive_transpose021(const void* in, void* out, int64_t B, int64_t R, int64_t S, int64_t E,
                       int elem_bytes, hipStream_t stream) {
  return run_transpose(in, out, B, R, S, E, elem_bytes, true, stream, "naive_transpose021");
}

int fuse_channel_shuffle(const void* in, void* out, int64_t N, int64_t C, int64_t H, int64_t W,
                         int64_t groups, int layout, int elem_bytes, hipStream_t stream) {
  int64_t B, R, S, E;
  int rc = shuffle_shape(N, C, H, W, groups, layout, &B, &R, &S, &E);
  if (rc) return rc;
  return run_transpose(in, out, B, R, S, E, elem_bytes, false, stream, "fuse_channel_shuffle");
}

int naive_channel_shuffle(const void* in, void* out, int64_t N, int64_t C, int64_t H, int64_t W,
                          int64_t groups, int layout, int elem_bytes, hipStream_t stream) {
  int64_t B, R, S, E;
  int rc = shuffle_shape(N, C, H, W, groups, layout, &B, &R, &S, &E);
  if (rc) return rc;
  return run_transpose(in, out, B, R, S, E, elem_bytes, true, stream, "naive_channel_shuffle");
}

int fuse_rmsnorm_linear(const void* x, const void* w_norm, const void* Wt, const void* bias,
                        void* out, int64_t M, int64_t N, int64_t K, float eps, float scale,
                        np_dtype dt, hipStream_t stream) {
  int rc = validate_rms_linear(x, w_norm, Wt, bias, out, M, N, K, eps, scale, dt);
  if (rc) return rc;
  if (M == 0) return ok();
  if ((rc = check_device())) return rc;
  hipError_t e = np::launch_rmsnorm_linear(x, w_norm, Wt, bias, out, (int)M, (int)N, (int)K, eps,
                                           scale, dt, true, stream);
  if (e != hipSuccess) return hip_fail(e, "fuse_rmsnorm_linear");
  return ok();
}

int unfused_rmsnorm_linear(const void* x, const void* w_norm, const void* Wt, const void* bias,
                           void* out, int64_t M, int64_t N, int64_t K, float eps, float scale,
                           np_dtype dt, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  int rc = validate_rms_linear(x, w_norm, Wt, bias, out, M, N, K, eps, scale, dt);
  if (rc) return rc;
  if (M * std::max(K, N) >= kUnfusedMax || M >= kUnfusedRowMax)
    return fail(NP_EINVAL, "the unfused baseline takes fewer than 2^31 elements and 2^23 rows");
  if (M == 0) return ok();
  const uint64_t need = (uint64_t)M * K * 2;
  if (!workspace || workspace_bytes < need || !aligned16(workspace))
    return fail(NP_EINVAL, "workspace needs %llu bytes, 16-byte aligned",
                (unsigned long long)need);
  if ((rc = check_device())) return rc;
  // RMSNorm -> y (stored); GEMM + bias -> out; scale -> out
  hipError_t e = np::launch_add_rmsnorm(x, nullptr, w_norm, nullptr, workspace, M, K, eps, dt,
                                        true, stream);
  if (e == hipSuccess)
    e = np::launch_rmsnorm_linear(workspace, nullptr, Wt, bias, out, (int)M, (int)N, (int)K, eps,
                                  1.0f, dt, false, stream);
  if (e == hipSuccess) e = np::launch_unary(NP_MUL_C, scale, out, out, M * N, dt, stream);
  if (e != hipSuccess) return hip_fail(e, "unfused_rmsnorm_linear");
  return ok();
}

int np_fold_norm_weight(const void* w_norm, const void* Wt, void* Wt_folded, int64_t N, int64_t K,
                        np_dtype dt, hipStream_t stream) {
  if (dt != NP_BF16 && dt != NP_F16) return fail(NP_EINVAL, "fold takes fp16 or bf16");
  if (N < 1 || N >= ((int64_t)1 << 31) || K < 8 || K >= ((int64_t)1 << 31) || K % 8 != 0)
    return fail(NP_EINVAL, "bad sizes N = %lld, K = %lld (K a multiple of 8)", (long long)N,
                (long long)K);
  if (!w_norm || !Wt || !Wt_folded) return fail(NP_EINVAL, "NULL argument");
  if (!aligned16(w_norm) || !aligned16(Wt) || !aligned16(Wt_folded))
    return fail(NP_EINVAL, "w_norm, Wt and Wt_folded must be 16-byte aligned");
  const uint64_t bytes = (uint64_t)N * K * 2, a = (uint64_t)(uintptr_t)Wt,
                 o = (uint64_t)(uintptr_t)Wt_folded, wa = (uint64_t)(uintptr_t)w_norm;
  if (a != o && a < o + bytes && o < a + bytes)
    return fail(NP_EINVAL, "Wt_folded partially overlaps Wt");
  if (wa < o + bytes && o < wa + (uint64_t)K * 2) return fail(NP_EINVAL, "Wt_folded overlaps w_norm");
  int rc = check_device();
  if (rc) return rc;
  hipError_t e = np::launch_fold_norm_weight(w_norm, Wt, Wt_folded, N, K, dt, stream);
  if (e != hipSuccess) return hip_fail(e, "np_fold_norm_weight");
  return ok();
}

int np_transpose_plan(const void* in, const void* out, int64_t B, int64_t R, int64_t S,
                      int64_t E, int elem_bytes, int naive) {
  int64_t total = 0;
  int rc = validate_transpose(in, out, B, R, S, E, elem_bytes, &total);
  if (rc) return rc;
  if (total == 0) return ok();
  const TrPlan p = plan_transpose(in, out, B, R, S, E, elem_bytes, naive != 0);
  ok();
  return p.item | (p.kernel << 8) | (p.vec ? 1 << 12 : 0) | (p.diagonal ? 1 << 13 : 0);
}

}  // extern "C"
