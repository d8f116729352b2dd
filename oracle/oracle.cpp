// CPU oracle for the fused-chain library -- TEST INFRASTRUCTURE ONLY.
// Plain scalar C++17, double precision (long double for row sums), built with
// the host compiler (-O2 -ffp-contract=off, no fast-math). It shares no code
// with the GPU library; see oracle.h for the definitions it evaluates.
#include "oracle.h"

#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

enum Dt { kF32 = 0, kF16 = 1, kBF16 = 2 };

// A binary floating-point format: p significand bits (hidden bit included),
// emin = exponent of the smallest normal, emax = exponent of the largest finite.
struct Fmt {
  int p, emin, emax;
};
constexpr Fmt F32{24, -126, 127};   // IEEE 754 binary32
constexpr Fmt F16{11, -14, 15};     // IEEE 754 binary16
constexpr Fmt BF16{8, -126, 127};   // bfloat16: binary32 exponent, 8-bit significand

const Fmt& fmt_of(int dt) { return dt == kF32 ? F32 : dt == kF16 ? F16 : BF16; }

constexpr double U32 = 1.0 / 16777216.0;  // 2^-24, unit roundoff of binary32
constexpr double KAPPA_ARITH = 2.0;
constexpr double KAPPA_TRANS = 8.0;

// Spacing of representable numbers of format f around |a| (a != 0).
double quantum(double a, const Fmt& f) {
  int e;
  std::frexp(std::fabs(a), &e);
  int E = e - 1;  // |a| in [2^E, 2^(E+1))
  if (E < f.emin) E = f.emin;
  return std::ldexp(1.0, E - (f.p - 1));
}

// Round a double to format f, round-to-nearest, ties to even; overflow -> inf.
double round_to(double x, const Fmt& f) {
  if (std::isnan(x) || std::isinf(x) || x == 0.0) return x;
  double a = std::fabs(x);
  double q = quantum(a, f);
  double r = a / q;  // exact: division by a power of two
  double fl = std::floor(r);
  double d = r - fl;
  if (d > 0.5 || (d == 0.5 && std::fmod(fl, 2.0) == 1.0)) fl += 1.0;
  double v = fl * q;
  double maxv = std::ldexp(2.0 - std::ldexp(1.0, -(f.p - 1)), f.emax);
  if (v > maxv) v = INFINITY;
  return std::copysign(v, x);
}

// Bit patterns of an already representable value.
uint16_t encode_small(double v, int mant_bits, int bias, int exp_all_ones, const Fmt& f) {
  uint16_t s = std::signbit(v) ? 0x8000 : 0;
  if (std::isnan(v)) return (uint16_t)((exp_all_ones << mant_bits) | (1u << (mant_bits - 1)));
  double a = std::fabs(v);
  if (std::isinf(a)) return s | (uint16_t)(exp_all_ones << mant_bits);
  if (a == 0.0) return s;
  double min_normal = std::ldexp(1.0, f.emin);
  if (a < min_normal) {  // subnormal: a = m * 2^(emin - mant_bits)
    double m = a / std::ldexp(1.0, f.emin - mant_bits);
    return s | (uint16_t)m;
  }
  int e;
  std::frexp(a, &e);
  int E = e - 1;
  double m = a / std::ldexp(1.0, E - mant_bits) - std::ldexp(1.0, mant_bits);
  return s | (uint16_t)((E + bias) << mant_bits) | (uint16_t)m;
}

double decode_small(uint16_t h, int mant_bits, int exp_bits, int bias) {
  int s = h >> 15;
  int e = (h >> mant_bits) & ((1 << exp_bits) - 1);
  int m = h & ((1 << mant_bits) - 1);
  double v;
  if (e == 0) {
    v = std::ldexp((double)m, 1 - bias - mant_bits);
  } else if (e == (1 << exp_bits) - 1) {
    v = m ? NAN : INFINITY;
  } else {
    v = std::ldexp((double)(m + (1 << mant_bits)), e - bias - mant_bits);
  }
  return s ? -v : v;
}

double f16_val(uint16_t h) { return decode_small(h, 10, 5, 15); }
double bf16_val(uint16_t b) { return decode_small(b, 7, 8, 127); }
uint16_t f16_bits(double v) { return encode_small(v, 10, 15, 31, F16); }
uint16_t bf16_bits(double v) { return encode_small(v, 7, 127, 255, BF16); }

double load(const void* p, int dt, int64_t i) {
  if (dt == kF32) return (double)static_cast<const float*>(p)[i];
  uint16_t b = static_cast<const uint16_t*>(p)[i];
  return dt == kF16 ? f16_val(b) : bf16_val(b);
}

// Store a value that is already representable in dt.
void store(void* p, int dt, int64_t i, double v) {
  if (dt == kF32) {
    static_cast<float*>(p)[i] = (float)v;  // exact: v is a binary32 value
  } else {
    static_cast<uint16_t*>(p)[i] = dt == kF16 ? f16_bits(v) : bf16_bits(v);
  }
}

bool valid_dt(int dt) { return dt == kF32 || dt == kF16 || dt == kBF16; }

double sigmoid(double v) { return 1.0 / (1.0 + std::exp(-v)); }

// A value and a bound on how far an fp32 evaluation may be from it.
struct Tracked {
  double v, b;
};

// Round the tracked value to format f (a cast node or a stored intermediate).
Tracked cast_node(Tracked t, const Fmt& f) {
  double r = round_to(t.v, f);
  bool straddle = round_to(t.v - t.b, f) != round_to(t.v + t.b, f);
  double b = straddle ? t.b + quantum(t.v, f) : 0.0;
  return {r, b};
}

enum Kind {
  LOAD = 0, ADD_IN, MUL_IN, ADD_C, MUL_C, SCALE, RELU, SIGMOID, EXP, TANH, CAST_F16, CAST_BF16,
  N_KINDS
};

}  // namespace

extern "C" {

double oracle_f16_to_double(uint16_t h) { return f16_val(h); }
uint16_t oracle_double_to_f16(double x) { return f16_bits(round_to(x, F16)); }
double oracle_bf16_to_double(uint16_t b) { return bf16_val(b); }
uint16_t oracle_double_to_bf16(double x) { return bf16_bits(round_to(x, BF16)); }
float oracle_double_to_f32(double x) { return (float)round_to(x, F32); }

void oracle_round_array(const double* x, int64_t n, int dt, void* out) {
  const Fmt& f = fmt_of(dt);
  for (int64_t i = 0; i < n; ++i) store(out, dt, i, round_to(x[i], f));
}

int oracle_chain(const int32_t* kinds, const int32_t* args, const float* consts, int n_ops,
                 const void* const* inputs, int n_inputs, int in_dt, void* out, int out_dt,
                 int64_t n, int eager, double* exact, double* bound) {
  if (!kinds || !args || !consts || n_ops <= 0 || !inputs || n_inputs <= 0 || n < 0) return -1;
  if (!valid_dt(in_dt) || !valid_dt(out_dt) || (n > 0 && !out)) return -1;
  if (kinds[0] != LOAD) return -1;
  for (int j = 0; j < n_ops; ++j) {
    if (kinds[j] < 0 || kinds[j] >= N_KINDS) return -1;
    if ((kinds[j] == LOAD || kinds[j] == ADD_IN || kinds[j] == MUL_IN) &&
        (args[j] < 0 || args[j] >= n_inputs || !inputs[args[j]]))
      return -1;
  }
  const Fmt& fo = fmt_of(out_dt);
  for (int64_t i = 0; i < n; ++i) {
    Tracked t{0.0, 0.0};
    for (int j = 0; j < n_ops; ++j) {
      const double c = (double)consts[j];
      const double v = t.v, b = t.b;
      switch (kinds[j]) {
        case LOAD:
          t = {load(inputs[args[j]], in_dt, i), 0.0};
          break;
        case ADD_IN: {
          double s = v + load(inputs[args[j]], in_dt, i);
          t = {s, b + KAPPA_ARITH * U32 * std::fabs(s)};
          break;
        }
        case MUL_IN: {
          double w = load(inputs[args[j]], in_dt, i);
          double p = v * w;
          t = {p, std::fabs(w) * b + KAPPA_ARITH * U32 * std::fabs(p)};
          break;
        }
        case ADD_C: {
          double s = v + c;
          t = {s, b + KAPPA_ARITH * U32 * std::fabs(s)};
          break;
        }
        case MUL_C:
        case SCALE: {
          double p = v * c;
          t = {p, std::fabs(c) * b + KAPPA_ARITH * U32 * std::fabs(p)};
          break;
        }
        case RELU:
          // the page's form: t > 0 ? t : 0 (never -0; NaN maps to +0)
          t = {v > 0.0 ? v : 0.0, b};
          break;
        case SIGMOID: {
          double s = sigmoid(v);
          double m = std::fmax(0.0, std::fabs(v) - b);  // sup of sigma' on [v-b, v+b]
          double sm = sigmoid(m);
          t = {s, sm * (1.0 - sm) * b + KAPPA_TRANS * U32 * s};
          break;
        }
        case EXP: {
          double e = std::exp(v);
          t = {e, e * std::expm1(b) + KAPPA_TRANS * U32 * e};
          break;
        }
        case TANH: {
          double th = std::tanh(v);
          double m = std::tanh(std::fmax(0.0, std::fabs(v) - b));
          t = {th, (1.0 - m * m) * b + KAPPA_TRANS * U32 * std::fabs(th)};
          break;
        }
        case CAST_F16:
          t = cast_node(t, F16);
          break;
        case CAST_BF16:
          t = cast_node(t, BF16);
          break;
      }
      // the running value lives in a binary32 register: beyond its range it is inf
      if (std::isfinite(t.v) && std::isinf(round_to(t.v, F32))) t.v = std::copysign(INFINITY, t.v);
      if (eager && kinds[j] != LOAD) t = cast_node(t, fo);
    }
    if (exact) exact[i] = t.v;
    if (bound) bound[i] = t.b;
    store(out, out_dt, i, round_to(t.v, fo));
  }
  return 0;
}

int oracle_det_decode(const void* const* levels, int n_levels, const int32_t* H,
                      const int32_t* W, const float* strides, const float* anchors,
                      int n_anchors, int n_ch, int batch, int in_dt, float* out, int eager) {
  if (!levels || n_levels <= 0 || !H || !W || !strides || !anchors || n_anchors <= 0 ||
      n_ch < 5 || batch <= 0 || !valid_dt(in_dt) || !out)
    return -1;
  int64_t total_rows = 0;
  for (int l = 0; l < n_levels; ++l) {
    if (H[l] <= 0 || W[l] <= 0 || !levels[l]) return -1;
    total_rows += (int64_t)n_anchors * H[l] * W[l];
  }
  const Fmt& fs = fmt_of(in_dt);  // storage format of the unfused tail
  auto R = [&](double v) { return eager ? round_to(v, fs) : v; };
  for (int b = 0; b < batch; ++b) {
    int64_t row_off = 0;
    for (int l = 0; l < n_levels; ++l) {
      const int64_t hw = (int64_t)H[l] * W[l];
      const double s = strides[l];
      for (int a = 0; a < n_anchors; ++a) {
        const double aw = anchors[(l * n_anchors + a) * 2 + 0];
        const double ah = anchors[(l * n_anchors + a) * 2 + 1];
        for (int y = 0; y < H[l]; ++y) {
          for (int x = 0; x < W[l]; ++x) {
            const int64_t cell = (int64_t)y * W[l] + x;
            const int64_t row = row_off + (int64_t)a * hw + cell;
            float* o = out + ((int64_t)b * total_rows + row) * n_ch;
            for (int k = 0; k < n_ch; ++k) {
              // input element [b, a*n_ch + k, y, x]
              int64_t idx = (((int64_t)b * n_anchors * n_ch + (int64_t)a * n_ch + k) * hw) + cell;
              double t = load(levels[l], in_dt, idx);
              double v;
              if (k == 0) {
                v = R(R(R(sigmoid(t)) + x) * s);
              } else if (k == 1) {
                v = R(R(R(sigmoid(t)) + y) * s);
              } else if (k == 2) {
                v = R(R(std::exp(t)) * aw);
              } else if (k == 3) {
                v = R(R(std::exp(t)) * ah);
              } else {
                v = R(sigmoid(t));
              }
              o[k] = (float)round_to(v, F32);
            }
          }
        }
      }
      row_off += (int64_t)n_anchors * hw;
    }
  }
  return 0;
}

int oracle_add_rmsnorm(const void* x, const void* r, const void* w, void* h_out, void* out,
                       int64_t rows, int64_t cols, float eps, int dt, int eager, double* exact) {
  if (!x || !out || rows < 0 || cols <= 0 || !valid_dt(dt)) return -1;
  if (!(eps > 0.0f) || !std::isfinite(eps)) return -1;
  const Fmt& f = fmt_of(dt);
  std::vector<double> h((size_t)cols);
  for (int64_t i = 0; i < rows; ++i) {
    const int64_t base = i * cols;
    for (int64_t j = 0; j < cols; ++j) {
      double s = load(x, dt, base + j) + (r ? load(r, dt, base + j) : 0.0);
      h[j] = round_to(s, f);  // the stored residual sum is part of the definition
      if (h_out) store(h_out, dt, base + j, h[j]);
    }
    if (!eager) {
      long double ss = 0.0L;
      for (int64_t j = 0; j < cols; ++j) ss += (long double)h[j] * (long double)h[j];
      long double ms = ss / (long double)cols;
      long double rstd = 1.0L / std::sqrt(ms + (long double)eps);
      for (int64_t j = 0; j < cols; ++j) {
        long double wj = w ? (long double)load(w, dt, j) : 1.0L;
        double e = (double)((long double)h[j] * rstd * wj);
        if (exact) exact[base + j] = e;
        store(out, dt, base + j, round_to(e, f));
      }
    } else {
      // add -> square -> row mean -> (+eps, 1/sqrt) -> * rstd -> * w, each stored in dt
      long double ss = 0.0L;
      for (int64_t j = 0; j < cols; ++j) ss += (long double)round_to(h[j] * h[j], f);
      double m = round_to((double)(ss / (long double)cols), f);
      double rs = round_to((double)(1.0L / std::sqrt((long double)m + (long double)eps)), f);
      for (int64_t j = 0; j < cols; ++j) {
        double y = round_to(h[j] * rs, f);
        double wj = w ? load(w, dt, j) : 1.0;
        double e = y * wj;
        if (exact) exact[base + j] = e;
        store(out, dt, base + j, round_to(e, f));
      }
    }
  }
  return 0;
}

int oracle_add_layernorm(const void* x, const void* r, const void* gamma, const void* beta,
                         void* h_out, void* out, int64_t rows, int64_t cols, float eps, int dt,
                         int eager, double* exact) {
  if (!x || !out || rows < 0 || cols <= 0 || !valid_dt(dt)) return -1;
  if (!(eps > 0.0f) || !std::isfinite(eps)) return -1;
  const Fmt& f = fmt_of(dt);
  std::vector<double> h((size_t)cols);
  for (int64_t i = 0; i < rows; ++i) {
    const int64_t base = i * cols;
    for (int64_t j = 0; j < cols; ++j) {
      double s = load(x, dt, base + j) + (r ? load(r, dt, base + j) : 0.0);
      h[j] = round_to(s, f);  // the stored residual sum is what the norm sees
      if (h_out) store(h_out, dt, base + j, h[j]);
    }
    if (!eager) {
      long double sum = 0.0L;
      for (int64_t j = 0; j < cols; ++j) sum += (long double)h[j];
      const long double mu = sum / (long double)cols;
      long double sq = 0.0L;
      for (int64_t j = 0; j < cols; ++j) {
        const long double d = (long double)h[j] - mu;
        sq += d * d;
      }
      const long double rstd = 1.0L / std::sqrt(sq / (long double)cols + (long double)eps);
      for (int64_t j = 0; j < cols; ++j) {
        const long double g = gamma ? (long double)load(gamma, dt, j) : 1.0L;
        const long double b = beta ? (long double)load(beta, dt, j) : 0.0L;
        const double e = (double)(((long double)h[j] - mu) * rstd * g + b);
        if (exact) exact[base + j] = e;
        store(out, dt, base + j, round_to(e, f));
      }
    } else {
      long double sum = 0.0L;
      for (int64_t j = 0; j < cols; ++j) sum += (long double)h[j];
      const double mu = round_to((double)(sum / (long double)cols), f);
      std::vector<double> d((size_t)cols);
      long double sq = 0.0L;
      for (int64_t j = 0; j < cols; ++j) {
        d[j] = round_to(h[j] - mu, f);
        sq += (long double)round_to(d[j] * d[j], f);
      }
      const double var = round_to((double)(sq / (long double)cols), f);
      const double rs = round_to((double)(1.0L / std::sqrt((long double)var + (long double)eps)), f);
      for (int64_t j = 0; j < cols; ++j) {
        double y = round_to(d[j] * rs, f);
        if (gamma) y = round_to(y * load(gamma, dt, j), f);
        const double e = beta ? y + load(beta, dt, j) : y;
        if (exact) exact[base + j] = e;
        store(out, dt, base + j, round_to(e, f));
      }
    }
  }
  return 0;
}

int oracle_rope_inv_freq(float base, int head_dim, float* inv) {
  if (!(base > 0.0f) || head_dim <= 0 || (head_dim & 1) || !inv) return -1;
  for (int i = 0; i < head_dim / 2; ++i)
    inv[i] = (float)round_to(std::pow((double)base, -2.0 * i / head_dim), F32);
  return 0;
}

int oracle_qkv_rope(const void* qkv, void* q, void* k, void* v, int64_t T, int n_heads,
                    int head_dim, const int32_t* positions, float base, float q_scale, int dt,
                    int eager, double* exact_q, double* exact_k, double* bound_q,
                    double* bound_k) {
  if (!qkv || !q || !k || !v || T < 0 || n_heads <= 0 || head_dim <= 0 || (head_dim & 1) ||
      !valid_dt(dt) || !(base > 0.0f) || !std::isfinite(q_scale))
    return -1;
  const Fmt& f = fmt_of(dt);
  const int half = head_dim / 2;
  std::vector<float> inv((size_t)half);
  oracle_rope_inv_freq(base, head_dim, inv.data());
  std::vector<double> cs((size_t)half), sn((size_t)half);
  const double qs = (double)q_scale;
  for (int64_t t = 0; t < T; ++t) {
    const double pos = round_to(positions ? (double)positions[t] : (double)t, F32);
    for (int i = 0; i < half; ++i) {
      const double theta = round_to(pos * (double)inv[i], F32);  // the fp32 angle
      cs[i] = std::cos(theta);
      sn[i] = std::sin(theta);
    }
    for (int s = 0; s < 3; ++s) {
      for (int h = 0; h < n_heads; ++h) {
        const int64_t src = ((t * 3 + s) * n_heads + h) * (int64_t)head_dim;
        const int64_t dst = ((int64_t)h * T + t) * head_dim;
        if (s == 2) {  // V: bit copy
          for (int d = 0; d < head_dim; ++d) {
            if (dt == kF32)
              static_cast<float*>(v)[dst + d] = static_cast<const float*>(qkv)[src + d];
            else
              static_cast<uint16_t*>(v)[dst + d] = static_cast<const uint16_t*>(qkv)[src + d];
          }
          continue;
        }
        void* o = s == 0 ? q : k;
        double* ex = s == 0 ? exact_q : exact_k;
        double* bd = s == 0 ? bound_q : bound_k;
        for (int i = 0; i < half; ++i) {
          const double u = load(qkv, dt, src + i);
          const double w = load(qkv, dt, src + i + half);
          const double o1 = u * cs[i] - w * sn[i];
          const double o2 = w * cs[i] + u * sn[i];
          const double b1 = KAPPA_TRANS * U32 * (std::fabs(u * cs[i]) + std::fabs(w * sn[i]));
          const double b2 = KAPPA_TRANS * U32 * (std::fabs(w * cs[i]) + std::fabs(u * sn[i]));
          Tracked r1{o1, b1}, r2{o2, b2};
          if (s == 0) {
            if (eager) {
              r1 = cast_node(r1, f);
              r2 = cast_node(r2, f);
            }
            r1 = {r1.v * qs, std::fabs(qs) * r1.b + KAPPA_ARITH * U32 * std::fabs(r1.v * qs)};
            r2 = {r2.v * qs, std::fabs(qs) * r2.b + KAPPA_ARITH * U32 * std::fabs(r2.v * qs)};
          }
          if (ex) {
            ex[dst + i] = r1.v;
            ex[dst + i + half] = r2.v;
          }
          if (bd) {
            bd[dst + i] = r1.b;
            bd[dst + i + half] = r2.b;
          }
          store(o, dt, dst + i, round_to(r1.v, f));
          store(o, dt, dst + i + half, round_to(r2.v, f));
        }
      }
    }
  }
  return 0;
}

}  // extern "C"

int oracle_rmsnorm_linear(const void* x, const void* w_norm, const void* Wt, const void* bias,
                          void* out, int64_t M, int64_t N, int64_t K, float eps, float scale,
                          int dt, int eager, double* exact, double* cond) {
  if (!x || !Wt || !out || M < 0 || N < 0 || K <= 0 || !valid_dt(dt)) return -1;
  if (!(eps > 0.0f) || !std::isfinite(eps) || !std::isfinite(scale)) return -1;
  const Fmt& f = fmt_of(dt);
  const long double sc = (long double)scale;
  std::vector<double> a((size_t)K);
  for (int64_t m = 0; m < M; ++m) {
    long double ss = 0.0L;
    for (int64_t k = 0; k < K; ++k) {
      const long double v = load(x, dt, m * K + k);
      ss += v * v;
    }
    const long double rstd = 1.0L / std::sqrt(ss / (long double)K + (long double)eps);
    for (int64_t k = 0; k < K; ++k) {
      const double xv = load(x, dt, m * K + k);
      const double wv = w_norm ? load(w_norm, dt, k) : 1.0;
      // fused: the operand is the product x * w held in fp32, as the
      // section's kernel holds it (exact for 16-bit dt: the product of two
      // such values fits binary32); eager: the RMSNorm kernel's output
      // x * rstd * w, stored in dt
      a[k] = eager ? round_to((double)((long double)xv * rstd * (long double)wv), f)
                   : round_to(xv * wv, F32);
    }
    for (int64_t n = 0; n < N; ++n) {
      long double acc = 0.0L, mag = 0.0L;
      for (int64_t k = 0; k < K; ++k) {
        const long double t = (long double)a[k] * (long double)load(Wt, dt, n * K + k);
        acc += t;
        mag += t < 0 ? -t : t;
      }
      const long double b = bias ? (long double)load(bias, dt, n) : 0.0L;
      double e;
      if (!eager) {
        e = (double)(sc * (rstd * acc + b));
        if (cond) cond[m * N + n] = (double)(std::fabs(sc) * rstd * mag);
      } else {
        const double z = round_to((double)(acc + b), f);
        e = (double)(sc * (long double)z);
        if (cond) cond[m * N + n] = (double)(std::fabs(sc) * mag);
      }
      if (exact) exact[m * N + n] = e;
      store(out, dt, m * N + n, round_to(e, f));
    }
  }
  return 0;
}

int oracle_channel_shuffle(const void* in, void* out, int64_t N, int64_t C, int64_t H,
                           int64_t W, int64_t groups, int layout, int elem_bytes) {
  if (!in || !out || N < 0 || C < 0 || H < 0 || W < 0 || groups <= 0 || elem_bytes < 1 ||
      elem_bytes > 16 || (layout != 0 && layout != 1))
    return -1;
  if (C % groups != 0) return -1;
  const int64_t per = C / groups;  // channels per group
  const unsigned char* src = static_cast<const unsigned char*>(in);
  unsigned char* dst = static_cast<unsigned char*>(out);
  const size_t es = (size_t)elem_bytes;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t g = 0; g < groups; ++g)
      for (int64_t i = 0; i < per; ++i) {
        const int64_t c_in = g * per + i;
        const int64_t c_out = i * groups + g;
        for (int64_t y = 0; y < H; ++y)
          for (int64_t x = 0; x < W; ++x) {
            int64_t a, b;  // element offsets of (n, c, y, x) in the input and output
            if (layout == 0) {
              a = ((n * C + c_in) * H + y) * W + x;
              b = ((n * C + c_out) * H + y) * W + x;
            } else {
              a = ((n * H + y) * W + x) * C + c_in;
              b = ((n * H + y) * W + x) * C + c_out;
            }
            std::memcpy(dst + (size_t)b * es, src + (size_t)a * es, es);
          }
      }
  return 0;
}

int oracle_transpose021(const void* in, void* out, int64_t B, int64_t R, int64_t S, int64_t E,
                        int elem_bytes) {
  if (!in || !out || B < 0 || R < 0 || S < 0 || E < 0 || elem_bytes < 1 || elem_bytes > 16)
    return -1;
  const unsigned char* src = static_cast<const unsigned char*>(in);
  unsigned char* dst = static_cast<unsigned char*>(out);
  const size_t es = (size_t)elem_bytes;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t r = 0; r < R; ++r)
      for (int64_t s = 0; s < S; ++s)
        for (int64_t e = 0; e < E; ++e) {
          const int64_t a = ((b * R + r) * S + s) * E + e;
          const int64_t o = ((b * S + s) * R + r) * E + e;
          std::memcpy(dst + (size_t)o * es, src + (size_t)a * es, es);
        }
  return 0;
}
