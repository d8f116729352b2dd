// Runtime specialisation of elementwise chains (DeepJIT write-up,
// hotelren.com/news/5350627):
//  - section 3.1/3.3: generate the kernel source at run time with the sizes,
//    the vector width and the op list written in as constants, so the compiler
//    sees straight-line code and constant bounds;
//  - section 3.2: compile at run time and load the module (hipRTC for gfx950,
//    hipModuleLoadData, hipModuleGetFunction in the current context);
//  - section 3.3 / 6.2: a process-wide cache keyed by a hash of source,
//    architecture and options; compile only at warm-up (fuse_chain_prepare),
//    never on the launch path;
//  - section 6.2: the compiled code object also persisted on disk (when
//    NP_CACHE_DIR names a directory), so a restarted process loads it instead
//    of compiling;
//  - section 6.3: no fast-math; section 6.4: modules live until np_shutdown.
#include "rtc.h"

#include <errno.h>
#include <hip/hiprtc.h>
#include <sys/stat.h>
#include <unistd.h>

#include <atomic>
#include <chrono>
#include <cfloat>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <map>
#include <unordered_map>
#include <mutex>
#include <sstream>
#include <vector>

namespace np {
namespace {

// fastmath.h, pasted into generated sources (written by the build as a raw string)
const char* kFastMathSource =
#include "gen_fastmath.inc"
    ;

const char* type_name(int dt) {
  return dt == NP_F32 ? "float" : dt == NP_F16 ? "_Float16" : "__bf16";
}

std::string hexf(float c) {
  char buf[64];
  std::snprintf(buf, sizeof buf, "%af", (double)c);  // exact binary32 literal
  return buf;
}

std::string op_line(int kind, int arg, float c, bool fast) {
  const std::string x = "x" + std::to_string(arg) + "[e]";
  switch (kind) {
    case NP_LOAD: return "v = " + x + ";";
    case NP_ADD_IN: return "v = v + " + x + ";";
    case NP_MUL_IN: return "v = v * " + x + ";";
    case NP_ADD_C: return "v = v + " + hexf(c) + ";";
    case NP_MUL_C:
    case NP_SCALE: return "v = v * " + hexf(c) + ";";
    case NP_RELU: return "v = v > 0.0f ? v : 0.0f;";
    case NP_SIGMOID: return fast ? "v = np_fast_sigmoid(v);" : "v = 1.0f / (1.0f + expf(-v));";
    case NP_EXP: return fast ? "v = np_fast_exp(v);" : "v = expf(v);";
    case NP_TANH: return fast ? "v = np_fast_tanh(v);" : "v = tanhf(v);";
    case NP_CAST_F16: return "v = (float)(_Float16)v;";
    case NP_CAST_BF16: return "v = (float)(__bf16)v;";
  }
  return "";
}

// fp16-output chains (the fast transcendental policy) are also folded at
// generation time; the rewritten chain equals the original in exact
// arithmetic:
//  - runs of constant multiplies (mul_c, scale) become one multiply by their
//    product, runs of add_c one add of their sum (constants combined in
//    double, rounded once);
//  - a multiply followed by an add becomes one fused multiply-add;
//  - an affine map in front of an exp (x a + b, or (x + b) a = x a + a b)
//    folds into the exp's constants, exp(x a + b) = e^b 2^(x a log2 e), and a
//    multiply after it into its factor: e^b c 2^(x a log2 e), and the factor
//    into the exponent, 2^(x a log2 e + log2 |e^b c|) (np_fast_exp_shifted:
//    one FMA and v_exp_f32);
//  - likewise in front of a sigmoid: 1 / (1 + e^-b 2^(-x a log2 e))
//    (np_fast_sigmoid_affine);
//  - the factor of a folded exp moves into the constant of an exp or sigmoid
//    that follows it directly (2^(x c1) e1 c2 = 2^(x c1) (e1 c2));
//  - a cast that repeats the cast before it is dropped.
// Each tanh is then emitted in the cheapest form that holds on the range of
// its argument (value ranges below).
bool is_mul(int k) { return k == NP_MUL_C || k == NP_SCALE; }

constexpr double kLog2e = 1.4426950408889634074;
constexpr double kInf = HUGE_VAL;

// ---- value ranges ----------------------------------------------------------
// Before every op the specialiser tracks an interval that holds every binary32
// value the generated code can compute there (NaN aside: NaN passes through
// every emitted form). A loaded input may be any value of its type,
// infinities included. Each op maps the interval through its monotone real
// function; the result is widened by 2^-16 of the largest finite magnitude
// among operand, constant and result, plus 2^-126 -- more than the rounding
// and approximation error of any form emitted for it (<= 4 ulp of the result,
// 2^-24 of the operands of a folded sum, or |t| / 2 ulp for the exponent t,
// |t| < 152, of a folded exp or sigmoid) -- and a bound beyond the binary32 range becomes
// infinite (the computed value overflows there). Ops whose computed result
// always has the sign of the exact one (multiply, exp, sigmoid, tanh, casts)
// do not widen across zero. Casts widen by their own half ulp.
struct Range {
  double lo, hi;
};

constexpr double kRangeRel = 0x1p-16;

double finite_mag(const Range& r) {
  return std::fmax(std::isfinite(r.lo) ? std::fabs(r.lo) : 0.0,
                   std::isfinite(r.hi) ? std::fabs(r.hi) : 0.0);
}

Range widen(const Range& r, double d, bool keeps_sign, double max_finite) {
  Range w{r.lo - d, r.hi + d};
  if (keeps_sign && r.lo >= 0.0) w.lo = std::fmax(w.lo, 0.0);
  if (keeps_sign && r.hi <= 0.0) w.hi = std::fmin(w.hi, 0.0);
  if (w.lo < -max_finite) w.lo = -kInf;
  if (w.hi > max_finite) w.hi = kInf;
  return w;
}

// an op's exact image r of the operand interval -> the computed values
Range computed(const Range& r, double operand_mag, bool keeps_sign) {
  const double d = std::fmax(operand_mag, finite_mag(r)) * kRangeRel + 0x1p-126;
  return widen(r, d, keeps_sign, FLT_MAX);
}

Range cast_to(const Range& r, double half_ulp_rel, double half_ulp_min, double max_finite) {
  return widen(r, finite_mag(r) * half_ulp_rel + half_ulp_min, true, max_finite);
}

double sigmoid_d(double t) { return 1.0 / (1.0 + std::exp(-t)); }

std::vector<Range> op_ranges(const ChainArgs& a) {
  std::vector<Range> before(a.n_ops);
  Range r{-kInf, kInf};
  for (int i = 0; i < a.n_ops; ++i) {
    before[i] = r;
    const double c = a.c[i];
    switch (a.kind[i]) {
      case NP_ADD_C:
        r = computed({r.lo + c, r.hi + c}, std::fmax(finite_mag(r), std::fabs(c)), false);
        break;
      case NP_MUL_C:
      case NP_SCALE:
        // 0 * inf is NaN, which the interval does not hold
        r = computed(c > 0 ? Range{r.lo * c, r.hi * c}
                           : c < 0 ? Range{r.hi * c, r.lo * c} : Range{0.0, 0.0},
                     0.0, true);
        break;
      case NP_RELU: r = {0.0, std::fmax(r.hi, 0.0)}; break;  // a NaN input gives 0
      case NP_EXP: r = computed({std::exp(r.lo), std::exp(r.hi)}, 0.0, true); break;
      case NP_SIGMOID: r = computed({sigmoid_d(r.lo), sigmoid_d(r.hi)}, 0.0, true); break;
      case NP_TANH: r = computed({std::tanh(r.lo), std::tanh(r.hi)}, 0.0, true); break;
      case NP_CAST_F16: r = cast_to(r, 0x1p-11, 0x1p-25, 65504.0); break;
      case NP_CAST_BF16: r = cast_to(r, 0x1p-8, 0x1p-134, 0x1.fep127); break;
      default: r = {-kInf, kInf}; break;  // a loaded input: any value
    }
  }
  return before;
}

// ---- constants held in vector registers -------------------------------------
// Operands that cannot be literals (a second constant in one FMA, the addend of
// a mixed-precision FMA) are pinned once per thread, kp[i] = np_pin(c), and
// referred to by index in the chain, so the unrolled elements share them.
struct Pins {
  std::vector<float> v;
  std::string ref(float c) {
    for (size_t i = 0; i < v.size(); ++i)
      if (std::memcmp(&v[i], &c, 4) == 0) return "kp[" + std::to_string(i) + "]";
    v.push_back(c);
    return "kp[" + std::to_string(v.size() - 1) + "]";
  }
};

// ---- tanh on a known range -------------------------------------------------
// Odd Taylor series tanh x = x + sum_k T_k x^(2k+1) (coefficients from the
// Bernoulli numbers: -1/3, 2/15, -17/315, 62/2835, -1382/155925). For
// |x| <= 1/2 its terms alternate in sign and shrink by a factor below 0.41 x^2,
// so cutting it after T_k x^(2k+1) leaves a relative error below
// |T_(k+1)| x^(2k+2) / (1 - x^2/3). A cut is taken when that is at most 2^-26
// (a quarter of a binary32 ulp); Horner's rounding adds < 1/4 ulp (the
// correction term is under 0.09 x), the final FMA 1/2 ulp.
constexpr double kTanhT[6] = {1.0,           -1.0 / 3.0,       2.0 / 15.0,
                              -17.0 / 315.0, 62.0 / 2835.0,   -1382.0 / 155925.0};
constexpr double kTanhTau = 0x1p-26;
// the leading coefficient of the minimax polynomial in fastmath.h (NP_TANH_P4),
// which the generated code passes to np_fast_tanh_*_k from a pinned register
constexpr float kTanhP4 = -0.005704987328499556f;

std::string tanh_on(const Range& r, Pins* pins) {
  const double m = std::fmax(std::fabs(r.lo), std::fabs(r.hi));
  const double shrink = 1.0 / (1.0 - m * m / 3.0);
  if (m <= 0.5) {
    if (m * m / 3.0 * shrink <= kTanhTau) return "";  // tanh x = x to 2^-26
    for (int k = 1; k <= 4; ++k) {
      if (std::fabs(kTanhT[k + 1]) * std::pow(m, 2 * k + 2) * shrink > kTanhTau) continue;
      std::string l = "{ const float z = v * v; ";
      if (k == 1) return l + "v = __builtin_fmaf(v * z, " + hexf((float)kTanhT[1]) + ", v); }";
      l += "float p = " + pins->ref((float)kTanhT[k]) + "; ";
      for (int j = k - 1; j >= 1; --j) l += "p = __builtin_fmaf(p, z, " + hexf((float)kTanhT[j]) + "); ";
      return l + "v = __builtin_fmaf(v * z, p, v); }";
    }
  }
  if (r.lo >= 0.625) return "v = np_fast_tanh_exp_pos(v);";
  if (r.hi <= -0.625) return "v = np_fast_tanh_exp_neg(v);";
  const std::string k4 = pins->ref(kTanhP4);
  if (m < 0.625) return "v = np_fast_tanh_poly_k(v, " + k4 + ");";
  if (r.lo >= 0.0) return "v = np_fast_tanh_pos_k(v, " + k4 + ");";
  if (r.hi <= 0.0) return "v = np_fast_tanh_neg_k(v, " + k4 + ");";
  return "v = np_fast_tanh_k(v, " + k4 + ");";
}

// ---- folded op list --------------------------------------------------------
enum : int { K_FMA = 100, K_EXPA, K_SIGA };

struct Node {
  int kind;                 // an NP_ op kind, or K_FMA / K_EXPA / K_SIGA
  int arg = 0;              // input index (LOAD, ADD_IN, MUL_IN)
  double m = 1.0, b = 0.0;  // MUL_C: m; ADD_C: b; FMA: v m + b; EXPA / SIGA: constant m, factor b
  Range in{-kInf, kInf};    // range of v in front of a tanh
};

// A folded constant must stay a normal binary32 number (or zero): e^b of a
// large |b| would overflow where the unfolded add would not.
bool foldable(double x) {
  const double a = std::fabs(x);
  return a == 0.0 || (a >= 0x1p-100 && a <= 0x1p100);
}

std::vector<Node> fold_fast(const ChainArgs& a) {
  const std::vector<Range> before = op_ranges(a);
  std::vector<Node> out;
  const int n = a.n_ops;
  int i = 0;
  auto run = [&](int j, bool mul, double* acc) {  // consume a run of mul (or add) constants
    *acc = mul ? 1.0 : 0.0;
    while (j < n && (mul ? is_mul(a.kind[j]) : a.kind[j] == NP_ADD_C)) {
      *acc = mul ? *acc * (double)a.c[j] : *acc + (double)a.c[j];
      ++j;
    }
    return j;
  };
  auto transcendental = [&](int j) {
    return j < n && (a.kind[j] == NP_EXP || a.kind[j] == NP_SIGMOID);
  };
  // the exp or sigmoid at j after the affine map x m + b, folded into one node
  // when its constants stay foldable; *next = the op after it
  auto fold_at = [&](int j, double m, double b, Node* t, int* next) {
    if (a.kind[j] == NP_EXP) {
      double after = 1.0;
      *next = run(j + 1, true, &after);
      *t = {K_EXPA, 0, m * kLog2e, std::exp(b) * after};
    } else {
      *next = j + 1;
      *t = {K_SIGA, 0, -m * kLog2e, std::exp(-b)};
    }
    return foldable(t->m) && foldable(t->b);
  };
  while (i < n) {
    const int k = a.kind[i];
    if (is_mul(k) || k == NP_ADD_C || k == NP_EXP || k == NP_SIGMOID) {
      double m = 1.0, b = 0.0;
      int j = i, next = 0;
      Node t{0};
      if (is_mul(k)) j = run(j, true, &m);
      if (j < n && a.kind[j] == NP_ADD_C) j = run(j, false, &b);
      if (k == NP_ADD_C && j < n && is_mul(a.kind[j])) {
        // (x + b) m in front of an exp or sigmoid is x m + b m
        double m2 = 1.0;
        const int j2 = run(j, true, &m2);
        if (transcendental(j2) && fold_at(j2, m2, b * m2, &t, &next)) {
          out.push_back(t);
          i = next;
          continue;
        }
      }
      if (transcendental(j)) {
        if (fold_at(j, m, b, &t, &next)) {
          out.push_back(t);
          i = next;
          continue;
        }
        if (j == i) {  // a bare exp or sigmoid whose following factor cannot fold
          out.push_back({t.kind, 0, t.kind == K_EXPA ? kLog2e : -kLog2e, 1.0});
          i = j + 1;
          continue;
        }
        // otherwise the affine map stays a separate statement
      }
      const bool has_mul = is_mul(k), has_add = a.kind[j - 1] == NP_ADD_C;
      if (has_mul && has_add)
        out.push_back({K_FMA, 0, m, b});
      else if (has_mul)
        out.push_back({NP_MUL_C, 0, m, 0.0});
      else
        out.push_back({NP_ADD_C, 0, 1.0, b});
      i = j;
      continue;
    }
    if ((k == NP_CAST_F16 || k == NP_CAST_BF16) && i > 0 && a.kind[i - 1] == k) {
      ++i;  // casting again to the same type changes nothing
      continue;
    }
    Node op{k, a.arg[i], (double)a.c[i], (double)a.c[i]};
    op.in = before[i];
    out.push_back(op);
    ++i;
  }
  // an exp's factor moves into the constant of the exp or sigmoid after it
  for (size_t q = 0; q + 1 < out.size(); ++q) {
    if (out[q].kind != K_EXPA || (out[q + 1].kind != K_EXPA && out[q + 1].kind != K_SIGA))
      continue;
    const double c = out[q + 1].m * out[q].b;
    if (!foldable(c)) continue;
    out[q + 1].m = c;
    out[q].b = 1.0;
  }
  return out;
}

std::string emit(const Node& n, Pins* pins) {
  switch (n.kind) {
    case K_FMA:
      return "v = __builtin_fmaf(v, " + hexf((float)n.m) + ", " + hexf((float)n.b) + ");";
    case K_EXPA: {
      if (n.b == 1.0) return "v = __builtin_amdgcn_exp2f(v * " + hexf((float)n.m) + ");";
      if (n.b == 0.0)
        return "v = np_fast_exp_affine(v, " + hexf((float)n.m) + ", " + hexf(0.0f) + ");";
      const std::string call = "np_fast_exp_shifted(v, " + hexf((float)n.m) + ", " +
                               pins->ref((float)std::log2(std::fabs(n.b))) + ")";
      return n.b < 0.0 ? "v = -" + call + ";" : "v = " + call + ";";
    }
    case K_SIGA:
      return "v = np_fast_sigmoid_affine(v, " + hexf((float)n.m) + ", " + pins->ref((float)n.b) +
             ");";
    case NP_MUL_C: return "v = v * " + hexf((float)n.m) + ";";
    case NP_ADD_C: return "v = v + " + hexf((float)n.b) + ";";
    case NP_TANH: {
      char buf[96];
      std::snprintf(buf, sizeof buf, "// tanh argument in [%a, %a]", n.in.lo, n.in.hi);
      const std::string f = tanh_on(n.in, pins);
      return std::string(buf) + (f.empty() ? " (tanh x = x there)" : "\n  " + f);
    }
    default: return op_line(n.kind, n.arg, (float)n.m, true);
  }
}

// Emits the folded ops; a cast to fp16 is merged with a constant multiply, add
// or FMA right before it (np_{mul,add,fma}_to_f16: one rounding to fp16) and
// with a constant multiply, FMA or pure 2^(v c) right after it
// (np_{mul,fma}_from_f16 take the fp16 value as is), which saves the
// conversions between them.
bool affine_node(const Node& n) {
  return n.kind == NP_MUL_C || n.kind == NP_ADD_C || n.kind == K_FMA;
}

std::vector<std::string> emit_all(const std::vector<Node>& nodes, Pins* pins) {
  std::vector<std::string> out;
  const size_t n = nodes.size();
  size_t i = 0;
  while (i < n) {
    const bool before = affine_node(nodes[i]) && i + 1 < n && nodes[i + 1].kind == NP_CAST_F16;
    if (!before && nodes[i].kind != NP_CAST_F16) {
      out.push_back(emit(nodes[i], pins));
      ++i;
      continue;
    }
    std::string l = "{ const _Float16 h = ";
    if (before) {
      const Node& f = nodes[i];
      if (f.kind == NP_MUL_C)
        l += "np_mul_to_f16(v, " + hexf((float)f.m) + "); ";
      else if (f.kind == NP_ADD_C)
        l += "np_add_to_f16(v, " + hexf((float)f.b) + "); ";
      else
        l += "np_fma_to_f16(v, " + hexf((float)f.m) + ", " + pins->ref((float)f.b) + "); ";
      i += 2;  // the op and the cast
    } else {
      l += "(_Float16)v; ";
      i += 1;
    }
    const Node* g = i < n ? &nodes[i] : nullptr;
    if (g && g->kind == K_FMA) {
      l += "v = np_fma_from_f16(h, " + hexf((float)g->m) + ", " + pins->ref((float)g->b) + "); }";
      ++i;
    } else if (g && g->kind == NP_MUL_C) {
      l += "v = np_mul_from_f16(h, " + hexf((float)g->m) + "); }";
      ++i;
    } else if (g && g->kind == K_EXPA && g->b == 1.0) {
      l += "v = __builtin_amdgcn_exp2f(np_mul_from_f16(h, " + hexf((float)g->m) + ")); }";
      ++i;
    } else {
      l += "v = (float)h; }";
    }
    out.push_back(l);
  }
  return out;
}

struct Entry {
  hipModule_t mod = nullptr;
  hipFunction_t fn = nullptr;         // vector kernel
  hipFunction_t fn_scalar = nullptr;  // one element per thread
  hipFunction_t fn_lut = nullptr;     // table gather (tabulable chains, table built)
  size_t src_hash = 0;
  int dev = 0;
  int cus = 256;                      // compute units of dev (the gather's grid)
};

// From this many elements the table gather wins: below it, staging the
// 128 KiB table on every CU costs more than evaluating the chain.
std::atomic<int64_t> g_lut_min_n{int64_t(1) << 22};

// Same threshold as the generic kernel: below it, one element per thread.
constexpr int64_t kMinVecGroups = 65536;

std::mutex g_mu;
std::unordered_map<std::string, Entry> g_cache;  // spec key -> loaded kernel

// The key of a specialisation, built on every fuse_chain call: the device,
// dtypes, input count, op count and n, then each op's kind, input index and
// constant bits, copied as fixed-size bytes (formatting them as text took
// microseconds per call for a 30-op chain). n sits at byte kKeyN.
constexpr size_t kKeyN = 5 * sizeof(int32_t);
std::string spec_key(const ChainArgs& a, int n_inputs, int in_dt, int out_dt, int64_t n,
                     int dev) {
  const int32_t head[5] = {dev, in_dt, out_dt, n_inputs, a.n_ops};
  std::string k;
  k.reserve(sizeof(head) + sizeof(n) + (size_t)a.n_ops * 12);
  k.append(reinterpret_cast<const char*>(head), sizeof(head));
  k.append(reinterpret_cast<const char*>(&n), sizeof(n));
  for (int i = 0; i < a.n_ops; ++i) {
    int32_t op[3] = {a.kind[i], a.arg[i], 0};
    std::memcpy(&op[2], &a.c[i], 4);
    k.append(reinterpret_cast<const char*>(op), sizeof(op));
  }
  return k;
}

const char* kOptions[] = {"--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang",
                          "-target-feature", "-Xclang", "-packed-fp32-ops"};
constexpr int kNumOptions = sizeof(kOptions) / sizeof(kOptions[0]);

int compile(const std::string& src, std::vector<char>* code, std::string* log) {
  hiprtcProgram prog;
  if (hiprtcCreateProgram(&prog, src.c_str(), "np_chain_spec.hip", 0, nullptr, nullptr) !=
      HIPRTC_SUCCESS) {
    *log = "hiprtcCreateProgram failed";
    return NP_ECOMPILE;
  }
  hiprtcResult r = hiprtcCompileProgram(prog, kNumOptions, kOptions);
  size_t log_size = 0;
  hiprtcGetProgramLogSize(prog, &log_size);
  if (log_size > 1) {
    std::string l(log_size, '\0');
    hiprtcGetProgramLog(prog, &l[0]);
    *log = l;
  }
  if (r != HIPRTC_SUCCESS) {
    hiprtcDestroyProgram(&prog);
    return NP_ECOMPILE;
  }
  size_t sz = 0;
  hiprtcGetCodeSize(prog, &sz);
  code->resize(sz);
  hiprtcGetCode(prog, code->data());
  hiprtcDestroyProgram(&prog);
  return NP_OK;
}

// ---- code objects on disk (DeepJIT write-up, section 6.2: the second cache
// level, compiled output kept on disk so a restarted process skips compiling)
//
// A file <dir>/<fnv-1a 64 of the key text>.npco holds the 8-byte magic
// "NPCHAIN1", the key text's length (u64) and text, the code object's length
// (u64) and bytes. The key text is the hipRTC version, the library's HIP
// version, the options and the whole generated source; a file is used only
// when its key text equals the expected one byte for byte, so a hash
// collision, a stale file or a truncated one is a miss. Files are written
// under a unique temporary name and renamed into place, so concurrent
// processes never read a partial file. The cache is best effort: any I/O
// failure falls back to compiling.
constexpr char kMagic[8] = {'N', 'P', 'C', 'H', 'A', 'I', 'N', '1'};
std::atomic<int64_t> g_disk_loads{0}, g_disk_stores{0}, g_disk_rejects{0};
std::atomic<uint64_t> g_tmp_counter{0};

// NP_CACHE_DIR, or "" (no disk cache) when it is unset or empty
std::string cache_dir() {
  const char* d = std::getenv("NP_CACHE_DIR");
  return d ? std::string(d) : std::string();
}

std::string key_text(const std::string& src) {
  int major = 0, minor = 0;
  (void)hiprtcVersion(&major, &minor);
  std::ostringstream k;
  k << "hiprtc " << major << "." << minor << " | hip " << HIP_VERSION << " |";
  for (int i = 0; i < kNumOptions; ++i) k << ' ' << kOptions[i];
  k << '\n' << src;
  return k.str();
}

std::string cache_path(const std::string& dir, const std::string& key) {
  uint64_t h = 1469598103934665603ull;  // FNV-1a, 64-bit
  for (unsigned char c : key) {
    h ^= c;
    h *= 1099511628211ull;
  }
  char name[32];
  std::snprintf(name, sizeof(name), "/%016llx.npco", (unsigned long long)h);
  return dir + name;
}

bool make_dirs(const std::string& dir) {
  for (size_t i = 1; i <= dir.size(); ++i) {
    if (i == dir.size() || dir[i] == '/') {
      const std::string part = dir.substr(0, i);
      if (mkdir(part.c_str(), 0755) != 0 && errno != EEXIST) return false;
    }
  }
  struct stat st;
  return stat(dir.c_str(), &st) == 0 && S_ISDIR(st.st_mode);
}

// the cached code object for this key, if a valid file holds it
bool disk_load(const std::string& dir, const std::string& key, std::vector<char>* code) {
  FILE* f = std::fopen(cache_path(dir, key).c_str(), "rb");
  if (!f) return false;
  bool ok = false;
  char magic[8];
  uint64_t klen = 0, clen = 0;
  if (std::fread(magic, 1, 8, f) == 8 && std::memcmp(magic, kMagic, 8) == 0 &&
      std::fread(&klen, 8, 1, f) == 1 && klen == key.size()) {
    std::string k(klen, '\0');
    if (std::fread(&k[0], 1, klen, f) == klen && k == key && std::fread(&clen, 8, 1, f) == 1 &&
        clen > 0 && clen < (uint64_t(1) << 30)) {
      code->resize(clen);
      char extra;
      ok = std::fread(code->data(), 1, clen, f) == clen && std::fread(&extra, 1, 1, f) == 0;
    }
  }
  std::fclose(f);
  if (!ok) {
    code->clear();
    g_disk_rejects.fetch_add(1);
  }
  return ok;
}

void disk_store(const std::string& dir, const std::string& key, const std::vector<char>& code) {
  if (!make_dirs(dir)) return;
  const std::string path = cache_path(dir, key);
  char suffix[64];
  std::snprintf(suffix, sizeof(suffix), ".tmp.%ld.%llu", (long)getpid(),
                (unsigned long long)g_tmp_counter.fetch_add(1));
  const std::string tmp = path + suffix;
  FILE* f = std::fopen(tmp.c_str(), "wb");
  if (!f) return;
  const uint64_t klen = key.size(), clen = code.size();
  bool ok = std::fwrite(kMagic, 1, 8, f) == 8 && std::fwrite(&klen, 8, 1, f) == 1 &&
            std::fwrite(key.data(), 1, klen, f) == klen && std::fwrite(&clen, 8, 1, f) == 1 &&
            std::fwrite(code.data(), 1, clen, f) == clen;
  ok = (std::fclose(f) == 0) && ok;
  if (ok && std::rename(tmp.c_str(), path.c_str()) == 0) {
    g_disk_stores.fetch_add(1);
  } else {
    std::remove(tmp.c_str());
  }
}

}  // namespace

// Kernel names carry the op count and the size written in (0: size at launch),
// so a profiler tells the specialisations apart.
// A chain over one 16-bit input with a 16-bit output is a function of the
// 65,536 input bit patterns: the specialised module also carries that function
// as a table (np_lut, filled once at prepare time by the module's own chain
// code) and a kernel that streams the input through it.
static bool tabulable(int n_inputs, int in_dt, int out_dt) {
  return n_inputs == 1 && in_dt != NP_F32 && out_dt != NP_F32;
}

static std::string spec_name(const ChainArgs& a, int64_t n, bool scalar) {
  return std::string(scalar ? "np_chain_scalar" : "np_chain_spec") + "_k" +
         std::to_string(a.n_ops) + "_n" + std::to_string(n);
}

std::string rtc_source(const ChainArgs& a, int n_inputs, int in_dt, int out_dt, int64_t n) {
  const int G = (in_dt != NP_F32 || out_dt != NP_F32) ? 8 : 4;
  const bool fast = out_dt == NP_F16;  // same transcendental policy as the generic kernel
  std::ostringstream s;
  s << "// generated: fused elementwise chain, " << a.n_ops << " ops\n"
    << kFastMathSource << "\n"
    << "typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));\n"
    << "typedef " << type_name(in_dt) << " tin;\n"
    << "typedef " << type_name(out_dt) << " tout;\n"
    << "#define NPS_N " << n << "LL\n"
    << "#define NPS_G " << G << "\n"
    << "#define NPS_IN_PER_VEC " << 16 / (in_dt == NP_F32 ? 4 : 2) << "\n"
    << "#define NPS_OUT_PER_VEC " << 16 / (out_dt == NP_F32 ? 4 : 2) << "\n"
    << "__device__ __forceinline__ float chain(";
  for (int j = 0; j < n_inputs; ++j) s << (j ? ", " : "") << "const float* x" << j;
  s << ", int e, const float* kp) {\n  float v = 0.0f;\n";
  Pins pins;
  if (fast) {
    for (const std::string& l : emit_all(fold_fast(a), &pins)) s << "  " << l << "\n";
  } else {
    for (int i = 0; i < a.n_ops; ++i)
      s << "  " << op_line(a.kind[i], a.arg[i], a.c[i], fast) << "\n";
  }
  s << "  return v;\n}\n";
  // the pinned constants, once per thread
  std::string kp_decl = "  const float* const kp = nullptr;\n";
  if (!pins.v.empty()) {
    kp_decl = "  const float kp[" + std::to_string(pins.v.size()) + "] = {";
    for (size_t i = 0; i < pins.v.size(); ++i) kp_decl += (i ? ", np_pin(" : "np_pin(") + hexf(pins.v[i]) + ")";
    kp_decl += "};\n";
  }
  // vector kernel: one group of NPS_G elements per thread, dwordx4 accesses,
  // non-temporal stores; the < NPS_G leftover elements go to the first threads
  s << "extern \"C\" __global__ __launch_bounds__(256) void " << spec_name(a, n, false) << "(";
  for (int j = 0; j < n_inputs; ++j) s << "const tin* in" << j << ", ";
  s << "tout* out, long long n_rt) {\n"
    << "  const long long n = NPS_N ? NPS_N : n_rt;\n"
    << "  const long long ngroups = n / NPS_G;\n"
    << "  const long long g = (long long)blockIdx.x * 256 + threadIdx.x;\n"
    << kp_decl
    << "  if (g < ngroups) {\n";
  for (int j = 0; j < n_inputs; ++j) {
    s << "    float x" << j << "[NPS_G];\n"
      << "#pragma unroll\n"
      << "    for (int q = 0; q < NPS_G / NPS_IN_PER_VEC; ++q) {\n"
      << "      u32x4 raw = *(const u32x4*)(in" << j << " + g * NPS_G + q * NPS_IN_PER_VEC);\n"
      << "      tin t[NPS_IN_PER_VEC]; __builtin_memcpy(t, &raw, 16);\n"
      << "#pragma unroll\n"
      << "      for (int i = 0; i < NPS_IN_PER_VEC; ++i) x" << j
      << "[q * NPS_IN_PER_VEC + i] = (float)t[i];\n"
      << "    }\n";
  }
  s << "    tout o[NPS_G];\n"
    << "#pragma unroll\n"
    << "    for (int e = 0; e < NPS_G; ++e) o[e] = (tout)chain(";
  for (int j = 0; j < n_inputs; ++j) s << (j ? ", " : "") << "x" << j;
  s << ", e, kp);\n"
    << "#pragma unroll\n"
    << "    for (int q = 0; q < NPS_G / NPS_OUT_PER_VEC; ++q) {\n"
    << "      u32x4 raw; __builtin_memcpy(&raw, o + q * NPS_OUT_PER_VEC, 16);\n"
    << "      __builtin_nontemporal_store(raw, (u32x4*)(out + g * NPS_G + q * NPS_OUT_PER_VEC));\n"
    << "    }\n"
    << "  }\n"
    << "  const long long tail0 = ngroups * NPS_G;\n"
    << "  if (g < n - tail0) {\n"
    << "    const long long i = tail0 + g;\n";
  for (int j = 0; j < n_inputs; ++j) s << "    float x" << j << "[1] = {(float)in" << j << "[i]};\n";
  s << "    out[i] = (tout)chain(";
  for (int j = 0; j < n_inputs; ++j) s << (j ? ", " : "") << "x" << j;
  s << ", 0, kp);\n  }\n}\n";
  // scalar kernel: one element per thread (small n, where it fills the chip better)
  s << "extern \"C\" __global__ __launch_bounds__(256) void " << spec_name(a, n, true) << "(";
  for (int j = 0; j < n_inputs; ++j) s << "const tin* in" << j << ", ";
  s << "tout* out, long long n_rt) {\n"
    << "  const long long n = NPS_N ? NPS_N : n_rt;\n"
    << "  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;\n"
    << "  if (i >= n) return;\n"
    << kp_decl;
  for (int j = 0; j < n_inputs; ++j) s << "  float x" << j << "[1] = {(float)in" << j << "[i]};\n";
  s << "  out[i] = (tout)chain(";
  for (int j = 0; j < n_inputs; ++j) s << (j ? ", " : "") << "x" << j;
  s << ", 0, kp);\n}\n";
  if (tabulable(n_inputs, in_dt, out_dt)) {
    const std::string base = spec_name(a, n, false);
    // the table: out bits for every input bit pattern, by the chain code above
    s << "__device__ __attribute__((aligned(16))) unsigned short np_lut[65536];\n"
      << "extern \"C\" __global__ __launch_bounds__(256) void " << base << "_tab(void) {\n"
      << "  const int i = blockIdx.x * 256 + threadIdx.x;\n"
      << kp_decl
      << "  const unsigned short bits = (unsigned short)i;\n"
      << "  tin x; __builtin_memcpy(&x, &bits, 2);\n"
      << "  float x0[1] = {(float)x};\n"
      << "  const tout y = (tout)chain(x0, 0, kp);\n"
      << "  unsigned short yb; __builtin_memcpy(&yb, &y, 2);\n"
      << "  np_lut[i] = yb;\n"
      << "}\n";
    // the gather kernel: one 512-thread workgroup per CU stages the 128 KiB
    // table in LDS, then takes contiguous blocks of 2048 16-byte vectors (32
    // KiB), block b + i * grid on its i-th pass, four vectors per thread at
    // NT-vector spacing so every load and store instruction of a wave covers
    // 1 KiB in one piece. Loads and stores are non-temporal: a stream this long
    // cannot stay in the Infinity Cache between calls. (Each thread's vectors
    // one grid stride apart, the usual persistent loop, ran 6 % slower here.)
    s << "extern \"C\" __global__ __launch_bounds__(512) void " << base
      << "_lut(const tin* in0, tout* out, long long n_rt) {\n"
      << "  __shared__ __attribute__((aligned(16))) unsigned short lut[65536];\n"
      << "  const long long n = NPS_N ? NPS_N : n_rt;\n"
      << "  const long long nv = n / 8;\n"
      << "  const long long nblk = nv / 2048;\n"
      << "  const u32x4* src = reinterpret_cast<const u32x4*>(in0);\n"
      << "  u32x4* dst = reinterpret_cast<u32x4*>(out);\n"
      << "  const int t = threadIdx.x;\n"
      << "  for (int i = t; i < 8192; i += 512)\n"
      << "    reinterpret_cast<u32x4*>(lut)[i] = reinterpret_cast<const u32x4*>(np_lut)[i];\n"
      << "  __syncthreads();\n"
      << "  auto map = [&](u32x4 x) {\n"
      << "    u32x4 o;\n"
      << "#pragma unroll\n"
      << "    for (int j = 0; j < 4; ++j)\n"
      << "      o[j] = (unsigned)lut[x[j] & 0xffffu] | ((unsigned)lut[x[j] >> 16] << 16);\n"
      << "    return o;\n"
      << "  };\n"
      << "  u32x4 r[4];\n"
      << "  for (long long k = blockIdx.x; k < nblk; k += gridDim.x) {\n"
      << "    const long long v = k * 2048 + t;\n"
      << "#pragma unroll\n"
      << "    for (int u = 0; u < 4; ++u) r[u] = __builtin_nontemporal_load(src + v + u * 512);\n"
      << "#pragma unroll\n"
      << "    for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(map(r[u]), dst + v + u * 512);\n"
      << "  }\n"
      << "  // the vectors after the last whole block, then the elements after the last vector\n"
      << "  for (long long v = nblk * 2048 + (long long)blockIdx.x * 512 + t; v < nv;\n"
      << "       v += (long long)gridDim.x * 512)\n"
      << "    __builtin_nontemporal_store(map(__builtin_nontemporal_load(src + v)), dst + v);\n"
      << "  const long long e = nv * 8 + (long long)blockIdx.x * 512 + t;\n"
      << "  if (e < n) {\n"
      << "    unsigned short b; __builtin_memcpy(&b, in0 + e, 2);\n"
      << "    const unsigned short y = lut[b];\n"
      << "    __builtin_memcpy(out + e, &y, 2);\n"
      << "  }\n"
      << "}\n";
  }
  return s.str();
}

int rtc_prepare(const ChainArgs& a, int n_inputs, int in_dt, int out_dt, std::string* log) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    *log = "no device";
    return NP_EDEVICE;
  }
  const std::string key = spec_key(a, n_inputs, in_dt, out_dt, a.n, dev);
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_cache.count(key)) return NP_OK;
  }
  const std::string src = rtc_source(a, n_inputs, in_dt, out_dt, a.n);
  std::string opts;
  for (int i = 0; i < kNumOptions; ++i) opts += std::string(kOptions[i]) + " ";
  const size_t h = std::hash<std::string>()(src + "|gfx950|" + opts);
  // the same source compiled before (other n with identical text cannot occur:
  // n is part of the text) -- reuse its module
  {
    std::lock_guard<std::mutex> lk(g_mu);
    for (auto& kv : g_cache) {
      if (kv.second.src_hash == h && kv.second.dev == dev) {
        g_cache[key] = kv.second;
        return NP_OK;
      }
    }
  }
  // the code object: from the disk cache when one is configured and holds it,
  // else compiled (and then stored there)
  const std::string dir = cache_dir();
  const std::string ktext = dir.empty() ? std::string() : key_text(src);
  std::vector<char> code;
  bool from_disk = !dir.empty() && disk_load(dir, ktext, &code);
  if (!from_disk) {
    const int rc = compile(src, &code, log);
    if (rc) return rc;
    if (!dir.empty()) disk_store(dir, ktext, code);
  }
  Entry e;
  e.src_hash = h;
  e.dev = dev;
  {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        cus > 0)
      e.cus = cus;
  }
  auto load = [&]() {
    if (hipModuleLoadData(&e.mod, code.data()) == hipSuccess &&
        hipModuleGetFunction(&e.fn, e.mod, spec_name(a, a.n, false).c_str()) == hipSuccess &&
        hipModuleGetFunction(&e.fn_scalar, e.mod, spec_name(a, a.n, true).c_str()) == hipSuccess)
      return true;
    if (e.mod) (void)hipModuleUnload(e.mod);
    e.mod = nullptr;
    (void)hipGetLastError();
    return false;
  };
  bool loaded = load();
  if (!loaded && from_disk) {  // a cached object that does not load: compile it afresh
    g_disk_rejects.fetch_add(1);
    from_disk = false;
    const int rc = compile(src, &code, log);
    if (rc) return rc;
    disk_store(dir, ktext, code);
    loaded = load();
  }
  if (!loaded) {
    *log = "module load failed";
    return NP_ELAUNCH;
  }
  if (from_disk) g_disk_loads.fetch_add(1);
  if (tabulable(n_inputs, in_dt, out_dt)) {
    // fill the module's table once (65,536 threads), on a private stream
    // waited for here: prepare is the warm-up-time call; without a table the
    // chain is evaluated per element
    const std::string base = spec_name(a, a.n, false);
    hipFunction_t tab = nullptr, lut = nullptr;
    hipStream_t st = nullptr;
    if (hipModuleGetFunction(&tab, e.mod, (base + "_tab").c_str()) == hipSuccess &&
        hipModuleGetFunction(&lut, e.mod, (base + "_lut").c_str()) == hipSuccess &&
        hipStreamCreateWithFlags(&st, hipStreamNonBlocking) == hipSuccess) {
      if (hipModuleLaunchKernel(tab, 256, 1, 1, 256, 1, 1, 0, st, nullptr, nullptr) == hipSuccess &&
          hipStreamSynchronize(st) == hipSuccess)
        e.fn_lut = lut;
      (void)hipStreamDestroy(st);
    }
    (void)hipGetLastError();  // a failed table leaves the per-element kernels in use
  }
  std::lock_guard<std::mutex> lk(g_mu);
  // another thread may have prepared the same chain meanwhile: keep its entry
  // (launches may already use it) and release this module
  if (!g_cache.emplace(key, e).second) (void)hipModuleUnload(e.mod);
  return NP_OK;
}

bool rtc_launch(const ChainArgs& a, int n_inputs, int in_dt, int out_dt, hipStream_t s,
                hipError_t* err) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  const int G = (in_dt != NP_F32 || out_dt != NP_F32) ? 8 : 4;
  const int64_t ngroups = a.n / G;
  const bool scalar = ngroups < kMinVecGroups;
  hipFunction_t fn = nullptr;
  bool lut = false;
  int cus = 0;
  std::string key = spec_key(a, n_inputs, in_dt, out_dt, a.n, dev);
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_cache.empty()) return false;
    auto it = g_cache.find(key);
    if (it == g_cache.end()) {  // the same chain prepared for any n
      const int64_t zero = 0;
      key.replace(kKeyN, sizeof(zero), reinterpret_cast<const char*>(&zero), sizeof(zero));
      it = g_cache.find(key);
    }
    if (it == g_cache.end()) return false;
    lut = it->second.fn_lut != nullptr && a.n >= g_lut_min_n.load(std::memory_order_relaxed);
    fn = lut ? it->second.fn_lut : scalar ? it->second.fn_scalar : it->second.fn;
    cus = it->second.cus;
  }
  const int64_t work = scalar ? a.n : ngroups;
  int64_t blocks = (work + 255) / 256;
  if (blocks < 1) blocks = 1;
  unsigned threads = 256;
  if (lut) {  // one workgroup per CU (the table takes 128 KiB of its LDS)
    blocks = cus;
    threads = 512;
  }
  void* params[NP_MAX_INPUTS + 2];
  const void* ins[NP_MAX_INPUTS];
  void* out = a.out;
  long long n = a.n;
  for (int j = 0; j < n_inputs; ++j) {
    ins[j] = a.in[j];
    params[j] = &ins[j];
  }
  params[n_inputs] = &out;
  params[n_inputs + 1] = &n;
  *err = hipModuleLaunchKernel(fn, (unsigned)blocks, 1, 1, threads, 1, 1, 0, s, params, nullptr);
  return true;
}

void rtc_clear() {
  std::lock_guard<std::mutex> lk(g_mu);
  std::map<hipModule_t, bool> seen;
  for (auto& kv : g_cache) {
    if (kv.second.mod && !seen[kv.second.mod]) {
      seen[kv.second.mod] = true;
      (void)hipModuleUnload(kv.second.mod);
    }
  }
  g_cache.clear();
}

}  // namespace np

extern "C" int64_t np_chain_source(const np_op* ops, int n_ops, int n_inputs, np_dtype in_dt,
                                   np_dtype out_dt, int64_t n, char* buf, size_t len) {
  if (!ops || n_ops < 1 || n_ops > NP_MAX_OPS || n_inputs < 1 || n_inputs > NP_MAX_INPUTS ||
      n < 0)
    return NP_EINVAL;
  np::ChainArgs a{};
  a.n_ops = n_ops;
  for (int i = 0; i < n_ops; ++i) {
    if (ops[i].kind < NP_LOAD || ops[i].kind > NP_CAST_BF16) return NP_EINVAL;
    a.kind[i] = ops[i].kind;
    a.arg[i] = ops[i].arg;
    a.c[i] = ops[i].c;
  }
  const std::string src = np::rtc_source(a, n_inputs, in_dt, out_dt, n);
  if (buf && len > 0) {
    const size_t m = src.size() < len - 1 ? src.size() : len - 1;
    std::memcpy(buf, src.data(), m);
    buf[m] = '\0';
  }
  return (int64_t)src.size() + 1;
}

extern "C" int np_chain_compile(const np_op* ops, int n_ops, int n_inputs, np_dtype in_dt,
                                np_dtype out_dt, int64_t n, double* compile_ms,
                                size_t* code_bytes) {
  if (!ops || n_ops < 1 || n_ops > NP_MAX_OPS || n_inputs < 1 || n_inputs > NP_MAX_INPUTS ||
      n < 0)
    return NP_EINVAL;
  np::ChainArgs a{};
  a.n_ops = n_ops;
  for (int i = 0; i < n_ops; ++i) {
    if (ops[i].kind < NP_LOAD || ops[i].kind > NP_CAST_BF16) return NP_EINVAL;
    a.kind[i] = ops[i].kind;
    a.arg[i] = ops[i].arg;
    a.c[i] = ops[i].c;
  }
  std::vector<char> code;
  std::string log;
  const std::string src = np::rtc_source(a, n_inputs, in_dt, out_dt, n);
  const auto t0 = std::chrono::steady_clock::now();
  int rc = np::compile(src, &code, &log);
  const auto t1 = std::chrono::steady_clock::now();
  if (compile_ms) *compile_ms = std::chrono::duration<double, std::milli>(t1 - t0).count();
  if (code_bytes) *code_bytes = code.size();
  const std::string dir = np::cache_dir();
  if (rc == NP_OK && !dir.empty()) np::disk_store(dir, np::key_text(src), code);
  return rc;
}

extern "C" void np_chain_cache_stats(int64_t* loads, int64_t* stores, int64_t* rejects) {
  if (loads) *loads = np::g_disk_loads.load();
  if (stores) *stores = np::g_disk_stores.load();
  if (rejects) *rejects = np::g_disk_rejects.load();
}

extern "C" int64_t np_set_chain_table_min(int64_t n) {
  if (n < 0) return np::g_lut_min_n.load();
  return np::g_lut_min_n.exchange(n);
}
