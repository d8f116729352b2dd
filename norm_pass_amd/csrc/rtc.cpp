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
//  - section 6.3: no fast-math; section 6.4: modules live until np_shutdown.
#include "rtc.h"

#include <hip/hiprtc.h>

#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <functional>
#include <map>
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
//    multiply after it into its factor: e^b c 2^(x a log2 e)
//    (np_fast_exp_affine: v_exp_f32 of x·a·log2 e, times the factor);
//  - a cast that repeats the cast before it is dropped.
bool is_mul(int k) { return k == NP_MUL_C || k == NP_SCALE; }

std::string exp_affine(double a, double b, double factor) {
  const float c = (float)(a * 1.4426950408889634074);  // a log2(e)
  const float e = (float)(std::exp(b) * factor);
  return "v = np_fast_exp_affine(v, " + hexf(c) + ", " + hexf(e) + ");";
}

std::vector<std::string> fold_fast(const ChainArgs& a) {
  std::vector<std::string> out;
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
  while (i < n) {
    const int k = a.kind[i];
    if (is_mul(k) || k == NP_ADD_C || k == NP_EXP) {
      double m = 1.0, b = 0.0;
      int j = i;
      if (is_mul(k)) j = run(j, true, &m);
      if (j < n && a.kind[j] == NP_ADD_C) j = run(j, false, &b);
      if (!is_mul(k) && k == NP_ADD_C && j < n && is_mul(a.kind[j])) {
        // (x + b) m in front of an exp is x m + b m
        double m2 = 1.0;
        const int j2 = run(j, true, &m2);
        if (j2 < n && a.kind[j2] == NP_EXP) {
          double after = 1.0;
          const int j3 = run(j2 + 1, true, &after);
          out.push_back(exp_affine(m2, b * m2, after));
          i = j3;
          continue;
        }
      }
      if (j < n && a.kind[j] == NP_EXP) {
        double after = 1.0;
        const int j2 = run(j + 1, true, &after);
        out.push_back(exp_affine(m, b, after));
        i = j2;
        continue;
      }
      const bool has_mul = is_mul(k), has_add = a.kind[j - 1] == NP_ADD_C;
      if (has_mul && has_add)
        out.push_back("v = __builtin_fmaf(v, " + hexf((float)m) + ", " + hexf((float)b) + ");");
      else if (has_mul)
        out.push_back("v = v * " + hexf((float)m) + ";");
      else
        out.push_back("v = v + " + hexf((float)b) + ";");
      i = j;
      continue;
    }
    if ((k == NP_CAST_F16 || k == NP_CAST_BF16) && i > 0 && a.kind[i - 1] == k) {
      ++i;  // casting again to the same type changes nothing
      continue;
    }
    out.push_back(op_line(k, a.arg[i], a.c[i], true));
    ++i;
  }
  return out;
}

struct Entry {
  hipModule_t mod = nullptr;
  hipFunction_t fn = nullptr;         // vector kernel
  hipFunction_t fn_scalar = nullptr;  // one element per thread
  size_t src_hash = 0;
};

// Same threshold as the generic kernel: below it, one element per thread.
constexpr int64_t kMinVecGroups = 65536;

std::mutex g_mu;
std::map<std::string, Entry> g_cache;  // spec key -> loaded kernel

std::string spec_key(const ChainArgs& a, int n_inputs, int in_dt, int out_dt, int64_t n,
                     int dev) {
  std::ostringstream k;
  k << dev << '|' << in_dt << '|' << out_dt << '|' << n_inputs << '|' << n << '|';
  for (int i = 0; i < a.n_ops; ++i) {
    uint32_t cb;
    std::memcpy(&cb, &a.c[i], 4);
    k << a.kind[i] << ',' << a.arg[i] << ',' << cb << ';';
  }
  return k.str();
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

}  // namespace

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
  s << ", int e) {\n  float v = 0.0f;\n";
  if (fast) {
    for (const std::string& l : fold_fast(a)) s << "  " << l << "\n";
  } else {
    for (int i = 0; i < a.n_ops; ++i)
      s << "  " << op_line(a.kind[i], a.arg[i], a.c[i], fast) << "\n";
  }
  s << "  return v;\n}\n";
  // vector kernel: one group of NPS_G elements per thread, dwordx4 accesses,
  // non-temporal stores; the < NPS_G leftover elements go to the first threads
  s << "extern \"C\" __global__ __launch_bounds__(256) void np_chain_spec(";
  for (int j = 0; j < n_inputs; ++j) s << "const tin* in" << j << ", ";
  s << "tout* out, long long n_rt) {\n"
    << "  const long long n = NPS_N ? NPS_N : n_rt;\n"
    << "  const long long ngroups = n / NPS_G;\n"
    << "  const long long g = (long long)blockIdx.x * 256 + threadIdx.x;\n"
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
  s << ", e);\n"
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
  s << ", 0);\n  }\n}\n";
  // scalar kernel: one element per thread (small n, where it fills the chip better)
  s << "extern \"C\" __global__ __launch_bounds__(256) void np_chain_spec_scalar(";
  for (int j = 0; j < n_inputs; ++j) s << "const tin* in" << j << ", ";
  s << "tout* out, long long n_rt) {\n"
    << "  const long long n = NPS_N ? NPS_N : n_rt;\n"
    << "  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;\n"
    << "  if (i >= n) return;\n";
  for (int j = 0; j < n_inputs; ++j) s << "  float x" << j << "[1] = {(float)in" << j << "[i]};\n";
  s << "  out[i] = (tout)chain(";
  for (int j = 0; j < n_inputs; ++j) s << (j ? ", " : "") << "x" << j;
  s << ", 0);\n}\n";
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
      if (kv.second.src_hash == h && kv.first.rfind(std::to_string(dev) + "|", 0) == 0) {
        g_cache[key] = kv.second;
        return NP_OK;
      }
    }
  }
  std::vector<char> code;
  int rc = compile(src, &code, log);
  if (rc) return rc;
  Entry e;
  e.src_hash = h;
  if (hipModuleLoadData(&e.mod, code.data()) != hipSuccess ||
      hipModuleGetFunction(&e.fn, e.mod, "np_chain_spec") != hipSuccess ||
      hipModuleGetFunction(&e.fn_scalar, e.mod, "np_chain_spec_scalar") != hipSuccess) {
    *log = "module load failed";
    if (e.mod) (void)hipModuleUnload(e.mod);
    return NP_ELAUNCH;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  g_cache[key] = e;
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
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_cache.empty()) return false;
    auto it = g_cache.find(spec_key(a, n_inputs, in_dt, out_dt, a.n, dev));
    if (it == g_cache.end()) it = g_cache.find(spec_key(a, n_inputs, in_dt, out_dt, 0, dev));
    if (it == g_cache.end()) return false;
    fn = scalar ? it->second.fn_scalar : it->second.fn;
  }
  const int64_t work = scalar ? a.n : ngroups;
  int64_t blocks = (work + 255) / 256;
  if (blocks < 1) blocks = 1;
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
  *err = hipModuleLaunchKernel(fn, (unsigned)blocks, 1, 1, 256, 1, 1, 0, s, params, nullptr);
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
  const auto t0 = std::chrono::steady_clock::now();
  int rc = np::compile(np::rtc_source(a, n_inputs, in_dt, out_dt, n), &code, &log);
  const auto t1 = std::chrono::steady_clock::now();
  if (compile_ms) *compile_ms = std::chrono::duration<double, std::milli>(t1 - t0).count();
  if (code_bytes) *code_bytes = code.size();
  return rc;
}
