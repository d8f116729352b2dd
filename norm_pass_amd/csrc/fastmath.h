// Transcendentals for chains whose output is fp16: a few fp32 ulps of error
// (the fp16 output keeps 11 significand bits), built on the hardware's base-2
// exponential (v_exp_f32) and reciprocal (v_rcp_f32). This file is compiled
// into the library and also pasted verbatim into runtime-specialised kernels,
// so it uses only compiler builtins.
//
// exp(x) = 2^(x log2 e): the argument is clamped to [-200, 200] (exp is 0 or
// inf in binary32 beyond that), the product x * log2(e) is split into its
// rounded value t and the rounding error err (an FMA recovers it exactly, a
// second FMA adds the error of the binary32 constant: Cody and Waite's
// argument splitting), v_exp_f32 evaluates 2^t, and the result is scaled by
// 2^err ~ 1 + err ln 2 (rounded to binary32, <= 0.5 ulp). Results below 2^-126
// are flushed to zero by the hardware exponential; an fp16 output cannot hold
// them anyway. Error <= 2 ulp.
// sigmoid(x) = 1 / (1 + exp(-x)) with the hardware reciprocal. Error <= 4 ulp.
// tanh(x): for |x| < 0.625 the odd polynomial x + x^3 P(x^2), P of degree 4
// fitted to minimise the relative error on [0, 0.625] (a Lawson-weighted least
// squares fit; 0.07 ulp approximation error); otherwise 1 - 2 / (1 + e^(2|x|)),
// whose cancellation is at most 3.7x there. Error <= 2 ulp.
#pragma once

#define NP_FM_INLINE __device__ __forceinline__

NP_FM_INLINE float np_fast_exp(float x) {
  const float kLog2e = 1.44269502162933349609375f;      // binary32 nearest to log2(e)
  const float kLog2eLo = 1.925963033500011e-08f;        // log2(e) - kLog2e
  const float kLn2 = 0.693147180559945309f;
  const float xc = __builtin_amdgcn_fmed3f(x, -200.0f, 200.0f);
  const float t = xc * kLog2e;
  const float err = __builtin_fmaf(xc, kLog2eLo, __builtin_fmaf(xc, kLog2e, -t));
  return __builtin_amdgcn_exp2f(t) * __builtin_fmaf(err, kLn2, 1.0f);
}

// e * exp(x a) for constants c = a log2(e) and e (an affine map before an exp
// and a factor after it, folded into the exp by the runtime specialiser):
// 2^(x c) by v_exp_f32, times e (the specialiser uses it for e = 0 only; the
// shifted form below serves every other factor). Without the argument splitting of
// np_fast_exp the rounding of x c adds |x c| / 2 ulp of relative error (the
// specialiser's fp16-output chains keep |x c| small; at |x c| = 16 this is 2^-20,
// 1/512 of an fp16 ulp). Infinite or NaN arguments give inf, 0 or NaN as exp
// does; 2^(x c) below 2^-126 is flushed to zero.
NP_FM_INLINE float np_fast_exp_affine(float x, float c, float e) {
  return __builtin_amdgcn_exp2f(x * c) * e;
}

// |e| exp(x a) for a factor e != 0, as 2^(x c + d) with d = log2 |e| (the
// caller negates the result when e < 0): one FMA forms the exponent, so the
// factor costs no multiply. The FMA's rounding adds |x c + d| / 2 ulp of
// relative error, as the product x c does above; a result the factor brings
// back into range is not lost to an overflow or flush of 2^(x c) first.
NP_FM_INLINE float np_fast_exp_shifted(float x, float c, float d) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(x, c, d));
}

NP_FM_INLINE float np_fast_sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.0f + np_fast_exp(-x));
}

// sigmoid(x a + b) = 1 / (1 + e^-b 2^(x c)) for constants c = -a log2(e) and
// e = e^-b (an affine map folded into the sigmoid by the runtime specialiser).
// The rounding of x c adds |x c| / 2 ulp to the exponential's relative error,
// and the sigmoid's relative error is at most that of the exponential. An
// overflowing 2^(x c) gives 1 / inf = 0; an underflowing one gives 1.
NP_FM_INLINE float np_fast_sigmoid_affine(float x, float c, float e) {
  return __builtin_amdgcn_rcpf(__builtin_fmaf(__builtin_amdgcn_exp2f(x * c), e, 1.0f));
}

// tanh for |x| < 0.625: the odd polynomial evaluated on x itself. Every step is
// symmetric under a sign change, so this equals the |x| form with the sign put
// back, except that -0 gives +0.
#define NP_TANH_P4 -0.005704987328499556f  // leading coefficient of P

// k4: P's leading coefficient, passed in so that a caller can keep it in a
// register (two constants in one FMA need one of them in a vector register)
NP_FM_INLINE float np_fast_tanh_poly_k(float x, float k4) {
  const float z = x * x;
  float p = __builtin_fmaf(k4, z, 0.0206390880048275f);
  p = __builtin_fmaf(p, z, -0.05373971536755562f);
  p = __builtin_fmaf(p, z, 0.13331441581249237f);
  p = __builtin_fmaf(p, z, -0.3333328068256378f);
  return __builtin_fmaf(x * z, p, x);
}

NP_FM_INLINE float np_fast_tanh_poly(float x) { return np_fast_tanh_poly_k(x, NP_TANH_P4); }

// tanh for x >= 0.625 (and +inf): 1 - 2 / (1 + e^(2x)), e^(2x) = 2^(2x log2 e).
NP_FM_INLINE float np_fast_tanh_exp_pos(float x) {
  const float e = __builtin_amdgcn_exp2f(x * 2.88539008177792681f);
  return __builtin_fmaf(-2.0f, __builtin_amdgcn_rcpf(1.0f + e), 1.0f);
}

// tanh for x <= -0.625 (and -inf): 2 / (1 + e^(-2x)) - 1, the negation of the
// form above at -x (the same bits with the sign flipped).
NP_FM_INLINE float np_fast_tanh_exp_neg(float x) {
  const float e = __builtin_amdgcn_exp2f(x * -2.88539008177792681f);
  return __builtin_fmaf(2.0f, __builtin_amdgcn_rcpf(1.0f + e), -1.0f);
}

NP_FM_INLINE float np_fast_tanh_k(float x, float k4) {
  const float a = __builtin_fabsf(x);
  float r;
  if (a < 0.625f)  // a branch, not a select: a wave whose lanes agree runs one side
    r = np_fast_tanh_poly_k(a, k4);
  else
    r = np_fast_tanh_exp_pos(a);
  return __builtin_copysignf(r, x);
}

NP_FM_INLINE float np_fast_tanh(float x) { return np_fast_tanh_k(x, NP_TANH_P4); }

// tanh when the sign of x is known (x >= 0, x <= 0): one branch, no sign
// handling. NaN takes the exponential side and stays NaN.
NP_FM_INLINE float np_fast_tanh_pos_k(float x, float k4) {
  float r;
  if (x < 0.625f)
    r = np_fast_tanh_poly_k(x, k4);
  else
    r = np_fast_tanh_exp_pos(x);
  return r;
}

NP_FM_INLINE float np_fast_tanh_neg_k(float x, float k4) {
  float r;
  if (x > -0.625f)
    r = np_fast_tanh_poly_k(x, k4);
  else
    r = np_fast_tanh_exp_neg(x);
  return r;
}

NP_FM_INLINE float np_fast_tanh_pos(float x) { return np_fast_tanh_pos_k(x, NP_TANH_P4); }
NP_FM_INLINE float np_fast_tanh_neg(float x) { return np_fast_tanh_neg_k(x, NP_TANH_P4); }

// Casts to fp16 merged with the affine ops around them (fp16-output chains, by
// the runtime specialiser), on gfx950's mixed-precision FMAs:
// round_f16(v m + b) in one v_fma_mixlo_f16 (a single rounding of the fused
// product-sum, where a separate fp32 op and cast round twice: both are within
// half an fp16 ulp plus half an fp32 ulp of v m + b), and (float)h m + b in
// one v_fma_mix_f32 with the f16 operand taken as is (exact widening, then one
// fp32 rounding, as a multiply or FMA after the cast). A zero result may come
// out +0 where the separate ops give -0; the value is the same. The constants
// travel in scalar registers.
NP_FM_INLINE _Float16 np_fma_to_f16(float v, float m, float b) {
  _Float16 r;
  asm("v_fma_mixlo_f16 %0, %1, %2, %3" : "=v"(r) : "v"(v), "s"(m), "v"(b));
  return r;
}

NP_FM_INLINE _Float16 np_mul_to_f16(float v, float m) {
  _Float16 r;
  asm("v_fma_mixlo_f16 %0, %1, %2, 0" : "=v"(r) : "v"(v), "s"(m));
  return r;
}

NP_FM_INLINE _Float16 np_add_to_f16(float v, float b) {
  _Float16 r;
  asm("v_fma_mixlo_f16 %0, %1, 1.0, %2" : "=v"(r) : "v"(v), "s"(b));
  return r;
}

NP_FM_INLINE float np_fma_from_f16(_Float16 h, float m, float b) {
  float r;
  asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "s"(m), "v"(b));
  return r;
}

NP_FM_INLINE float np_mul_from_f16(_Float16 h, float m) {
  float r;
  asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "s"(m));
  return r;
}

// An opaque copy of x in a vector register. Generated kernels pin the
// constants an instruction cannot take as a literal (gfx9 allows one literal or
// scalar operand per instruction) once per thread: left to itself, the compiler
// rematerialises them with a move for every element it unrolls.
NP_FM_INLINE float np_pin(float x) {
  asm("" : "+v"(x));
  return x;
}
