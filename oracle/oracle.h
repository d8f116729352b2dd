/*
 * CPU oracle for the fused-chain library -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the bench's CPU-baseline leg may load
 * this library. It is a plain, slow, scalar evaluation of what each fused
 * chain computes, written from the definitions, in double precision (long
 * double for row sums), with one rounding per stored output (plus the
 * roundings that are part of a definition: explicit cast nodes, the stored
 * residual sum h of the residual-add + RMSNorm chain, and the fp32 RoPE angle).
 * It has its own IEEE binary16 / bfloat16 / binary32 converters written from
 * the bit layouts. It shares no code with the GPU library.
 *
 * Every function returns 0 on success and -1 on an invalid argument.
 *
 * dtype codes: 0 = fp32, 1 = fp16 (IEEE binary16), 2 = bf16 (bfloat16).
 * Half-precision tensors are arrays of uint16 bit patterns.
 *
 * Error bounds ("bound" outputs). For each element the oracle can also return
 * the exact (unrounded, double) value of the definition and a running bound
 * beta on how far an fp32 evaluation of the same definition may land from it
 * (first-order propagation: beta_out = sup|f'| * beta_in + kappa * 2^-24 *
 * |f(v)|, kappa = 2 for +, x and kappa = 8 for exp / sigmoid / tanh / sin /
 * cos; a cast node resets beta to 0 unless [v-beta, v+beta] straddles a
 * rounding boundary of the cast format, in which case one ulp of that format
 * is added). Tests use it only to recognise ill-conditioned elements
 * (cancellation, a rounding decided by the last bit), whose count they report.
 */
#ifndef NORM_PASS_ORACLE_H
#define NORM_PASS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* --- converters (exposed so tests can pin them against library routines) */
double oracle_f16_to_double(uint16_t h);
uint16_t oracle_double_to_f16(double x);    /* round to nearest even */
double oracle_bf16_to_double(uint16_t b);
uint16_t oracle_double_to_bf16(double x);   /* round to nearest even */
float oracle_double_to_f32(double x);       /* round to nearest even */
void oracle_round_array(const double* x, int64_t n, int dt, void* out);

/*
 * Elementwise chain over a running value (DeepJIT write-up,
 * hotelren.com/news/5350627, sections 3.2-4.2: one value per element, a fixed
 * sequence of elementwise ops, inputs read once, output written once).
 *
 * ops: kinds[i], args[i] (input index for load/add_in/mul_in), consts[i].
 * kinds: 0 load(k) 1 add_in(k) 2 mul_in(k) 3 add_c 4 mul_c 5 scale 6 relu
 *        7 sigmoid 8 exp 9 tanh 10 cast_f16 11 cast_bf16.
 * inputs: n_inputs pointers to n elements of in_dt. out: n elements of out_dt.
 * eager = 0: fused semantics (exact intermediates, rounding only at cast
 *            nodes and at the output). The running value has the range of
 *            binary32 (the write-up's kernels hold it in a float register):
 *            a value beyond it becomes +-inf.
 * eager = 1: unfused semantics: every op stores its result in out_dt, as a
 *            chain of separate kernels with that storage type does.
 * exact / bound: optional (may be NULL) [n] doubles.
 */
int oracle_chain(const int32_t* kinds, const int32_t* args, const float* consts, int n_ops,
                 const void* const* inputs, int n_inputs, int in_dt, void* out, int out_dt,
                 int64_t n, int eager, double* exact, double* bound);

/*
 * YOLO-style detection-head decode (DeepJIT write-up, sections 1.1 and 5.2:
 * the sigmoid / exp / mul / add / slice / concat / cast tail of a detector).
 * levels[l]: [batch, n_anchors*n_ch, H[l], W[l]] of in_dt, channel a*n_ch+k.
 * anchors: [n_levels][n_anchors][2] (w, h) in pixels. out: fp32
 * [batch, sum_l n_anchors*H[l]*W[l], n_ch], rows ordered level, anchor, y, x.
 *   out[.,0] = (sigmoid(t0) + x) * stride   out[.,1] = (sigmoid(t1) + y) * stride
 *   out[.,2] = exp(t2) * anchor_w           out[.,3] = exp(t3) * anchor_h
 *   out[.,k] = sigmoid(tk), k >= 4
 * eager = 1: every step stores in_dt (the 23-kernel unfused tail), the final
 * concat + cast to fp32 is exact.
 */
int oracle_det_decode(const void* const* levels, int n_levels, const int32_t* H,
                      const int32_t* W, const float* strides, const float* anchors,
                      int n_anchors, int n_ch, int batch, int in_dt, float* out, int eager);

/*
 * Residual-add + RMSNorm (TeleTron write-up, 2kiu.com/news/5927820,
 * sections 3.3 and 4.2): h = x + r (stored, rounded to dt),
 * out = h / sqrt(mean(h^2) + eps) * w, row-major [rows, cols].
 * r == NULL: h = x. w == NULL: weight 1. h_out may be NULL.
 * eager = 1: the six-kernel unfused form (add; square; row mean; +eps and
 * reciprocal square root; multiply by rstd; multiply by w), each result
 * stored in dt (the row statistics as [rows] tensors of dt).
 * exact: optional [rows, cols] unrounded out values.
 */
int oracle_add_rmsnorm(const void* x, const void* r, const void* w, void* h_out, void* out,
                       int64_t rows, int64_t cols, float eps, int dt, int eager, double* exact);

/*
 * Residual-add + LayerNorm (DeepJIT write-up, section 4.3: one block per row,
 * mean and variance of the row, normalise, affine gamma / beta; the runtime
 * page "CUDA算子与AI运行时", section 4.1, states the same definition):
 * h = x + r (stored, rounded to dt), mu = mean(h), var = mean((h - mu)^2)
 * (population variance), out = (h - mu) / sqrt(var + eps) * gamma + beta.
 * r / gamma / beta / h_out may be NULL (no residual, gamma 1, beta 0, h not
 * stored). eager = 1: the nine-kernel unfused form (add; row mean; subtract
 * the mean; square; row mean; +eps and 1/sqrt; multiply by rstd; multiply by
 * gamma; add beta), each result stored in dt.
 */
int oracle_add_layernorm(const void* x, const void* r, const void* gamma, const void* beta,
                         void* h_out, void* out, int64_t rows, int64_t cols, float eps, int dt,
                         int eager, double* exact);

/*
 * QKV split + rotate-half RoPE + Q scale (TeleTron write-up, section 3.1: the
 * QKV projection epilogue of multi-head split, rotary position encoding and
 * scaling). qkv: [T, 3, n_heads, head_dim]; q, k, v: [n_heads, T, head_dim].
 * inv_i = fp32(base^(-2i/head_dim)), theta = fp32(fp32(pos) * inv_i),
 * o[i] = u cos - w sin, o[i+half] = w cos + u sin for (u, w) = (x[i], x[i+half]);
 * Q = o * q_scale, K = o, V = copy. positions == NULL: pos = t.
 * eager = 1: split, rope-q, rope-k, scale-q as separate stores in dt.
 * exact_* / bound_*: optional [n_heads, T, head_dim].
 */
int oracle_qkv_rope(const void* qkv, void* q, void* k, void* v, int64_t T, int n_heads,
                    int head_dim, const int32_t* positions, float base, float q_scale, int dt,
                    int eager, double* exact_q, double* exact_k, double* bound_q,
                    double* bound_k);

/* fp32 inverse-frequency table inv_i = fp32(base^(-2i/head_dim)), i < head_dim/2 */
int oracle_rope_inv_freq(float base, int head_dim, float* inv);

/*
 * RMSNorm + linear + scale (TeleTron write-up, 2kiu.com/news/5927820, section
 * 4.2: the row's RMS scale factor is computed inside the kernel and used
 * directly in the linear layer's accumulation, so no normalised tensor is
 * stored; section 3.1: a norm followed by a projection). x [M, K], w_norm [K]
 * (NULL: weight 1), Wt [N, K] (the linear weight with K contiguous: out = y
 * Wt^T), bias [N] (NULL: 0), out [M, N], all of dt:
 *   rstd_m = 1 / sqrt(mean_k x_mk^2 + eps)
 *   a_mk   = fp32(x_mk * w_k)           (the section's kernel keeps the
 *                                        weighted input in an fp32 array; for
 *                                        16-bit dt the product is exact there,
 *                                        so a_mk is x_mk * w_k itself)
 *   out_mn = round_dt(scale * (rstd_m * sum_k a_mk * Wt_nk + bias_n))
 * The mean square is taken of x (RMSNorm's definition), not of x * w as the
 * section's listing squares it; the two agree when w = 1.
 * eager = 1: the unfused form, three stored steps: y = round_dt(x rstd w);
 * z = round_dt(sum_k y_mk Wt_nk + bias_n); out = round_dt(scale * z).
 * exact: optional [M, N] unrounded values. cond: optional [M, N]
 * |scale| * rstd_m * sum_k |a_mk Wt_nk| (the size of the dot product's terms,
 * which bounds what a different summation order can change).
 */
int oracle_rmsnorm_linear(const void* x, const void* w_norm, const void* Wt, const void* bias,
                          void* out, int64_t M, int64_t N, int64_t K, float eps, float scale,
                          int dt, int eager, double* exact, double* cond);

/*
 * ChannelShuffle (runtime page "CUDA算子与AI运行时", gtnt.cn/news/145880,
 * section 2: the channels of an [N, C, H, W] tensor viewed as [groups,
 * C/groups], the two axes swapped, viewed back as C channels). Output channel
 * i*groups + g holds input channel g*(C/groups) + i, for g < groups,
 * i < C/groups. layout 0 = NCHW, 1 = NHWC ([N, H, W, C], the same channel
 * permutation applied to each pixel). Elements are elem_bytes (1..16) bytes,
 * copied bit for bit. Returns -1 unless groups divides C.
 */
int oracle_channel_shuffle(const void* in, void* out, int64_t N, int64_t C, int64_t H,
                           int64_t W, int64_t groups, int layout, int elem_bytes);

/*
 * Batched transpose of the middle two axes (the strided transpose the same
 * section describes): in [B, R, S, E] -> out [B, S, R, E], i.e.
 * out[b][s][r][e] = in[b][r][s][e], elements of elem_bytes (1..16) bytes.
 */
int oracle_transpose021(const void* in, void* out, int64_t B, int64_t R, int64_t S, int64_t E,
                        int elem_bytes);

#ifdef __cplusplus
}
#endif
#endif
