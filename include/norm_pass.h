/*
 * norm_pass_amd -- single-pass fused kernels for chains of small memory-bound
 * operators on AMD Instinct MI355X (gfx950).
 *
 * The problem (DeepJIT write-up, hotelren.com/news/5350627, section 1.1; the
 * NaiveRT write-up, zhaixingw.cn/coding/291.html, "the 75% that fusion
 * saves"): a chain of N small elementwise / normalisation / layout operators,
 * run as N kernels, pays N launches and N full read/write round trips of its
 * tensors through HBM. Each call below runs the whole chain as ONE kernel that
 * reads each input from HBM once and writes each output once. The unfused_*
 * calls run the same chains as one kernel per operator (the N-launch
 * baseline the fused calls are measured against).
 *
 * Calling convention (the C-ABI operator contract of the page
 * "CUDA算子与AI运行时：从内存对齐到stream调度的落地实践", gtnt.cn/news/145880,
 * sections 4.1 and 4.3, and its stream advice in sections 2.2 and 5.2):
 *  - plain pointers and sizes; no C++ types or exceptions cross this boundary;
 *  - every call returns an int status: NP_OK (0) on success, a negative code on
 *    failure, with a thread-local message from np_last_error();
 *  - every call enqueues its kernel(s) on the caller's stream and returns
 *    without synchronising; 0 means the legacy null stream (allowed, but it
 *    serialises with other streams); a fault during execution surfaces at the
 *    caller's next synchronisation;
 *  - all device buffers belong to the caller and must stay alive until the
 *    stream work completes (DeepJIT write-up, section 6.5); the library
 *    allocates no device memory; host arrays (ops, sizes, strides, anchors) are
 *    read during the call only;
 *  - pointers need not be aligned: a buffer that is not 16-byte aligned, or a
 *    size that is not a multiple of the 16-byte vector width, takes a scalar
 *    path instead of an error (DeepJIT write-up, sections 4.2 and 6.5);
 *  - an output may alias an input exactly (same pointer, same shape) for the
 *    elementwise and norm calls; partial overlap is undefined; the QKV and
 *    detection calls forbid aliasing;
 *  - the first call on a device checks that it is a gfx950 GPU (NP_EDEVICE
 *    otherwise); argument checks run before any HIP call.
 * Floating point: fp16 / bf16 data are computed in fp32 and rounded once per
 * stored value, to nearest even (TeleTron write-up, 2kiu.com/news/5927820,
 * section 3.4: element-wise work in high precision).
 */
#ifndef NORM_PASS_H
#define NORM_PASS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NP_VERSION 1

/* Status codes. The runtime page's host function (section 4.3) returns 0 on
 * success and -1 when the launch reports an error (it checks the last runtime
 * error after the launch and never synchronises the device); these codes keep
 * 0 and -1 and split the other failures by cause. */
#define NP_OK 0
#define NP_EINVAL (-1)   /* invalid argument (nothing was launched) */
#define NP_ELAUNCH (-3)  /* a HIP call or kernel launch failed */
#define NP_ECOMPILE (-4) /* runtime specialisation failed (generic kernel stays in use) */
#define NP_EDEVICE (-5)  /* no device, or not a gfx950 device */

typedef enum { NP_F32 = 0, NP_F16 = 1, NP_BF16 = 2 } np_dtype;

/* Elementwise chain ops (DeepJIT write-up, sections 4.1-4.2). The chain keeps one
 * running fp32 value per element. */
typedef enum {
  NP_LOAD = 0,      /* v = input[arg][i]                         */
  NP_ADD_IN = 1,    /* v = v + input[arg][i]                     */
  NP_MUL_IN = 2,    /* v = v * input[arg][i]                     */
  NP_ADD_C = 3,     /* v = v + c                                 */
  NP_MUL_C = 4,     /* v = v * c                                 */
  NP_SCALE = 5,     /* v = v * c (same as NP_MUL_C)              */
  NP_RELU = 6,      /* v = v > 0 ? v : 0 (never -0; NaN -> 0)    */
  NP_SIGMOID = 7,   /* v = 1 / (1 + exp(-v))                     */
  NP_EXP = 8,       /* v = exp(v)                                */
  NP_TANH = 9,      /* v = tanh(v)                               */
  NP_CAST_F16 = 10, /* v = fp16(v), round to nearest even        */
  NP_CAST_BF16 = 11 /* v = bf16(v), round to nearest even        */
} np_op_kind;

typedef struct {
  int32_t kind; /* np_op_kind */
  int32_t arg;  /* input index for NP_LOAD / NP_ADD_IN / NP_MUL_IN, else 0 */
  float c;      /* constant for NP_ADD_C / NP_MUL_C / NP_SCALE, else 0 */
} np_op;

#define NP_MAX_OPS 32
#define NP_MAX_INPUTS 4

/* ---------------------------------------------------------------- helpers */

/* Make `device` current through its primary context and check that it is a
 * gfx950 GPU (DeepJIT write-up, section 3.2: before loading runtime-compiled
 * modules, retain the device's primary context and make it current, so the
 * library shares the framework's context instead of creating its own; in HIP
 * hipSetDevice does both). Optional: the first call on a device does the check
 * lazily. Returns NP_EDEVICE if the device is missing or not gfx950. */
int np_init(int device);

/* Message for the last failing call on this thread ("" if none): the text the
 * runtime page's host function prints with the runtime's error string
 * (section 4.3), kept per thread for the caller to read instead. The pointer
 * stays valid until the next call on this thread. */
const char* np_last_error(void);

/* NP_VERSION of the built library, for a caller to check the ABI it was
 * compiled against at run time (the runtime page, section 4.4: the host
 * runtime's version decides what an operator library must provide). */
int np_version(void);

/* Release runtime-compiled modules. Every stream that ran a specialised chain
 * must have been synchronised first (DeepJIT write-up, section 6.4: unloading a
 * module with work still queued faults). Safe to call more than once. */
void np_shutdown(void);

/* Generate and compile (without loading) the specialised kernel source that
 * fuse_chain_prepare would build for this chain; reports the compile time in
 * milliseconds and the code-object size. Needs no GPU (the DeepJIT write-up,
 * sections 3.3 and 6.2, quotes tens to hundreds of ms per runtime compile).
 * Always compiles; when NP_CACHE_DIR is set the code object is also stored in
 * the disk cache (see fuse_chain_prepare), so a machine without a GPU can fill
 * the cache ahead of time. Returns NP_OK, NP_EINVAL or NP_ECOMPILE.
 * compile_ms / code_bytes may be NULL. */
int np_chain_compile(const np_op* ops, int n_ops, int n_inputs, np_dtype in_dt, np_dtype out_dt,
                     int64_t n, double* compile_ms, size_t* code_bytes);

/* Counters of the disk cache of specialised code objects since the process
 * started (DeepJIT write-up, section 6.2): loads = fuse_chain_prepare found a
 * valid file and skipped compiling; stores = files written (by prepare or
 * np_chain_compile); rejects = files present but unusable (another key, a
 * truncated file, or a code object the runtime would not load), each followed
 * by a compile. Any pointer may be NULL. */
void np_chain_cache_stats(int64_t* loads, int64_t* stores, int64_t* rejects);

/* Write the generated kernel source for a chain (what fuse_chain_prepare
 * compiles) into buf (NUL-terminated, truncated to len); returns the full size
 * including the NUL, or NP_EINVAL. The DeepJIT write-up, section 5.2, logs each
 * generated kernel while debugging; this is that hook. */
int64_t np_chain_source(const np_op* ops, int n_ops, int n_inputs, np_dtype in_dt,
                        np_dtype out_dt, int64_t n, char* buf, size_t len);

/* --------------------------------------------------------- fused calls */

/*
 * fuse_chain: one elementwise chain in one kernel (DeepJIT write-up, sections
 * 3.2-4.2: fused add -> relu -> scale, the fused multi-input chain and its
 * 16-byte vector form). ops[0] must be NP_LOAD. inputs: n_inputs (1..4) dense
 * 1-D device arrays of n elements of in_dt, no broadcasting. out: n elements of
 * out_dt. The running value is fp32; it is rounded only at NP_CAST_* ops and
 * once at the store. n == 0 returns NP_OK without a launch. Uses a runtime
 * specialisation prepared by fuse_chain_prepare for this exact op list, dtypes
 * and n when one exists, else the precompiled generic kernel; never compiles.
 * Errors: NP_EINVAL for n_ops outside 1..NP_MAX_OPS, an unknown op, an input
 * index >= n_inputs, a NULL pointer, n < 0 or n >= 2^40.
 */
int fuse_chain(const np_op* ops, int n_ops, const void* const* inputs, int n_inputs,
               np_dtype in_dt, void* out, np_dtype out_dt, int64_t n, hipStream_t stream);

/*
 * fuse_chain_prepare: specialise a chain at warm-up time (DeepJIT write-up,
 * sections 3.1 and 3.3: generate source with the sizes, vector width and op list
 * as constants, compile at run time, cache the module under a hash of source,
 * architecture and options). n_or_0 == 0 prepares a kernel for any n. Compiles
 * with hipRTC for gfx950 on the current device; cached per process. Returns
 * NP_ECOMPILE (the generic kernel remains in use) if compilation fails, and
 * NP_OK without compiling when NP_DISABLE_RTC=1 is set in the environment.
 * Disk cache (section 6.2, the cache level that survives a restart): when the
 * environment variable NP_CACHE_DIR names a directory (created if missing), the
 * code object is looked up there first, by the exact text of hipRTC's version,
 * the options and the generated source, and written there after a compile
 * (a temporary file renamed into place, safe across processes). Unset or
 * empty: no disk cache. The library never writes files otherwise.
 */
int fuse_chain_prepare(const np_op* ops, int n_ops, int n_inputs, np_dtype in_dt,
                       np_dtype out_dt, int64_t n_or_0);

/*
 * Tabulated chains. A chain over a single fp16 / bf16 input with an fp16 /
 * bf16 output is a function of the 65,536 input bit patterns: the specialised
 * module then also holds that function as a table, filled once by
 * fuse_chain_prepare with the module's own chain code (a launch on a private
 * stream that prepare waits for), and fuse_chain streams the input through the
 * table -- one gather per element from a copy staged in LDS -- once n reaches
 * a threshold (default 2^22; below it staging the 128 KiB table on every CU
 * costs more than evaluating the chain). The outputs are the same bits as the
 * per-element kernel's. np_set_chain_table_min sets the threshold for later
 * calls (INT64_MAX: never use the table) and returns the previous value; a
 * negative n only returns the current one. This is a specialisation detail,
 * not a separate operation (the DeepJIT write-up, section 3.3: constants
 * folded into the generated code at warm-up time, here the whole function).
 */
int64_t np_set_chain_table_min(int64_t n);

/*
 * fuse_det_decode: YOLO-style detection-head decode in one kernel (DeepJIT
 * write-up, sections 1.1, 2.2 and 5.2: the sigmoid / exp / mul / add / slice /
 * concat / cast tail of a detector). level_logits[l]: device NCHW tensor
 * [batch, n_anchors * n_ch, H[l], W[l]] of in_dt, channel a * n_ch + k.
 * strides[l] (pixels per cell), anchors_wh[(l * n_anchors + a) * 2 + {0,1}]
 * (anchor w, h in pixels): host arrays. out: device fp32
 * [batch, sum_l n_anchors * H[l] * W[l], n_ch], rows ordered level, anchor,
 * y, x; for row (l, a, y, x) and logit t_k:
 *   out[0] = (sigmoid(t0) + x) * stride   out[1] = (sigmoid(t1) + y) * stride
 *   out[2] = exp(t2) * anchor_w           out[3] = exp(t3) * anchor_h
 *   out[k] = sigmoid(t_k) for k >= 4.
 * Limits: 1 <= n_levels <= 8, 1 <= n_anchors <= 16, 5 <= n_ch <= 1024,
 * H[l] * W[l] <= 2^22 cells per level, and fewer than 2^23 tiles of 24 cells
 * (n_ch <= 256; 8 cells beyond) over all images, anchors and levels: one
 * 256-thread workgroup per tile in a single launch.
 * Errors: NP_EINVAL on NULL pointers or out-of-range sizes.
 */
int fuse_det_decode(const void* const* level_logits, int n_levels, const int32_t* H,
                    const int32_t* W, const float* strides, const float* anchors_wh,
                    int n_anchors, int n_ch, int batch, np_dtype in_dt, float* out,
                    hipStream_t stream);

/*
 * fuse_add_rmsnorm: residual add + RMSNorm in one pass (TeleTron write-up,
 * sections 3.3 and 4.2: per-row reduction then elementwise scaling, fp32
 * accumulation, eps inside the square root). Row-major contiguous [rows, cols]
 * of dt:
 *   h = x + r (rounded to dt, stored to h_out, and used by the norm)
 *   out = h / sqrt(mean_j(h_j^2) + eps) * w_j
 * r == NULL: h = x. w == NULL: weight 1. h_out == NULL: h is not stored.
 * Errors: NP_EINVAL for NULL x/out, rows < 0, cols < 1 or cols > 2^24, eps not
 * finite and > 0.
 */
int fuse_add_rmsnorm(const void* x, const void* r, const void* w, void* h_out, void* out,
                     int64_t rows, int64_t cols, float eps, np_dtype dt, hipStream_t stream);

/*
 * fuse_add_layernorm: residual add + LayerNorm in one pass (DeepJIT write-up,
 * section 4.3: one block per row computing the row's mean and variance,
 * normalising and applying gamma / beta, instead of separate mean, variance and
 * normalise kernels; the runtime page, section 4.1, gives the same formula).
 * Row-major contiguous [rows, cols] of dt:
 *   h = x + r (rounded to dt, stored to h_out, and used by the norm)
 *   mu = mean_j(h_j), var = mean_j((h_j - mu)^2)  (population variance,
 *   computed as a second pass over the row, not as E[h^2] - mu^2)
 *   out = (h - mu) / sqrt(var + eps) * gamma_j + beta_j
 * r == NULL: h = x. gamma == NULL: 1. beta == NULL: 0. h_out == NULL: not stored.
 * Errors as fuse_add_rmsnorm.
 */
int fuse_add_layernorm(const void* x, const void* r, const void* gamma, const void* beta,
                       void* h_out, void* out, int64_t rows, int64_t cols, float eps, np_dtype dt,
                       hipStream_t stream);

/*
 * fuse_qkv_rope: QKV split + rotate-half RoPE + Q scale in one pass (TeleTron
 * write-up, section 3.1: the multi-head split, rotary position encoding and
 * scaling after the QKV projection). qkv: [T, 3, n_heads, head_dim] row-major
 * (q, k, v outermost per token). q, k, v: [n_heads, T, head_dim]. For position
 * p = positions[t] (positions == NULL: p = t) and i < head_dim/2:
 *   inv_i = fp32(base^(-2i/head_dim)), theta = fp32(fp32(p) * inv_i),
 *   o[i] = u cos(theta) - w sin(theta), o[i + head_dim/2] = w cos + u sin,
 *   with (u, w) = (x[i], x[i + head_dim/2]); Q = o * q_scale, K = o, V = x.
 * positions: device int32 [T] or NULL. Limits: head_dim even, <= 512.
 * Errors: NP_EINVAL for NULL buffers, T < 0, n_heads < 1, bad head_dim,
 * base <= 0, non-finite q_scale.
 */
int fuse_qkv_rope(const void* qkv, void* q, void* k, void* v, int64_t T, int n_heads,
                  int head_dim, const int32_t* positions, float base, float q_scale,
                  np_dtype dt, hipStream_t stream);

/* Launch size. A dispatch grid counts at most 2^32 work-items, so the fused
 * calls split a long input into several launches on the same stream: the
 * chain every 2^30 elements, the norms every 2^22 rows, QKV + RoPE every
 * 2^21 tokens (fewer for very wide rows). The results do not depend on it. */

/* ------------------------------------------ unfused (N-launch) baselines */
/* The same chains as one kernel per operator, each kernel reading its operands
 * from HBM and storing its result in the storage type before the next launch
 * (NaiveRT write-up: K calls of cost L + T_k each; DeepJIT write-up, section
 * 1.1: every small kernel reads and writes the whole tensor). Results follow
 * the unfused definitions: rounding after every operator. Each runs one
 * thread per element in one launch per operator, so a call takes fewer than
 * 2^31 elements (and the norms fewer than 2^23 rows); larger calls return
 * NP_EINVAL. */

/* One launch per op after the initial NP_LOAD (a lone load is one copy
 * launch), in place in `out`. Requires in_dt == out_dt (the storage type). */
int unfused_chain(const np_op* ops, int n_ops, const void* const* inputs, int n_inputs,
                  np_dtype in_dt, void* out, np_dtype out_dt, int64_t n, hipStream_t stream);

/* 7 launches per level (permute to rows of n_ch; sigmoid on x, y; sigmoid on
 * objectness and classes; exp on w, h; times anchor; plus grid; times stride),
 * then one concat and one cast to fp32: 7 * n_levels + 2 launches.
 * workspace: device buffer of at least 2 * total_rows * n_ch * sizeof(in_dt)
 * bytes (total_rows = batch * sum_l n_anchors * H[l] * W[l]). */
int unfused_det_decode(const void* const* level_logits, int n_levels, const int32_t* H,
                       const int32_t* W, const float* strides, const float* anchors_wh,
                       int n_anchors, int n_ch, int batch, np_dtype in_dt, float* out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * unfused_det_decode_noalloc: unfused_det_decode (same kernels, same results)
 * for callers that cannot allocate device memory around a call -- code under
 * HIP graph capture, serving loops that must not call the allocator,
 * harnesses that forbid allocation. Instead of a caller workspace the call
 * stages through a 16 MiB array that the library owns, one per GPU, held
 * until the process ends; it calls no hipMalloc / hipFree. The staged bytes
 * (2 * batch * sum_l n_anchors * H[l] * W[l] * n_ch * sizeof(in_dt); 8,568,000
 * for one image of the 3-level 80/40/20 YOLO head) must fit in 16 MiB,
 * else NP_EINVAL. Calls that overlap on one GPU (concurrent streams or host
 * threads) share that array and race; calls on one stream are ordered.
 * Errors otherwise as unfused_det_decode.
 */
int unfused_det_decode_noalloc(const void* const* level_logits, int n_levels, const int32_t* H,
                               const int32_t* W, const float* strides, const float* anchors_wh,
                               int n_anchors, int n_ch, int batch, np_dtype in_dt, float* out,
                               hipStream_t stream);

/* 6 launches: add; square; row mean; (+eps, 1/sqrt); times rstd; times w.
 * workspace: at least (rows * cols + 2 * rows) * sizeof(dt) bytes, plus
 * rows * cols * sizeof(dt) when h_out == NULL. w == NULL skips the last launch. */
int unfused_add_rmsnorm(const void* x, const void* r, const void* w, void* h_out, void* out,
                        int64_t rows, int64_t cols, float eps, np_dtype dt, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* 9 launches: add; row mean; subtract the mean; square; row mean; (+eps,
 * 1/sqrt); times rstd; times gamma; plus beta (gamma / beta launches skipped
 * when NULL). workspace: at least (rows * cols + 3 * rows) * sizeof(dt) bytes,
 * plus rows * cols * sizeof(dt) when h_out == NULL. */
int unfused_add_layernorm(const void* x, const void* r, const void* gamma, const void* beta,
                          void* h_out, void* out, int64_t rows, int64_t cols, float eps,
                          np_dtype dt, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* 4 launches: split to head-major; RoPE on Q; RoPE on K; scale Q. */
int unfused_qkv_rope(const void* qkv, void* q, void* k, void* v, int64_t T, int n_heads,
                     int head_dim, const int32_t* positions, float base, float q_scale,
                     np_dtype dt, hipStream_t stream);

/* An empty kernel launched `count` times on the stream (direct measurement of
 * the per-launch cost, the NaiveRT write-up's "29 empty calls"). */
int np_empty_launches(int count, hipStream_t stream);

/*
 * fuse_rmsnorm_linear: RMSNorm + linear + scale in one matrix-core kernel
 * (TeleTron write-up, section 4.2: the row's RMS factor is computed in the
 * kernel and used directly in the linear layer's accumulation, bias and an
 * elementwise scale follow, and no normalised tensor is stored). Row-major,
 * dt = NP_BF16 or NP_F16:
 *   x [M, K], w_norm [K] (NULL: weight 1), Wt [N, K] (the linear weight with K
 *   contiguous, i.e. out = y Wt^T as a torch Linear stores it), bias [N]
 *   (NULL: 0), out [M, N]:
 *   rstd_m = 1 / sqrt(mean_k x_mk^2 + eps)
 *   out_mn = scale * (rstd_m * sum_k round_dt(x_mk w_k) Wt_nk + bias_n)
 *   (the product x w is rounded to dt once, as the matrix cores take dt
 *   operands; the sums are fp32).
 * Kernels: with w_norm == NULL and K a multiple of 64, both operands are
 * staged through registers into a two-stage LDS ring (the fastest form); with
 * w_norm == NULL and K a multiple of 32 otherwise, both stream straight into
 * LDS through a four-stage ring; in every other case x passes through
 * registers where it is multiplied by w_norm (see np_fold_norm_weight).
 * Limits: K a multiple of 8; M, N, K < 2^31; x, Wt, w_norm 16-byte aligned.
 * M = 0 is a no-op that touches no buffer.
 * Errors: NP_EINVAL for another dtype, bad sizes or alignment, NULL x / Wt /
 * out, eps not finite and > 0, scale not finite, out overlapping an input.
 */
int fuse_rmsnorm_linear(const void* x, const void* w_norm, const void* Wt, const void* bias,
                        void* out, int64_t M, int64_t N, int64_t K, float eps, float scale,
                        np_dtype dt, hipStream_t stream);

/*
 * unfused_rmsnorm_linear: the same three steps as separate launches: RMSNorm
 * (y = x rstd w rounded to dt, stored in the workspace, >= M * K * 2 bytes,
 * 16-byte aligned); the linear layer with its bias (same matrix-core GEMM,
 * result rounded to dt into out); the scale (out = scale * out in dt).
 */
int unfused_rmsnorm_linear(const void* x, const void* w_norm, const void* Wt, const void* bias,
                           void* out, int64_t M, int64_t N, int64_t K, float eps, float scale,
                           np_dtype dt, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * np_fold_norm_weight: Wt_folded[n][k] = round_dt(w_norm[k] * Wt[n][k]) (the
 * product is exact; one rounding). RMSNorm's weight multiplies every k of the
 * linear layer's input, so it can be moved into the (constant) linear weight
 * once: fuse_rmsnorm_linear(x, NULL, Wt_folded, ...) then computes
 *   scale * (rstd_m * sum_k x_mk round_dt(w_k Wt_nk) + bias_n),
 * the same value in exact arithmetic as with w_norm, rounded in the weight
 * instead of in the activation, and takes the faster kernel that stages both
 * operands unchanged. Wt_folded may be Wt itself (in place) but must not
 * partially overlap it or overlap w_norm. All buffers 16-byte aligned, dt
 * NP_BF16 or NP_F16, K a multiple of 8. Errors: NP_EINVAL.
 */
int np_fold_norm_weight(const void* w_norm, const void* Wt, void* Wt_folded, int64_t N, int64_t K,
                        np_dtype dt, hipStream_t stream);

/* ---- layout: strided transpose and ChannelShuffle --------------------------
 *
 * The runtime page "CUDA算子与AI运行时" (gtnt.cn/news/145880), sections 2 and
 * 2.1: ChannelShuffle is a reshape + transpose; done as an element-by-element
 * strided copy one side of every access is scattered, and the operator should
 * instead stage tiles on chip so that reads and writes are both contiguous.
 * All four calls copy bits (any element type of elem_bytes = 1..16 bytes),
 * so results are exact. Buffers are device memory owned by the caller, dense
 * row-major; in and out must not overlap (NP_EINVAL). Any alignment works:
 * misaligned pointers or pitches take narrower items, never an error.
 */
typedef enum { NP_NCHW = 0, NP_NHWC = 1 } np_layout;

/*
 * fuse_transpose021: in [B, R, S, E] -> out [B, S, R, E],
 * out[b][s][r][e] = in[b][r][s][e]. The E elements of one (r, s) pair (a unit
 * of E * elem_bytes bytes) move together. Kernel choice (host side, from the
 * shape and alignment): units of 1/2/4/8/16 bytes in matrices larger than
 * 16 KB go through LDS tiles of 512-byte rows (256 / 128 for 2- / 1-byte
 * units), in diagonal tile order when a row pitch is a power of two of at
 * least 4 KiB; matrices of <= 16 KB move as whole chunks through LDS; larger
 * units are copied unit by unit in output order. Limits: R, S, E < 2^31, B < 2^40, total <= 2^46 bytes; when neither
 * LDS kernel applies, one [R, S] matrix must hold < 2^31 items.
 * Errors: NP_EINVAL for negative sizes, elem_bytes outside 1..16, NULL or
 * overlapping buffers (unless the tensor is empty); nothing is launched then.
 */
int fuse_transpose021(const void* in, void* out, int64_t B, int64_t R, int64_t S, int64_t E,
                      int elem_bytes, hipStream_t stream);

/*
 * naive_transpose021: the same result with one thread per output element and
 * its input element found by index arithmetic (a generic strided copy, the
 * pages' "direct" version); the baseline the tiled kernels are measured
 * against. Same arguments and errors; one [R, S] matrix must hold < 2^31
 * elements.
 */
int naive_transpose021(const void* in, void* out, int64_t B, int64_t R, int64_t S, int64_t E,
                       int elem_bytes, hipStream_t stream);

/*
 * fuse_channel_shuffle: ChannelShuffle of a 4-D tensor with `groups` groups
 * (the runtime page, section 2: channels viewed as [groups, C / groups],
 * the two axes swapped): output channel i * groups + g holds input channel
 * g * (C / groups) + i. layout NP_NCHW: [N, C, H, W], the transpose of
 * [N, groups, C / groups, H * W]; NP_NHWC: [N, H, W, C], the transpose of
 * [N * H * W, groups, C / groups, 1].
 * Errors: as fuse_transpose021, and NP_EINVAL unless groups >= 1 divides C.
 */
int fuse_channel_shuffle(const void* in, void* out, int64_t N, int64_t C, int64_t H, int64_t W,
                         int64_t groups, int layout, int elem_bytes, hipStream_t stream);

/* naive_channel_shuffle: the same through naive_transpose021. */
int naive_channel_shuffle(const void* in, void* out, int64_t N, int64_t C, int64_t H, int64_t W,
                          int64_t groups, int layout, int elem_bytes, hipStream_t stream);

/*
 * np_transpose_plan: which kernel fuse_transpose021 (naive = 0) or
 * naive_transpose021 (naive = 1) would launch for these pointers and sizes,
 * without launching anything or touching a device (pointers are only looked
 * at for their alignment). Returns item_bytes | kernel << 8 | vec << 12 |
 * diagonal << 13 with kernel 1 = LDS tiles, 2 = whole matrices through LDS,
 * 3 = item by item, vec = 1 when both sides move as 16-byte vectors and
 * diagonal = 1 for the diagonal tile order; 0 for an empty tensor; a negative
 * status on invalid arguments (as fuse_transpose021).
 */
int np_transpose_plan(const void* in, const void* out, int64_t B, int64_t R, int64_t S,
                      int64_t E, int elem_bytes, int naive);

#ifdef __cplusplus
}
#endif
#endif /* NORM_PASS_H */
