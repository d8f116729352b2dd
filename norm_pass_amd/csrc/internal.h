// Host-side interface between the C ABI (abi.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "norm_pass.h"

namespace np {

// Kernel-argument image of an op list (passed by value; < 1 KiB).
struct ChainArgs {
  int32_t n_ops;
  int32_t kind[NP_MAX_OPS];
  int32_t arg[NP_MAX_OPS];
  float c[NP_MAX_OPS];
  const void* in[NP_MAX_INPUTS];
  void* out;
  int64_t n;
};

inline int dt_size(int dt) { return dt == NP_F32 ? 4 : 2; }

// fused elementwise chain (generic interpreter kernel); vec = 16-byte path
hipError_t launch_chain(const ChainArgs& a, int in_dt, int out_dt, int n_inputs, bool vec,
                        hipStream_t s);

// detection-head decode
// Arguments of the decode kernel. A workgroup reads the header first (fixed
// offsets: two 64-byte lines), finds its level there, then reads that level's
// record (fields and anchors, a few lines, all in one batch): two rounds of
// argument reads before its first plane load.
constexpr int kDetMaxLevels = 8, kDetMaxAnchors = 16;
struct DetLevel {
  const void* in;       // the level's logits [batch, n_anchors * n_ch, H, W]
  int64_t row_off;      // first output row of the level (within one batch image)
  int32_t hw, w;        // H * W and W
  float stride, inv_w;  // grid stride; 1 / W (float)
  float anchor[2 * kDetMaxAnchors];  // (width, height) per anchor
};
struct DetHeader {
  int32_t n_levels, n_anchors, n_ch, batch;
  int32_t tile_cells;                     // cells per tile
  int32_t tile_start[kDetMaxLevels + 1];  // prefix over levels of batch * n_anchors * tiles[l]
  int32_t tiles[kDetMaxLevels];           // tiles per (batch, anchor) of level l
  int32_t pad_;
  int64_t total_rows;                     // rows per batch image
  float* out;
};
struct DetArgs {
  DetHeader h;
  DetLevel lv[kDetMaxLevels];
};
hipError_t launch_det_decode(const DetArgs& a, int in_dt, bool vec_in, hipStream_t s);
int det_tile_cells(int n_ch);  // cells per workgroup tile of the decode kernel

// residual add + RMSNorm
hipError_t launch_add_rmsnorm(const void* x, const void* r, const void* w, void* h, void* out,
                              int64_t rows, int64_t cols, float eps, int dt, bool vec,
                              hipStream_t s);

// residual add + LayerNorm
hipError_t launch_add_layernorm(const void* x, const void* r, const void* g, const void* b,
                                void* h, void* out, int64_t rows, int64_t cols, float eps, int dt,
                                bool vec, hipStream_t s);

// RMSNorm + linear + scale (matrix cores); norm = false: plain GEMM + bias
hipError_t launch_rmsnorm_linear(const void* x, const void* w, const void* Wt, const void* b,
                                 void* out, int M, int N, int K, float eps, float scale, int dt,
                                 bool norm, hipStream_t s);

hipError_t launch_fold_norm_weight(const void* w, const void* Wt, void* Wf, int64_t N, int64_t K,
                                   int dt, hipStream_t s);

// QKV split + RoPE + scale
struct RopeArgs {
  const void* qkv;
  void* q;
  void* k;
  void* v;
  const int32_t* pos;
  int64_t T;           // tokens of the whole call (the head stride of q, k, v)
  int64_t t0, t_end;   // the tokens [t0, t_end) this launch covers
  int32_t H, D;
  float q_scale;
  float inv[256];
};
hipError_t launch_qkv_rope(const RopeArgs& a, int dt, bool vec, hipStream_t s);

// unfused single-op kernels (eager semantics: result stored in the storage type)
enum UnaryExtra { U_SQUARE = 100, U_RSQRT_EPS = 101, U_COPY = 102 };
hipError_t launch_unary(int kind, float c, const void* in, void* out, int64_t n, int dt,
                        hipStream_t s);
hipError_t launch_binary(int kind, const void* a, const void* b, void* out, int64_t n, int dt,
                         hipStream_t s);
hipError_t launch_row_mean(const void* in, void* out, int64_t rows, int64_t cols, int dt,
                           hipStream_t s);
hipError_t launch_row_scale(const void* in, const void* rs, void* out, int64_t rows,
                            int64_t cols, int dt, hipStream_t s);
hipError_t launch_col_scale(const void* in, const void* w, void* out, int64_t rows,
                            int64_t cols, int dt, hipStream_t s);
hipError_t launch_row_sub(const void* in, const void* m, void* out, int64_t rows, int64_t cols,
                          int dt, hipStream_t s);
hipError_t launch_col_add(const void* in, const void* b, void* out, int64_t rows, int64_t cols,
                          int dt, hipStream_t s);
hipError_t launch_qkv_split(const void* qkv, void* q, void* k, void* v, int64_t T, int H, int D,
                            int dt, hipStream_t s);
hipError_t launch_rope_inplace(void* x, int64_t T, int H, int D, const int32_t* pos,
                               const float* inv, int dt, hipStream_t s);
// detection tail pieces (rows of n_ch in the storage type)
enum DetOp { D_SIGMOID = 0, D_EXP = 1, D_MUL_ANCHOR = 2, D_ADD_GRID = 3, D_MUL_C = 4 };
hipError_t launch_det_permute(const void* in, void* rows_out, int batch, int A, int C, int H,
                              int W, int dt, hipStream_t s);
hipError_t launch_det_range_op(void* rows, int batch, int A, int C, int H, int W, int k0, int k1,
                               int op, float c, const float* anchors_a2, int dt, hipStream_t s);
hipError_t launch_det_concat(const void* const* parts, const int64_t* part_rows, int n_parts,
                             void* out, int batch, int64_t total_rows, int C, int dt,
                             hipStream_t s);
// layout: batched transpose [B, R, S, E] -> [B, S, R, E] of byte-sized items
// n / d for any n < 2^32: q = (umulhi(n, m) + n) >> s with the round-up
// multiplier m = floor(2^32 (2^s - d) / d) + 1, s = ceil(log2 d) (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994).
struct FastDiv {
  uint32_t d, m, s;
};
inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  const uint64_t m = (((1ull << 32) * ((1ull << s) - d)) / d) + 1;
  return FastDiv{d, (uint32_t)m, s};
}
struct TileArgs {  // units of 1..16 bytes, T x T tiles
  uint32_t R, S;
  uint32_t diagonal;  // diagonal tile order (power-of-two pitches)
  FastDiv tiles_per_b, n_rt, n_st;
};
constexpr uint32_t kSmallChunkBytes = 16384;
struct SmallArgs {  // whole matrices per block; B = matrices in this launch
  uint32_t B, R, S, per_chunk;
  FastDiv mat_items, re, e;  // items per matrix, R * E, E
};
struct ItemArgs {  // one thread per item; B * S * R * E items
  uint32_t n_items;
  FastDiv e, r, s;
};
int tile_side(int unit_bytes);
hipError_t launch_tr_tile(const void* in, void* out, const TileArgs& a, uint32_t n_tiles,
                          int unit_bytes, bool vec, hipStream_t s);
hipError_t launch_tr_small(const void* in, void* out, const SmallArgs& a, uint32_t grid,
                           int item_bytes, bool vec, hipStream_t s);
hipError_t launch_tr_items(const void* in, void* out, const ItemArgs& a, int item_bytes,
                           bool nt, hipStream_t s);

hipError_t launch_cast_to_f32(const void* in, float* out, int64_t n, int dt, hipStream_t s);

// the argument checks of fuse_det_decode / unfused_det_decode (NP_OK, or
// NP_EINVAL with the thread's error message set)
int validate_det_call(const void* const* lv, int n_levels, const int32_t* H, const int32_t* W,
                      const float* strides, const float* anchors, int n_anchors, int n_ch,
                      int batch, int in_dt, const float* out);
// set the thread's error message (np_last_error) and return code
int set_error(int code, const char* msg);
// the per-device gfx950 check every call makes before its first HIP call
int check_device_call();
hipError_t launch_empty(hipStream_t s);

}  // namespace np
