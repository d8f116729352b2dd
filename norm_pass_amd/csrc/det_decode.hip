// Fused detection-head decode: sigmoid / exp / anchor / grid / stride / concat /
// cast in one kernel (DeepJIT write-up, hotelren.com/news/5350627, sections 1.1,
// 2.2 and 5.2). The logits are channel-planar (NCHW) while the boxes are rows
// of n_ch floats, so the decode is a transpose; reading channel planes and
// writing rows directly would make one side strided (the page
// "CUDA算子与AI运行时", gtnt.cn/news/145880, section 2.1: a strided
// reshape/transpose drops bandwidth use from 82% to 37%). Each workgroup takes
// a tile of TP consecutive cells of one (level, batch, anchor):
//   phase 1: coalesced reads along the cells of each channel plane, decode in
//            fp32, write the value into an LDS tile laid out exactly like the
//            output rows (stride n_ch, odd for 85, so the column writes do not
//            conflict);
//   phase 2: the tile's output rows are one contiguous span of the
//            concatenated output; copy it linearly with dwordx4 stores.
#include <stddef.h>

#include "device.h"
#include "internal.h"

namespace np {
namespace {

#ifndef NP_DET_BLOCK
#define NP_DET_BLOCK 256
#endif
constexpr int kBlock = NP_DET_BLOCK;

// One formula for every channel, so that the lanes of a wave (which hold
// different channels) do not diverge: channels 2 and 3 need exp(t), all others
// sigmoid(t) = 1 / (1 + exp(-t)); one exp of +-t serves both. The exp is
// np_fast_exp (<= 2 fp32 ulp) and the reciprocal v_rcp_f32 (1 ulp) applied to
// (1 + e) 2^-32 and scaled back by 2^-32: the scaled input stays below 2^96,
// so the reciprocal never has to produce a subnormal (which it would flush),
// and the final exact multiply by 2^-32 rounds correctly into the subnormal
// range. Sigmoid error <= 4 ulp (5e-7 relative).
//   k = 0: (sigmoid + x) * stride   k = 1: (sigmoid + y) * stride
//   k = 2: exp * anchor_w           k = 3: exp * anchor_h      k >= 4: sigmoid
// Per-tile constants (stride, anchor, 1/W) are read once per workgroup.
struct TileConst {
  float stride, aw, ah, inv_w;
  int w;
};

__device__ __forceinline__ float decode_one(const TileConst& tc, int k, int cell, float t) {
  const bool is_exp = k == 2 || k == 3;
  const float e = np_fast_exp(is_exp ? t : -t);
  // cell / W and cell % W: (cell + 0.5) / W is >= 0.5 / W from an integer, far
  // above the float rounding for cell < 2^22, so truncation gives the row
  const int y = (int)(((float)cell + 0.5f) * tc.inv_w);
  const int x = cell - y * tc.w;
  const float grid = k == 0 ? (float)x : k == 1 ? (float)y : 0.0f;
  const float mul = k < 2 ? tc.stride : 1.0f;
  const float anc = k == 3 ? tc.ah : tc.aw;
  const float sig = __builtin_amdgcn_rcpf(__builtin_fmaf(e, 0x1p-32f, 0x1p-32f)) * 0x1p-32f;
  return is_exp ? e * anc : (sig + grid) * mul;
}

// The same values for the N consecutive cells of one channel k that a thread
// decodes from one vector, with every channel choice made once per thread: the
// lanes of a wave then run one instruction stream whatever their channels
// (with per-element selects the compiler branched, and the wave holding the
// box channels ran every branch). The cells c0 .. c0 + N - 1 lie in at most two
// grid rows when W >= N: cell c0 + i is at x0 + i - W [i >= W - x0], row y0 +
// [i >= W - x0], and the grid term is gA + gB i + gD [i >= W - x0] with
// (gA, gB, gD) = (x0, 1, -W) for k = 0, (y0, 0, 1) for k = 1 and 0 otherwise,
// all small integers, exact in fp32: the results are those of decode_one.
struct ChanConst {
  float gA, gB, gD, mul, anc, sgn;
  int wrap_at;
  bool is_exp;
};

__device__ __forceinline__ ChanConst chan_const(const TileConst& tc, int k, int c0) {
  ChanConst cc;
  const int y0 = (int)(((float)c0 + 0.5f) * tc.inv_w);
  const int x0 = c0 - y0 * tc.w;
  cc.is_exp = k == 2 || k == 3;
  cc.sgn = cc.is_exp ? 1.0f : -1.0f;
  cc.gA = k == 0 ? (float)x0 : k == 1 ? (float)y0 : 0.0f;
  cc.gB = k == 0 ? 1.0f : 0.0f;
  cc.gD = k == 0 ? -(float)tc.w : k == 1 ? 1.0f : 0.0f;
  cc.mul = k < 2 ? tc.stride : 1.0f;
  cc.anc = k == 3 ? tc.ah : tc.aw;
  cc.wrap_at = tc.w - x0;
  return cc;
}

__device__ __forceinline__ float decode_cell(const ChanConst& cc, int i, float t) {
  const float e = np_fast_exp(t * cc.sgn);
  const float grid = __builtin_fmaf(cc.gB, (float)i, cc.gA) + (i >= cc.wrap_at ? cc.gD : 0.0f);
  const float sig = __builtin_amdgcn_rcpf(__builtin_fmaf(e, 0x1p-32f, 0x1p-32f)) * 0x1p-32f;
  const float box = (sig + grid) * cc.mul;
  const float ex = e * cc.anc;
  return cc.is_exp ? ex : box;
}

// Cells per tile (the choice is explained at det_tile_cells below).
#ifndef NP_DET_TILE_CELLS
#define NP_DET_TILE_CELLS 24
#endif

#ifndef NP_DET_XCD_REMAP
#define NP_DET_XCD_REMAP 1
#endif

// Workgroups are dispatched to the 8 XCDs round robin (workgroup b -> XCD
// b % 8), and each XCD has its own L2. Consecutive tiles share the 128-byte
// lines of every channel plane (a 16-cell fp16 tile covers 32 bytes of a
// line), so map the j-th workgroup of XCD x to tile start(x) + j: each XCD
// processes one contiguous run of tiles and every line is fetched into one L2.
__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  constexpr int kXcds = 8;
  const int x = bid % kXcds;
  const int j = bid / kXcds;
  const int per = nb / kXcds;
  const int rem = nb % kXcds;
  return x * per + min(x, rem) + j;
}

// GF: vectors per channel row of a whole tile (tile cells / N), when known at
// compile time (0: read from the arguments), so that the thread -> (channel,
// vector) split is a division by a constant.
template <typename T, bool VEC, int GF>
__global__ __launch_bounds__(kBlock) void det_decode_kernel(DetArgs a) {
  extern __shared__ float tile[];
  // the header, copied at once as ints so that its reads go out together
  // (copied as a struct, the compiler spread them over several waits)
  int32_t hw_[sizeof(DetHeader) / 4];
  __builtin_memcpy(hw_, &a.h, sizeof(hw_));
  DetHeader h;
  __builtin_memcpy(&h, hw_, sizeof(h));
  const int bid = NP_DET_XCD_REMAP ? xcd_remap(blockIdx.x, gridDim.x) : blockIdx.x;
  asm volatile("" ::"s"(h.out), "s"(h.total_rows), "s"(bid));  // all in the first round
  // the level, by comparisons against the whole prefix rather than a search
  // whose every step waits for its own read
  const int nl = h.n_levels;
  int l = 0, ts = 0, tiles = h.tiles[0];
#pragma unroll
  for (int i = 1; i < kDetMaxLevels; ++i) {
    const int tsi = h.tile_start[i];
    const int ti = h.tiles[i];
    const bool past = i < nl && bid >= tsi;
    l += past ? 1 : 0;
    ts = past ? tsi : ts;
    tiles = past ? ti : tiles;
  }
  const int idx = bid - ts;
  const int A = h.n_anchors;
  const int C = h.n_ch;
  const int b = idx / (A * tiles);
  const int rem = idx - b * A * tiles;
  const int an = rem / tiles;
  const int tl = rem - an * tiles;
  // the level's record and the tile's anchor: one more batch of reads
  struct {
    const void* in;
    int64_t row_off;
    int32_t hw, w;
    float stride, inv_w;
  } L;
  static_assert(sizeof(L) == offsetof(DetLevel, anchor), "level record layout");
  __builtin_memcpy(&L, &a.lv[l], sizeof(L));
  float anc[2];
  __builtin_memcpy(anc, &a.lv[l].anchor[2 * an], sizeof(anc));
  asm volatile("" ::"s"(anc[0]), "s"(anc[1]));  // read with the record, not later
  const int HW = L.hw;
  const int TP = h.tile_cells;
  const int cell0 = tl * TP;
  const int ncell = min(TP, HW - cell0);
  const T* plane0 = static_cast<const T*>(L.in) + ((int64_t)(b * A + an) * C) * HW + cell0;
  TileConst tc;
  tc.stride = L.stride;
  tc.aw = anc[0];
  tc.ah = anc[1];
  tc.w = L.w;
  tc.inv_w = L.inv_w;

  // phase 1: channel planes -> decoded values in row layout
  if (VEC) {
    constexpr int N = Vec<T>::N;
    // ncell is a multiple of N on this path; a partial tile's missing vectors
    // are skipped, so the split follows the whole tile's vector count
    const int groups = GF ? GF : TP / N;
    const bool two_rows = tc.w >= N;  // a vector's cells span at most two grid rows
    for (int e = threadIdx.x; e < C * groups; e += kBlock) {
      const int k = e / groups;
      const int cg = e - k * groups;
      if (cg * N >= ncell) continue;
      float t[N];
      load_vec<T>(plane0 + (int64_t)k * HW + cg * N, t);
      if (two_rows) {
        const ChanConst cc = chan_const(tc, k, cell0 + cg * N);
#pragma unroll
        for (int i = 0; i < N; ++i) tile[(cg * N + i) * C + k] = decode_cell(cc, i, t[i]);
      } else {
#pragma unroll
        for (int i = 0; i < N; ++i) {
          const int c = cg * N + i;
          tile[c * C + k] = decode_one(tc, k, cell0 + c, t[i]);
        }
      }
    }
  } else {
    for (int e = threadIdx.x; e < C * ncell; e += kBlock) {
      const int k = e / ncell;
      const int c = e - k * ncell;
      const float t = to_f(plane0[(int64_t)k * HW + c]);
      tile[c * C + k] = decode_one(tc, k, cell0 + c, t);
    }
  }
  __syncthreads();

  // phase 2: contiguous output span of ncell rows
  const int64_t row0 = L.row_off + (int64_t)an * HW + cell0;
  float* dst = h.out + ((int64_t)b * h.total_rows + row0) * C;
  const int len = ncell * C;
  const int head = (int)(((16 - ((uintptr_t)dst & 15)) & 15) >> 2);  // floats to 16-B alignment
  if (((uintptr_t)dst & 3) == 0 && len > head + 4) {
    for (int i = threadIdx.x; i < head; i += kBlock) dst[i] = tile[i];
    const int nvec = (len - head) >> 2;
    for (int v = threadIdx.x; v < nvec; v += kBlock) {
      const int o = head + 4 * v;
      u32x4 q;
      q.x = __builtin_bit_cast(uint32_t, tile[o + 0]);
      q.y = __builtin_bit_cast(uint32_t, tile[o + 1]);
      q.z = __builtin_bit_cast(uint32_t, tile[o + 2]);
      q.w = __builtin_bit_cast(uint32_t, tile[o + 3]);
      store_raw_nt(dst + o, q);
    }
    for (int i = head + 4 * nvec + threadIdx.x; i < len; i += kBlock) dst[i] = tile[i];
  } else {
    for (int i = threadIdx.x; i < len; i += kBlock) dst[i] = tile[i];
  }
}

template <typename T>
hipError_t launch_t(const DetArgs& a, bool vec_in, hipStream_t s) {
  const int blocks = a.h.tile_start[a.h.n_levels];
  const size_t lds = (size_t)a.h.tile_cells * a.h.n_ch * sizeof(float);
  constexpr int kGF = NP_DET_TILE_CELLS / Vec<T>::N;
  if (vec_in && a.h.tile_cells == NP_DET_TILE_CELLS)
    hipLaunchKernelGGL((det_decode_kernel<T, true, kGF>), dim3(blocks), dim3(kBlock), lds, s, a);
  else if (vec_in)
    hipLaunchKernelGGL((det_decode_kernel<T, true, 0>), dim3(blocks), dim3(kBlock), lds, s, a);
  else
    hipLaunchKernelGGL((det_decode_kernel<T, false, 0>), dim3(blocks), dim3(kBlock), lds, s, a);
  return hipGetLastError();
}

}  // namespace

// Cells per tile. 24 at 85 channels: an 8.2 KiB LDS tile, ~1050 workgroups
// for the three YOLO levels, and 3 x 85 = 255 16-byte loads, one per thread of
// the 256, so a workgroup waits for one load round trip. Measured on MI355X:
// 5.7-5.8 us per call, against 6.1-6.3 us for 16, 32, 40 and 48 cells at
// 192-512 threads. The tile stays a multiple of 8 cells so that every tile is
// whole 16-byte vectors. Wide rows (n_ch > 256) use 8 cells to keep the tile
// within 32 KiB.
int det_tile_cells(int n_ch) { return n_ch <= 256 ? NP_DET_TILE_CELLS : 8; }

hipError_t launch_det_decode(const DetArgs& a, int in_dt, bool vec_in, hipStream_t s) {
  switch (in_dt) {
    case NP_F32: return launch_t<float>(a, vec_in, s);
    case NP_F16: return launch_t<_Float16>(a, vec_in, s);
    default: return launch_t<__bf16>(a, vec_in, s);
  }
}

}  // namespace np
