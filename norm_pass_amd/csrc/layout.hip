// Layout kernels: the batched transpose of the two middle axes
// [B, R, S, E] -> [B, S, R, E], and through it ChannelShuffle (runtime page
// "CUDA算子与AI运行时", sections 2 and 2.1: a strided transpose done element by
// element in output order reads addresses that lie far apart; staging tiles in
// on-chip memory keeps both the reads and the writes contiguous).
//
// A "unit" is the E elements that move together (u = E * elem_bytes bytes);
// an "item" (type W) is what one load or store moves. Kernels:
//   tr_tile<W>   the unit is the item, u in {1, 2, 4, 8, 16}: T x T unit tiles
//                pass through LDS; a tile row is 512 bytes (256 for u = 2, 128
//                for u = 1). 16-byte loads run along S in the input, 16-byte
//                stores along R in the output.
//   tr_small<W>  one R x S matrix fits in 16 KB: a chunk of whole matrices is
//                contiguous in both tensors, so it is loaded with 16-byte loads
//                into LDS and written back permuted with 16-byte stores.
//   tr_items<W>  one thread per item in output order, its input item found by
//                index arithmetic. With 16-byte items and units of >= 64 bytes
//                both sides are runs of whole units; with element-sized items
//                it is the naive strided copy the fused kernels are measured
//                against.
// Index arithmetic inside a launch is 32-bit (the host splits the batch axis
// so that a launch covers fewer than 2^31 items); divisions by runtime
// constants use multiply-high reciprocals.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"
#include "internal.h"

namespace np {

namespace {

__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
  return (uint32_t)(((uint64_t)__umulhi(n, f.m) + n) >> f.s);
}

template <int U>
struct Item;
template <>
struct Item<1> { typedef uint8_t T; };
template <>
struct Item<2> { typedef uint16_t T; };
template <>
struct Item<4> { typedef uint32_t T; };
template <>
struct Item<8> { typedef uint64_t T; };
template <>
struct Item<16> { typedef u32x4 T; };

template <int U>
struct TileGeom {
  // A tile row is 512 bytes for units of >= 4 bytes (256 for 2, 128 for 1):
  // long enough that each row read or written is a few whole DRAM bursts.
  static constexpr int ROWB = U >= 4 ? 512 : 128 * U;
  static constexpr int T = ROWB / U;                 // units per tile side
  static constexpr int NT = ROWB >= 512 ? 512 : 256; // threads per block
  static constexpr int VPR = ROWB / 16;              // 16-byte vectors per row
  static constexpr int RPP = NT / VPR;               // rows per pass of NT threads
  static constexpr int IPV = 16 / U;                 // units per vector
  // LDS row pitch: one pad word for 1- and 2-byte units (keeps a column's
  // units in different banks); 8- and 16-byte units pad by their own size so
  // LDS accesses stay aligned; 4-byte units: 640 bytes, with the placement
  // in swz4.
  static constexpr int PITCH = U == 4 ? 640 : ROWB + (U < 4 ? 4 : U);
  static constexpr int LDS = T * PITCH;              // 81,920 bytes at most (U = 4)
};

// Store 16 bytes into LDS at an address aligned to the unit size only.
template <int U>
__device__ __forceinline__ void lds_put16(uint8_t* p, u32x4 v) {
  if constexpr (U >= 16) {
    *reinterpret_cast<u32x4*>(p) = v;
  } else if constexpr (U == 8) {
    reinterpret_cast<uint64_t*>(p)[0] = (uint64_t)v.x | ((uint64_t)v.y << 32);
    reinterpret_cast<uint64_t*>(p)[1] = (uint64_t)v.z | ((uint64_t)v.w << 32);
  } else {
    uint32_t* q = reinterpret_cast<uint32_t*>(p);
    q[0] = v.x;
    q[1] = v.y;
    q[2] = v.z;
    q[3] = v.w;
  }
}

// 4-byte units: unit (i, c) of the 128 x 128 tile at word
// ((c / 4 + i / 4) mod 32) + 32 (c mod 4) of row i, rows 640 bytes apart (160
// words, so row i starts on bank 32 (i mod 2)). A wave stores rows i, i + 1
// (i even), lane (row, v) the units 4 v + m (m = 0..3) at four fixed offsets:
// for each store the banks are ((v + const) mod 32) + 32 ((row + m) mod 2),
// all 64. It
// reads units (4 v + k, j) and (4 v + k, j + 1) (j even): ((v + const) mod 32)
// + 32 ((k + j) mod 2), all 64 again. With the 516-byte pitch the reads were
// two-way conflicted (a wave's 32 reads of one output row fell on 16 banks).
__device__ __forceinline__ uint32_t swz4(int i, int c) {
  return (uint32_t)(i * 640 + 4 * ((((c >> 2) + (i >> 2)) & 31) + 32 * (c & 3)));
}

template <int U, bool VEC>
__global__ __launch_bounds__(TileGeom<U>::NT) void tr_tile(const uint8_t* __restrict__ in,
                                                           uint8_t* __restrict__ out, TileArgs a) {
  typedef TileGeom<U> G;
  typedef typename Item<U>::T W;
  __shared__ __attribute__((aligned(16))) uint8_t lds[G::LDS];
  const uint32_t tile = blockIdx.x;
  const uint32_t b = fdiv(tile, a.tiles_per_b);
  const uint32_t rem = tile - b * a.tiles_per_b.d;
  uint32_t rt, st;
  if (a.diagonal) {
    // Diagonal tile order (Ruetsch and Micikevicius, "Optimizing matrix
    // transpose in CUDA", 2009): blocks running together take tiles from all
    // tile rows and columns, so that with power-of-two pitches their reads and
    // writes do not all land on the same few memory channels.
    const uint32_t k = fdiv(rem, a.n_rt);
    rt = rem - k * a.n_rt.d;
    const uint32_t d = k + rt;
    st = d - fdiv(d, a.n_st) * a.n_st.d;
  } else {
    rt = fdiv(rem, a.n_st);
    st = rem - rt * a.n_st.d;
  }
  const uint32_t r0 = rt * G::T, s0 = st * G::T;
  const int nr = (int)min((uint32_t)G::T, a.R - r0);
  const int ns = (int)min((uint32_t)G::T, a.S - s0);
  const uint8_t* src = in + ((uint64_t)b * a.R + r0) * a.S * U + (uint64_t)s0 * U;
  uint8_t* dst = out + ((uint64_t)b * a.S + s0) * a.R * U + (uint64_t)r0 * U;
  const uint64_t in_pitch = (uint64_t)a.S * U, out_pitch = (uint64_t)a.R * U;
  const int tid = threadIdx.x;
  if constexpr (VEC) {
    // Row pitches and tile edges are whole 16-byte vectors on both sides.
    constexpr int P = G::T / G::RPP;  // passes
    const int lr = tid / G::VPR, lv = tid % G::VPR;
    // units 4 lv .. 4 lv + 3 of tile row i (4-byte units only)
    auto put4 = [&](int i, int lv_, u32x4 x) {
      uint32_t* q = reinterpret_cast<uint32_t*>(lds + swz4(i, 4 * lv_));
      q[0] = x.x;
      q[32] = x.y;
      q[64] = x.z;
      q[96] = x.w;
    };
    // unit (i, c) of the tile
    auto get = [&](int i, int c) -> W {
      if constexpr (U == 4) {
        return *reinterpret_cast<const W*>(lds + swz4(i, c));
      } else {
        return *reinterpret_cast<const W*>(lds + i * G::PITCH + c * U);
      }
    };
    if (nr == G::T && ns == G::T) {
      // Interior tile: every load is issued before the first LDS store, so
      // each wave keeps P loads in flight.
      u32x4 v[P];
#pragma unroll
      for (int p = 0; p < P; ++p) v[p] = load_raw(src + (p * G::RPP + lr) * in_pitch + lv * 16);
#pragma unroll
      for (int p = 0; p < P; ++p) {
        if constexpr (U == 4) {
          put4(p * G::RPP + lr, lv, v[p]);
        } else {
          lds_put16<U>(lds + (p * G::RPP + lr) * G::PITCH + lv * 16, v[p]);
        }
      }
      __syncthreads();
#pragma unroll
      for (int p = 0; p < P; ++p) {
        W e[G::IPV];
#pragma unroll
        for (int k = 0; k < G::IPV; ++k) e[k] = get(lv * G::IPV + k, p * G::RPP + lr);
        __builtin_memcpy(&v[p], e, 16);
      }
#pragma unroll
      for (int p = 0; p < P; ++p) store_raw_nt(dst + (p * G::RPP + lr) * out_pitch + lv * 16, v[p]);
      return;
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int i = p * G::RPP + lr;
      if (i < nr && lv * G::IPV < ns) {
        if constexpr (U == 4) {
          put4(i, lv, load_raw(src + i * in_pitch + lv * 16));
        } else {
          lds_put16<U>(lds + i * G::PITCH + lv * 16, load_raw(src + i * in_pitch + lv * 16));
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int j = p * G::RPP + lr;  // output row s - s0
      if (j < ns && lv * G::IPV < nr) {
        W e[G::IPV];
#pragma unroll
        for (int k = 0; k < G::IPV; ++k) e[k] = get(lv * G::IPV + k, j);
        u32x4 v;
        __builtin_memcpy(&v, e, 16);
        store_raw_nt(dst + j * out_pitch + lv * 16, v);
      }
    }
  } else {
    for (int idx = tid; idx < G::T * G::T; idx += G::NT) {
      const int i = idx / G::T, c = idx % G::T;
      if (i < nr && c < ns)
        *reinterpret_cast<W*>(lds + i * G::PITCH + c * U) =
            *reinterpret_cast<const W*>(src + i * in_pitch + c * U);
    }
    __syncthreads();
    for (int idx = tid; idx < G::T * G::T; idx += G::NT) {
      const int j = idx / G::T, c = idx % G::T;
      if (j < ns && c < nr)
        *reinterpret_cast<W*>(dst + j * out_pitch + c * U) =
            *reinterpret_cast<const W*>(lds + c * G::PITCH + j * U);
    }
  }
}

// Whole matrices through LDS. Items of W bytes, E items per unit, R x S units
// per matrix; the block handles matrices [blockIdx.x * per_chunk, ...).
template <int W, bool VEC>
__global__ __launch_bounds__(256) void tr_small(const uint8_t* __restrict__ in,
                                                uint8_t* __restrict__ out, SmallArgs a) {
  typedef typename Item<W>::T It;
  constexpr uint32_t IPV = 16 / W;
  constexpr uint32_t MAXV = kSmallChunkBytes / 16 / 256;  // vectors per thread, at most
  __shared__ __attribute__((aligned(16))) uint8_t lds[kSmallChunkBytes];
  const uint32_t m0 = blockIdx.x * a.per_chunk;
  const uint32_t mats = min(a.per_chunk, a.B - m0);
  const uint32_t R = a.R, S = a.S, E = a.e.d;
  const uint32_t n_items = mats * a.mat_items.d;
  const uint64_t base = (uint64_t)m0 * a.mat_items.d * W;
  const uint8_t* src = in + base;
  uint8_t* dst = out + base;
  const uint32_t tid = threadIdx.x;
  // load: the chunk is contiguous; all of a thread's loads are issued first
  uint32_t n_vec = 0;
  if constexpr (VEC) {
    n_vec = n_items / IPV;  // the same for every thread of the block
    if (n_vec > 0) {
      u32x4 x[MAXV];
      // indexes past the end re-load the last vector (in bounds, discarded),
      // so no branch separates the loads and all of them are in flight together
#pragma unroll
      for (uint32_t p = 0; p < MAXV; ++p)
        x[p] = load_raw(src + (uint64_t)min(tid + p * 256, n_vec - 1) * 16);
#pragma unroll
      for (uint32_t p = 0; p < MAXV; ++p)
        if (tid + p * 256 < n_vec) *reinterpret_cast<u32x4*>(lds + (tid + p * 256) * 16) = x[p];
    }
  }
  for (uint32_t i = n_vec * IPV + tid; i < n_items; i += 256)
    *reinterpret_cast<It*>(lds + i * W) = *reinterpret_cast<const It*>(src + (uint64_t)i * W);
  __syncthreads();
  // store: output item j of the chunk is (m, s, r, e) in output order; its
  // input item is ((m R + r) S + s) E + e
  const uint32_t SE = S * E, RSE = a.mat_items.d;
  auto input_item = [&](uint32_t j, uint32_t& s, uint32_t& r, uint32_t& e) {
    const uint32_t m = fdiv(j, a.mat_items);
    uint32_t t = j - m * RSE;
    s = fdiv(t, a.re);
    t -= s * a.re.d;
    r = fdiv(t, a.e);
    e = t - r * E;
    return ((m * R + r) * S + s) * E + e;
  };
  bool pairs = false;
  if constexpr (VEC && IPV % 2 == 0) {
    // Two groups of single-item units (ChannelShuffle with two groups, NHWC):
    // output items 2s and 2s + 1 of a matrix are input items s and S + s, so
    // an output vector is IPV / 2 such pairs -- one division per vector and a
    // compare-select per pair, where the general walk below costs three
    // divisions per vector and three compare-selects per item. (rocprofv3 on
    // the NHWC ChannelShuffle workload: 87 -> 25 VALU instructions per 16-byte
    // vector; the time moved little, 55 -> 55 us warm, 66 -> 64 us cold, as the
    // VALU work was already hidden behind the chunk's loads and stores.)
    pairs = R == 2 && E == 1;
    if (pairs) {
      const uint32_t RS = a.mat_items.d;  // 2 S
      for (uint32_t v = tid; v < n_vec; v += 256) {
        const uint32_t j = v * IPV;
        uint32_t mbase = fdiv(j, a.mat_items) * RS;
        uint32_t s = (j - mbase) >> 1;
        It x[IPV];
#pragma unroll
        for (uint32_t k = 0; k < IPV / 2; ++k) {
          x[2 * k] = *reinterpret_cast<const It*>(lds + (mbase + s) * W);
          x[2 * k + 1] = *reinterpret_cast<const It*>(lds + (mbase + S + s) * W);
          ++s;
          const bool wrap = s == S;
          s = wrap ? 0u : s;
          mbase += wrap ? RS : 0u;
        }
        u32x4 o;
        __builtin_memcpy(&o, x, 16);
        store_raw_nt(dst + (uint64_t)v * 16, o);
      }
    }
  }
  if constexpr (VEC) {
    for (uint32_t v = pairs ? n_vec : tid; v < n_vec; v += 256) {
      uint32_t s, r, e;
      uint32_t off = input_item(v * IPV, s, r, e);
      It x[IPV];
#pragma unroll
      for (uint32_t k = 0; k < IPV; ++k) {
        x[k] = *reinterpret_cast<const It*>(lds + off * W);
        // step to the next output item with selects, not branches: e, then r,
        // then s carry over; the input offset moves by the matching stride
        ++e;
        ++off;
        const bool ce = e == E;
        e = ce ? 0u : e;
        r += ce;
        off += ce ? SE - E : 0u;
        const bool cr = r == R;
        r = cr ? 0u : r;
        s += cr;
        off += cr ? E - RSE : 0u;
        const bool cs = s == S;
        s = cs ? 0u : s;
        off += cs ? RSE - SE : 0u;
      }
      u32x4 o;
      __builtin_memcpy(&o, x, 16);
      store_raw_nt(dst + (uint64_t)v * 16, o);
    }
  }
  for (uint32_t j = n_vec * IPV + tid; j < n_items; j += 256) {
    uint32_t s, r, e;
    const uint32_t off = input_item(j, s, r, e);
    *reinterpret_cast<It*>(dst + (uint64_t)j * W) = *reinterpret_cast<const It*>(lds + off * W);
  }
}

// One thread per output item. NT: non-temporal stores (the fused path; the
// naive baseline keeps plain stores, like a generic strided copy). Measured on
// [16384, 72] units of 256 bytes: 111 us with plain stores, 96 us with
// non-temporal ones.
template <int W, bool NT>
__global__ __launch_bounds__(256) void tr_items(const uint8_t* __restrict__ in,
                                                uint8_t* __restrict__ out, ItemArgs a) {
  typedef typename Item<W>::T It;
  const uint32_t j = blockIdx.x * 256u + threadIdx.x;
  if (j >= a.n_items) return;
  const uint32_t q = fdiv(j, a.e);  // output unit
  const uint32_t e = j - q * a.e.d;
  const uint32_t t = fdiv(q, a.r);
  const uint32_t r = q - t * a.r.d;
  const uint32_t b = fdiv(t, a.s);
  const uint32_t s = t - b * a.s.d;
  const uint32_t src = ((b * a.r.d + r) * a.s.d + s) * a.e.d + e;
  const It v = *reinterpret_cast<const It*>(in + (uint64_t)src * W);
  It* dst = reinterpret_cast<It*>(out + (uint64_t)j * W);
  if (NT)
    __builtin_nontemporal_store(v, dst);
  else
    *dst = v;
}

template <int U>
hipError_t launch_tile_u(const uint8_t* in, uint8_t* out, const TileArgs& a, uint32_t n_tiles,
                         bool vec, hipStream_t s) {
  const dim3 block(TileGeom<U>::NT);
  if (vec)
    hipLaunchKernelGGL((tr_tile<U, true>), dim3(n_tiles), block, 0, s, in, out, a);
  else
    hipLaunchKernelGGL((tr_tile<U, false>), dim3(n_tiles), block, 0, s, in, out, a);
  return hipGetLastError();
}

template <int W>
hipError_t launch_small_w(const uint8_t* in, uint8_t* out, const SmallArgs& a, uint32_t grid,
                          bool vec, hipStream_t s) {
  if (vec)
    hipLaunchKernelGGL((tr_small<W, true>), dim3(grid), dim3(256), 0, s, in, out, a);
  else
    hipLaunchKernelGGL((tr_small<W, false>), dim3(grid), dim3(256), 0, s, in, out, a);
  return hipGetLastError();
}

template <int W>
void launch_items_w(const uint8_t* in, uint8_t* out, const ItemArgs& a, dim3 grid, bool nt,
                    hipStream_t s) {
  if (nt)
    hipLaunchKernelGGL((tr_items<W, true>), grid, dim3(256), 0, s, in, out, a);
  else
    hipLaunchKernelGGL((tr_items<W, false>), grid, dim3(256), 0, s, in, out, a);
}

}  // namespace

int tile_side(int unit_bytes) {
  switch (unit_bytes) {
    case 1: return TileGeom<1>::T;
    case 2: return TileGeom<2>::T;
    case 4: return TileGeom<4>::T;
    case 8: return TileGeom<8>::T;
    case 16: return TileGeom<16>::T;
    default: return 0;
  }
}

hipError_t launch_tr_tile(const void* in, void* out, const TileArgs& a, uint32_t n_tiles,
                          int unit_bytes, bool vec, hipStream_t s) {
  const uint8_t* i = static_cast<const uint8_t*>(in);
  uint8_t* o = static_cast<uint8_t*>(out);
  switch (unit_bytes) {
    case 1: return launch_tile_u<1>(i, o, a, n_tiles, vec, s);
    case 2: return launch_tile_u<2>(i, o, a, n_tiles, vec, s);
    case 4: return launch_tile_u<4>(i, o, a, n_tiles, vec, s);
    case 8: return launch_tile_u<8>(i, o, a, n_tiles, vec, s);
    case 16: return launch_tile_u<16>(i, o, a, n_tiles, vec, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_tr_small(const void* in, void* out, const SmallArgs& a, uint32_t grid,
                           int item_bytes, bool vec, hipStream_t s) {
  const uint8_t* i = static_cast<const uint8_t*>(in);
  uint8_t* o = static_cast<uint8_t*>(out);
  switch (item_bytes) {
    case 1: return launch_small_w<1>(i, o, a, grid, vec, s);
    case 2: return launch_small_w<2>(i, o, a, grid, vec, s);
    case 4: return launch_small_w<4>(i, o, a, grid, vec, s);
    case 8: return launch_small_w<8>(i, o, a, grid, vec, s);
    case 16: return launch_small_w<16>(i, o, a, grid, vec, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_tr_items(const void* in, void* out, const ItemArgs& a, int item_bytes,
                           bool nt, hipStream_t s) {
  const uint8_t* i = static_cast<const uint8_t*>(in);
  uint8_t* o = static_cast<uint8_t*>(out);
  const dim3 grid((a.n_items + 255u) / 256u);
  switch (item_bytes) {
    case 1: launch_items_w<1>(i, o, a, grid, nt, s); break;
    case 2: launch_items_w<2>(i, o, a, grid, nt, s); break;
    case 4: launch_items_w<4>(i, o, a, grid, nt, s); break;
    case 8: launch_items_w<8>(i, o, a, grid, nt, s); break;
    case 16: launch_items_w<16>(i, o, a, grid, nt, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace np
