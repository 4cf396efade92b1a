// Internal helpers shared by the libzha translation units (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/zha.h"

namespace zha {

constexpr int kWave = 64;

// ---------------------------------------------------------------- workspace layout
//
// One workspace serves every operation; regions are disjoint so a route and the
// attend that consumes its leaf list may share one buffer.
//   [0, 256)            header: int32 status word (sticky first error)
//   build region        per sequence: int32 arrival counter of the one-launch
//                       append (zero between calls)
//   route region        per level l (1..L): kept list (ids, masks, count), list
//                       length, scores, true log-mass (quality), per-head kept
//                       counts and kept bitmaps; plus cut staging
//   attend region       split partials [B*Hq][split_cap][d+2] fp32, then the
//                       pipelined attend's group chunk prefix
struct WsLayout {
  size_t build_off = 0, build_bytes = 0;
  size_t route_off = 0, route_bytes = 0;
  size_t attend_off = 0, attend_bytes = 0;
  size_t total = 0;
  // per-level route arrays (offsets from the workspace base); index l-1
  size_t kids[ZHA_MAX_L], kmask[ZHA_MAX_L], kcount[ZHA_MAX_L];  // kept list per level
  size_t ucount[ZHA_MAX_L];  // candidate list length per level and group (diagnostics)
  size_t scores[ZHA_MAX_L], sel[ZHA_MAX_L], kept[ZHA_MAX_L];
  size_t logmass[ZHA_MAX_L];  // per head: true node log-mass (quality forward)
  size_t selbits[ZHA_MAX_L];  // per head: kept bits of the union list, 64 entries a word
  int64_t nwcap[ZHA_MAX_L];
  int64_t cap[ZHA_MAX_L];
  size_t stage = 0;        // cut staging: [B*Hq][stage_cap] (u32 key, f32 w)
  int64_t stage_cap = 0;
  int32_t split_cap = 0;   // partial slots per query head
  size_t prefix_off = 0;   // pipelined attend: per-group chunk prefix [B*H_kv + 1] (int32)
};

constexpr int kTileKeys = 64;       // keys per attend tile
constexpr int kTilesPerItem = 16;   // tiles per split (work item): 1024 keys
constexpr int kGatherItemTiles = 4; // gathered bf16 leaves of C < 16 keys: 256-key items
constexpr int kPartPad = 2;         // (m, l) ahead of the d outputs

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Node capacity of level l (1-based) for a cache of T_cap tokens.
inline int64_t level_cap(const zha_cfg& c, int l) {
  int64_t span = 1;
  for (int i = 0; i < l; ++i) span *= c.C;
  int64_t n = c.T_cap / span;
  return n < 1 ? 1 : n;
}

// Tiles per work item of the per-item attend kernels.  The kernel that gathers
// the rows of small leaves (bf16, C < 16) waits on every chunk's scattered
// loads, so it takes shorter items: four times the workgroups in flight.
inline int32_t item_tiles(const zha_cfg& c) {
  return (c.kv_dtype == ZHA_BF16 && c.C < 16) ? kGatherItemTiles : kTilesPerItem;
}

// Work items (splits) per query head: tiles of the largest leaf list, plus the
// tail item holding the open chunk and the sink.
inline int32_t split_capacity(const zha_cfg& c) {
  int64_t leaves = c.leaf_cap;
  int64_t dense_leaves = c.T_cap / c.C;
  if (dense_leaves > leaves) leaves = dense_leaves;
  int64_t tiles = ceil_div(leaves * c.C, kTileKeys);
  return (int32_t)(ceil_div(tiles, item_tiles(c)) + 1);
}

// Partial slots per query head.  The pipelined attend folds each workgroup's
// range of at least kMinRunChunks chunks (16 keys) into one partial per group it
// meets: a group of items work items meets at most 2 * items such ranges.  The
// other attend kernels write one partial per item.
constexpr int kMinRunChunks = 32;
inline int32_t run_capacity(const zha_cfg& c) { return 2 * split_capacity(c); }

inline WsLayout ws_layout(const zha_cfg& c) {
  WsLayout w;
  const int64_t BH = (int64_t)c.B * c.H_kv, BHq = BH * c.G;
  size_t off = 256;
  w.build_off = off;
  off = align_up(off + (size_t)c.B * 4, 256);
  w.build_bytes = off - w.build_off;
  w.route_off = off;
  for (int l = 1; l <= c.L; ++l) {
    int64_t cap = level_cap(c, l);
    w.cap[l - 1] = cap;
    w.kids[l - 1] = off;   off = align_up(off + (size_t)BH * cap * 4, 256);
    w.kmask[l - 1] = off;  off = align_up(off + (size_t)BH * cap * 4, 256);
    w.kcount[l - 1] = off; off = align_up(off + (size_t)BH * 4, 256);
    w.ucount[l - 1] = off; off = align_up(off + (size_t)BH * 4, 256);
    w.scores[l - 1] = off; off = align_up(off + (size_t)BHq * cap * 4, 256);
    w.logmass[l - 1] = off; off = align_up(off + (size_t)BHq * cap * 4, 256);
    w.sel[l - 1] = off;    off = align_up(off + (size_t)BHq * cap, 256);
    w.kept[l - 1] = off;   off = align_up(off + (size_t)BHq * 4, 256);
    w.nwcap[l - 1] = (cap + 63) / 64;
    w.selbits[l - 1] = off; off = align_up(off + (size_t)BHq * w.nwcap[l - 1] * 8, 256);
  }
  // Cut staging for lists too long for LDS: as long as the largest level.
  int64_t scap = 0;
  for (int l = 1; l <= c.L; ++l) scap = w.cap[l - 1] > scap ? w.cap[l - 1] : scap;
  int64_t lcap = c.leaf_cap > 0 ? c.leaf_cap : 1;
  if (lcap > scap) scap = lcap;
  w.stage_cap = scap;
  w.stage = off; off = align_up(off + (size_t)BHq * scap * 8, 256);
  w.route_bytes = off - w.route_off;
  w.attend_off = off;
  w.split_cap = run_capacity(c);
  off = align_up(off + (size_t)BHq * w.split_cap * (c.d + kPartPad) * 4, 256);
  w.prefix_off = off;
  off = align_up(off + (size_t)(BH + 1) * 4, 256);
  w.attend_bytes = off - w.attend_off;
  w.total = off;
  return w;
}

// ---------------------------------------------------------------- device helpers

// Every 64-byte line of a kernel's argument block read at once, first thing: an
// argument first read later, inside a branch, costs a memory round trip of its
// own (~0.5 us), and the short latency-bound kernels read many such lines one
// after another.  One scalar word per line goes into an empty asm statement,
// which makes all the lines' loads issue together and complete before any
// branch; the later reads of the arguments then hit the scalar cache.
template <class T>
__device__ inline void touch_args(const T& args) {
  constexpr int kLines = (int)((sizeof(T) + 63) / 64);
  static_assert(kLines <= 24, "argument block too large to touch at once");
  const int* w = reinterpret_cast<const int*>(&args);
  int v[24];
#pragma unroll
  for (int i = 0; i < 24; ++i) v[i] = i < kLines ? w[16 * i] : 0;
  asm volatile("" ::"s"(v[0]), "s"(v[1]), "s"(v[2]), "s"(v[3]), "s"(v[4]), "s"(v[5]),
               "s"(v[6]), "s"(v[7]), "s"(v[8]), "s"(v[9]), "s"(v[10]), "s"(v[11]));
  asm volatile("" ::"s"(v[12]), "s"(v[13]), "s"(v[14]), "s"(v[15]), "s"(v[16]), "s"(v[17]),
               "s"(v[18]), "s"(v[19]), "s"(v[20]), "s"(v[21]), "s"(v[22]), "s"(v[23]));
}

__device__ inline void set_status(int32_t* status, int32_t code) {
  atomicCAS(status, 0, code);
}

// bf16 (raw 16 bits) to fp32: exact.
__device__ inline float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ inline float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ inline uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t r = 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)((u + r) >> 16);
}

// Order-preserving map of a float to uint32 (larger float -> larger key).
__device__ inline uint32_t order_key(float x) {
  if (x == 0.0f) x = 0.0f;  // fold -0 into +0
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Lane-exchange within 32-lane halves, xor pattern (ds_swizzle bitmask mode).
template <int XOR>
__device__ inline float swz_xor(float v) {
  static_assert(XOR > 0 && XOR < 32, "xor within 32 lanes");
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (XOR << 10) | 0x1f));
}

__device__ inline float shfl_xor32(float v) {
  // lanes l and l ^ 32 (crosses the 32-lane halves)
  return __shfl_xor(v, 32, 64);
}

__device__ inline float wave_max(float v) {
  v = fmaxf(v, swz_xor<1>(v));
  v = fmaxf(v, swz_xor<2>(v));
  v = fmaxf(v, swz_xor<4>(v));
  v = fmaxf(v, swz_xor<8>(v));
  v = fmaxf(v, swz_xor<16>(v));
  v = fmaxf(v, shfl_xor32(v));
  return v;
}

__device__ inline float wave_sum(float v) {
  v += swz_xor<1>(v);
  v += swz_xor<2>(v);
  v += swz_xor<4>(v);
  v += swz_xor<8>(v);
  v += swz_xor<16>(v);
  v += shfl_xor32(v);
  return v;
}

// Exclusive prefix sum of one value per thread over the whole workgroup
// (blockDim.x a multiple of 64, at most 1024).  `scratch` holds 16 T in LDS.
// Returns the exclusive prefix; *total receives the block sum.  Deterministic.
template <typename T>
__device__ inline T block_exclusive_scan(T v, T* scratch, T* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  T x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    T y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  T before = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    const T t = scratch[w];
    if (w < wave) before += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

template <typename T>
__device__ inline T block_reduce_max(T v, T* scratch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    T y = __shfl_xor(v, off, 64);
    v = v > y ? v : y;
  }
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  T m = scratch[0];
  for (int w = 1; w < nw; ++w) m = m > scratch[w] ? m : scratch[w];
  __syncthreads();
  return m;
}

template <typename T>
__device__ inline T block_reduce_sum(T v, T* scratch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  T s = 0;
  for (int w = 0; w < nw; ++w) s += scratch[w];
  __syncthreads();
  return s;
}

// ---- fast collectives: DPP row operations + readlane, compile-time wave count
//
// Within each row of 16 lanes, quad_perm (lane^1, lane^2), row_half_mirror and
// row_mirror pair every lane with partners that differ in each of the low four
// lane bits, so four steps leave the row total in every lane of the row; the
// four row totals are combined through readlane.  Scans use row_shr:1,2,4,8
// (Hillis-Steele within a row) and add the totals of earlier rows.  64-bit
// values move as two 32-bit halves.

template <int CTRL>
__device__ inline uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ inline float dppf(float v) { return __uint_as_float(dpp32<CTRL>(__float_as_uint(v))); }
template <int CTRL>
__device__ inline uint64_t dpp64(uint64_t v) {
  return ((uint64_t)dpp32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp32<CTRL>((uint32_t)v);
}
__device__ inline uint32_t rl32(uint32_t v, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}
__device__ inline uint64_t rl64(uint64_t v, int lane) {
  return ((uint64_t)rl32((uint32_t)(v >> 32), lane) << 32) | rl32((uint32_t)v, lane);
}
__device__ inline float rlf(float v, int lane) { return __uint_as_float(rl32(__float_as_uint(v), lane)); }

constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

__device__ inline float wave_max_fast(float v) {
  v = fmaxf(v, dppf<kDppXor1>(v));
  v = fmaxf(v, dppf<kDppXor2>(v));
  v = fmaxf(v, dppf<kDppHalfMirror>(v));
  v = fmaxf(v, dppf<kDppMirror>(v));
  return fmaxf(fmaxf(rlf(v, 0), rlf(v, 16)), fmaxf(rlf(v, 32), rlf(v, 48)));
}
__device__ inline uint32_t wave_sum_u32(uint32_t v) {
  v += dpp32<kDppXor1>(v);
  v += dpp32<kDppXor2>(v);
  v += dpp32<kDppHalfMirror>(v);
  v += dpp32<kDppMirror>(v);
  return (rl32(v, 0) + rl32(v, 16)) + (rl32(v, 32) + rl32(v, 48));
}
__device__ inline uint64_t wave_sum_u64(uint64_t v) {
  v += dpp64<kDppXor1>(v);
  v += dpp64<kDppXor2>(v);
  v += dpp64<kDppHalfMirror>(v);
  v += dpp64<kDppMirror>(v);
  return (rl64(v, 0) + rl64(v, 16)) + (rl64(v, 32) + rl64(v, 48));
}
// Inclusive prefix sum over the 64 lanes.
template <typename T>
__device__ inline T wave_incl_scan(T x) {
  if constexpr (sizeof(T) == 8) {
    uint64_t v = (uint64_t)x;
    v += dpp64<0x111>(v);
    v += dpp64<0x112>(v);
    v += dpp64<0x114>(v);
    v += dpp64<0x118>(v);
    const uint64_t r0 = rl64(v, 15), r1 = rl64(v, 31), r2 = rl64(v, 47);
    const int row = (threadIdx.x & 63) >> 4;
    v += (row >= 1 ? r0 : 0ull) + (row >= 2 ? r1 : 0ull) + (row >= 3 ? r2 : 0ull);
    return (T)v;
  } else {
    uint32_t v = (uint32_t)x;
    v += dpp32<0x111>(v);
    v += dpp32<0x112>(v);
    v += dpp32<0x114>(v);
    v += dpp32<0x118>(v);
    const uint32_t r0 = rl32(v, 15), r1 = rl32(v, 31), r2 = rl32(v, 47);
    const int row = (threadIdx.x & 63) >> 4;
    v += (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
    return (T)v;
  }
}

// Block-wide collectives over NW waves (blockDim.x == 64 * NW).  `scratch`
// holds NW values in LDS.  Every thread returns the block result.
template <int NW>
__device__ inline float block_max_f(float v, float* scratch) {
  v = wave_max_fast(v);
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
  __syncthreads();
  float m = scratch[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) m = fmaxf(m, scratch[w]);
  __syncthreads();
  return m;
}
template <int NW, typename T>
__device__ inline T block_sum(T v, T* scratch) {
  T t;
  if constexpr (sizeof(T) == 8) t = (T)wave_sum_u64((uint64_t)v);
  else t = (T)wave_sum_u32((uint32_t)v);
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = t;
  __syncthreads();
  T s = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) s += scratch[w];
  __syncthreads();
  return s;
}
template <int NW, typename T>
__device__ inline T block_excl_scan(T v, T* scratch, T* total) {
  const T inc = wave_incl_scan<T>(v);
  if ((threadIdx.x & 63) == 63) scratch[threadIdx.x >> 6] = inc;
  __syncthreads();
  const int wave = threadIdx.x >> 6;
  T before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const T t = scratch[w];
    before += (w < wave) ? t : (T)0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return before + inc - v;
}

// Workgroups are dispatched to the 8 XCDs in turn by linear id (x fastest), and
// each XCD has its own L2.  For a grid width that is a multiple of 8 this maps
// blockIdx.x to a logical index such that XCD j runs the logical indices
// [j w/8, (j+1) w/8): neighbouring logical workgroups share an L2, so output
// lines they write together go back to HBM whole rather than as partial lines
// from several L2s.  Other widths keep blockIdx.x.
__device__ inline int xcd_grouped_x() {
  const int w = (int)gridDim.x, x = (int)blockIdx.x;
  return (w % 8 == 0) ? (x % 8) * (w / 8) + x / 8 : x;
}

// Order LDS traffic of one wave against itself (no cross-wave synchronisation).
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace zha

// Host-side helpers implemented in api.hip.
int32_t zha_check_cfg(const zha_cfg* cfg);
int32_t zha_check_ws(const zha_cfg* cfg, int32_t op, const void* ws, size_t ws_bytes);
