// Sparse and dense split-K decode attention with the (a, Z) merge.
//
// [ZHA] "전제와 한계" (premises and limits): each query attends exactly over the
// sink token 0, every key of its selected leaves, and the open chunk.
// [ATT] "같은 계산을 메모리 IO 를 줄여서 한다: FlashAttention 계열": online softmax
// (running max m, sum l, unnormalised output o, rescaled by e^{m_old - m_new})
// and Flash-Decoding (split the cache along its length, merge the splits).
// [ASM] "방법론": two attention states merge as a = (Z_A a_A + Z_B a_B)/(Z_A + Z_B).
//
// Work decomposition (one GPU): a "group" is one (sequence, KV head).  Its leaf
// list is read in 16-key chunks, grouped into work items (1024 keys; 256 for
// the kernel that gathers the rows of leaves shorter than 16 keys); the sink
// and the open chunk form the group's tail.  The pipelined kernel (bf16, dense
// or leaves of C >= 16 keys) gives each workgroup of a persistent grid a
// contiguous range of the group-ordered chunks and writes one partial per
// query head for each group its range meets; the other kernels walk whole items
// round-robin and write one partial per item.  The 4 waves of a workgroup take
// alternate chunks and merge their states before a partial is written.  A
// group's K/V chunk is read once for all G query heads of the group; heads that
// did not select a leaf see its keys masked to -inf.
//
// Scores are kept in log2 units: q is pre-multiplied by scale * log2(e).  K/V
// rows are read once per step and carry the non-temporal hint.
#include "zha_internal.hpp"

#include <mutex>

namespace zha {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4_t __attribute__((__vector_size__(4 * sizeof(uint32_t))));

constexpr int kWavesPerWg = 4;
constexpr int kMaxGroups = 2048;
constexpr int kAttendGrid = 512;      // two workgroups per CU: measured faster than four
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttendParams {
  const float* q;             // [BHq][d]
  const void* K;              // [BH][T_cap][d]
  const void* V;
  const int64_t* T;           // [B]
  const int32_t* leaf_ids;    // [BH][leaf_cap] or null (dense)
  const uint32_t* leaf_mask;  // [BH][leaf_cap] or null (dense)
  const int32_t* leaf_count;  // [BH] or null (dense)
  int32_t leaf_cap;
  float* part;                // [BHq][split_cap][d + 2]
  int32_t* prefix;            // [BH + 1] group chunk prefix (pipelined kernel)
  int32_t* status;
  int32_t B, H_kv, G, C;
  int64_t T_cap;
  int32_t split_cap;
  int32_t item_tiles;         // tiles per work item of the per-item kernels
  float qscale;               // scale * log2(e)
};

// Per-group geometry shared by the partial and merge kernels.
struct GroupInfo {
  int64_t T;
  int32_t n1;      // complete leaves
  int32_t U;       // leaf-list entries (dense: n1)
  int32_t tiles;   // 64-key tiles over the list
  int32_t items;   // work items incl. the tail item
};

// A group's raw inputs: the sequence length, the leaf count and the first
// leaf entry (for the sink).  The four loads are issued together, so they cost
// one round trip; a missing array (dense attention) reads the length instead.
struct GroupRaw {
  int64_t T;
  int32_t count;
  int32_t id0;
  uint32_t m0;
};

__device__ inline GroupRaw group_raw(const AttendParams& P, int gi) {
  const int64_t* tp = P.T + gi / P.H_kv;
  const int32_t* cp = P.leaf_count != nullptr ? P.leaf_count + gi : (const int32_t*)tp;
  const int64_t e0 = (int64_t)gi * P.leaf_cap;
  const int32_t* ip = P.leaf_ids != nullptr ? P.leaf_ids + e0 : (const int32_t*)tp;
  const uint32_t* mp = P.leaf_mask != nullptr ? P.leaf_mask + e0 : (const uint32_t*)tp;
  GroupRaw r;
  r.T = *tp;
  r.count = *cp;
  r.id0 = *ip;
  r.m0 = *mp;
  return r;
}

__device__ inline GroupInfo group_info_from(const AttendParams& P, const GroupRaw& r) {
  GroupInfo g;
  int64_t T = r.T;
  if (T < 0) T = 0;
  if (T > P.T_cap) T = P.T_cap;
  g.T = T;
  g.n1 = (int32_t)(T / P.C);
  if (P.leaf_ids == nullptr) {
    g.U = g.n1;
  } else {
    int32_t u = r.count;
    if (u < 0) u = 0;
    if (u > P.leaf_cap) u = P.leaf_cap;
    g.U = u;
  }
  g.tiles = (int32_t)(((int64_t)g.U * P.C + kTileKeys - 1) / kTileKeys);
  g.items = (g.tiles + P.item_tiles - 1) / P.item_tiles + 1;
  return g;
}

__device__ inline GroupInfo group_info(const AttendParams& P, int gi) {
  return group_info_from(P, group_raw(P, gi));
}

// Token and head mask of key slot `slot` (0..63) of tile `tile` of a group;
// tile == -1 is the tail tile (slot 0: sink, slots 1..: open chunk).  Slots that
// hold no key get token 0 (always inside the allocation) and mask 0.
struct Slot { int32_t tok; uint32_t mask; };

__device__ inline Slot slot_of(const AttendParams& P, int gi, const GroupInfo& g,
                               int tile, int slot, uint32_t full, uint32_t sinkmask) {
  Slot s{0, 0u};
  if (tile < 0) {
    if (slot == 0) {
      s.mask = sinkmask;
    } else {
      const int64_t t = (int64_t)g.n1 * P.C + (slot - 1);
      if (t < g.T) { s.tok = (int32_t)t; s.mask = full; }
    }
    return s;
  }
  const int64_t e = (int64_t)tile * kTileKeys + slot;
  const int64_t entry = e / P.C;
  if (entry < g.U) {
    const int kk = (int)(e - entry * P.C);
    if (P.leaf_ids == nullptr) {
      s.tok = (int32_t)(entry * P.C + kk);
      s.mask = full;
    } else {
      const int64_t off = (int64_t)gi * P.leaf_cap + entry;
      const int32_t leaf = P.leaf_ids[off];
      if (leaf >= 0 && leaf < g.n1) {
        s.tok = leaf * P.C + kk;
        s.mask = P.leaf_mask[off] & full;
      }
    }
  }
  return s;
}

// Sink mask of a group: heads that did not select leaf 0 take token 0 from the
// tail tile.  Dense attention and T < C never need it.
__device__ inline uint32_t sink_mask_from(const AttendParams& P, const GroupInfo& g,
                                          const GroupRaw& r, uint32_t full) {
  if (P.leaf_ids == nullptr || g.n1 == 0) return 0u;
  const uint32_t m0 = (g.U > 0 && r.id0 == 0) ? r.m0 : 0u;
  return full & ~m0;
}
__device__ inline uint32_t sink_mask(const AttendParams& P, int gi, const GroupInfo& g,
                                     uint32_t full) {
  return sink_mask_from(P, g, group_raw(P, gi), full);
}

// LDS of the partial kernels.
template <int D>
struct AttendSmem {
  int32_t item_prefix[kMaxGroups + 1];
  int32_t scan[16];
  float p[kWavesPerWg][kTileKeys][16];          // softmax numerators per slot, head
  float alpha[kWavesPerWg][16];                 // rescale factors per head
  float state[kWavesPerWg][16][D + 2];          // (m, l, o[D]) per wave and head
  float qf[16][D];                              // fp32 path: scaled queries
};

// Work items of every group, prefix-summed into LDS; returns the total.
template <int D>
__device__ inline int plan_items(const AttendParams& P, AttendSmem<D>& sm) {
  const int BH = P.B * P.H_kv;
  const int per = (BH + blockDim.x - 1) / blockDim.x;
  const int g0 = threadIdx.x * per;
  int mine = 0;
  for (int k = 0; k < per; ++k)
    if (g0 + k < BH) mine += group_info(P, g0 + k).items;
  int total = 0;
  int acc = block_exclusive_scan<int>(mine, sm.scan, &total);
  for (int k = 0; k < per; ++k)
    if (g0 + k < BH) {
      sm.item_prefix[g0 + k] = acc;
      acc += group_info(P, g0 + k).items;
    }
  if (threadIdx.x == 0) sm.item_prefix[BH] = total;
  __syncthreads();
  return total;
}

__device__ inline int find_group(const int32_t* prefix, int BH, int item) {
  int lo = 0, hi = BH;  // prefix[lo] <= item < prefix[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= item) lo = mid; else hi = mid;
  }
  return lo;
}

// WG-level merge of the per-wave states into one partial per query head;
// st(w, g, c) reads entry c of head g of wave w's state.
template <int D, typename ST>
__device__ inline void write_partial_state(const AttendParams& P, ST st, int gi, int item) {
  const int G = P.G;
  for (int idx = threadIdx.x; idx < G * (D + 2); idx += blockDim.x) {
    const int g = idx / (D + 2), c = idx % (D + 2);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWavesPerWg; ++w) M = fmaxf(M, st(w, g, 0));
    float v;
    if (c == 0) {
      v = M;
    } else {
      v = 0.0f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < kWavesPerWg; ++w) {
          const float mw = st(w, g, 0);
          if (mw != -INFINITY) v += st(w, g, c) * exp2f(mw - M);
        }
      }
    }
    const int64_t head = (int64_t)gi * G + g;
    P.part[(head * P.split_cap + item) * (D + 2) + c] = v;
  }
}

template <int D>
__device__ inline void write_partial(const AttendParams& P, AttendSmem<D>& sm, int gi,
                                     int item) {
  write_partial_state<D>(P, [&](int w, int g, int c) { return sm.state[w][g][c]; }, gi, item);
}

// ---------------------------------------------------------------- bf16 path
//
// QK^T on MFMA 16x16x32 bf16: rows = 16 keys, columns = the group's query heads
// (padded to 16), contraction over d in steps of 32.  The fp32 query (times
// scale*log2e) is split into two bf16 parts hi + lo, whose sum carries it to
// ~2^-17 relative (score error ~1e-4 at d = 128, far inside what bf16 keys
// allow); both products accumulate in fp32.  Lane l supplies row/column l%16
// and the 8 consecutive dims s*32 + (l/16)*8 of step s for both operands, so
// each lane's K load is 16 contiguous bytes.  P V on MFMA 16x16x16 bf16 (see
// compute_chunk); V rows load 16 bytes per lane, coalesced, and pass through
// the wave's LDS tile.
//
// Each wave walks 16-key chunks of an item (chunks w, w+4, ...).  When every
// chunk is 16 consecutive cache rows under one head mask (dense, or leaves of
// C >= 16 keys) the chunk's address and mask are wave-uniform and the next
// chunk's K/V loads are issued before the current chunk is computed (two
// register buffers).  Otherwise (the tail item with the sink and the open chunk,
// or C < 16) each key's row is looked up per lane.  The item's leaf entries are
// staged in LDS once.  The running max is raised lazily: only when a chunk's max
// exceeds it by more than kLazy (log2 units) are o and l rescaled, so
// probabilities stay below 2^kLazy.

constexpr float kLazy = 8.0f;
constexpr int kItemKeys = kTilesPerItem * kTileKeys;   // 1024

// A wave's LDS: the current chunk's V rows (bf16, rows padded by 32 bytes so
// the transposing reads spread over the banks), or, once the wave's chunks are
// done, its (m, l, o) state for the workgroup merge.  16-byte aligned: the rows
// are written 16 bytes at a time and read 8 at a time.
template <int D, int GP>
union __attribute__((aligned(16))) WaveBuf {
  uint16_t vt[16][D + 16];
  float state[GP][D + 2];
};

template <int D, int GP>
struct AttendSmemB {
  int32_t item_prefix[kMaxGroups + 1];
  int32_t scan[16];
  int32_t lid[kItemKeys / 2 + 2];               // leaf ids of the item (C >= 2)
  uint32_t lmask[kItemKeys / 2 + 2];
  WaveBuf<D, GP> wb[kWavesPerWg];
};

// Where the keys of one work item come from.
struct ItemView {
  int tail;           // 1: the sink + open-chunk item
  int64_t kbase;      // first list key of the item
  int nkeys;          // keys in the item
  int64_t first;      // first leaf entry staged in LDS
  int cshift;         // log2 C
  uint32_t smask;     // sink mask (tail item)
};

template <typename SM>
__device__ inline Slot item_slot(const AttendParams& P, const SM& sm, const GroupInfo& g,
                                 const ItemView& it, int e, uint32_t full) {
  Slot s{0, 0u};
  if (e >= it.nkeys) return s;
  if (it.tail) {
    if (e == 0) { s.mask = it.smask; }
    else {
      const int64_t t = (int64_t)g.n1 * P.C + (e - 1);
      if (t < g.T) { s.tok = (int32_t)t; s.mask = full; }
    }
    return s;
  }
  const int64_t gk = it.kbase + e;
  if (P.leaf_ids == nullptr) {
    s.tok = (int32_t)gk;
    s.mask = full;
    return s;
  }
  const int loc = (int)((gk >> it.cshift) - it.first);
  s.tok = sm.lid[loc] * P.C + (int32_t)(gk & (P.C - 1));
  s.mask = sm.lmask[loc];
  return s;
}

template <int D>
struct ChunkBuf {
  u32x4_t k[D / 32];
  u32x4_t v[16 / (kWave / (D / 8))];
  uint32_t kmask;     // head mask of this lane's K column key
  uint32_t vok;       // bit i: V row i holds an attended key
};

// General chunk load: rows looked up per lane.
template <int D, typename SM>
__device__ inline void load_chunk_any(const AttendParams& P, const SM& sm, const GroupInfo& g,
                                      const ItemView& it, int chunk, uint32_t full,
                                      int64_t kv_base, int lane, ChunkBuf<D>& buf) {
  constexpr int KSTEPS = D / 32, LPR = D / 8, RPI = kWave / LPR, VL = 16 / RPI;
  const uint16_t* Kb = (const uint16_t*)P.K;
  const uint16_t* Vb = (const uint16_t*)P.V;
  const Slot ks = item_slot(P, sm, g, it, chunk * 16 + (lane & 15), full);
  buf.kmask = ks.mask;
  const uint16_t* krow = Kb + (kv_base + ks.tok) * D + (lane >> 4) * 8;
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) buf.k[s] = __builtin_nontemporal_load((const u32x4_t*)(krow + s * 32));
  buf.vok = 0u;
#pragma unroll
  for (int i = 0; i < VL; ++i) {
    const Slot vs = item_slot(P, sm, g, it, chunk * 16 + RPI * i + lane / LPR, full);
    buf.v[i] = __builtin_nontemporal_load((const u32x4_t*)(Vb + (kv_base + vs.tok) * D + (lane % LPR) * 8));
    buf.vok |= (vs.mask ? 1u : 0u) << i;
  }
}

// Contiguous chunk load: rows row0 .. row0+nv-1 of the group under one head mask
// (row0, nv, hm wave-uniform).  Lanes past nv re-read row row0 and are masked.
template <int D>
__device__ inline void load_chunk_rows(const uint16_t* klane, const uint16_t* vlane, int lane,
                                       int64_t row0, int nv, uint32_t hm, ChunkBuf<D>& buf) {
  constexpr int KSTEPS = D / 32, LPR = D / 8, RPI = kWave / LPR, VL = 16 / RPI;
  const int kr = lane & 15;
  const int kof = kr < nv ? kr : 0;
  const uint16_t* kp = klane + (row0 + kof) * D;
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) buf.k[s] = __builtin_nontemporal_load((const u32x4_t*)(kp + s * 32));
  buf.vok = 0u;
#pragma unroll
  for (int i = 0; i < VL; ++i) {
    const int vr = RPI * i + lane / LPR;
    const int vof = vr < nv ? vr : 0;
    buf.v[i] = __builtin_nontemporal_load((const u32x4_t*)(vlane + (row0 + vof) * D));
    buf.vok |= (vr < nv && hm != 0u ? 1u : 0u) << i;
  }
  buf.kmask = kr < nv ? hm : 0u;
}

typedef short bf16x4_t __attribute__((ext_vector_type(4)));   // bf16 bits

// One 16-key chunk of a wave.  QK^T runs with K as the A operand, so lane l
// holds the scores of head l % 16 for keys 4(l/16) + i (i < 4): exactly the A
// operand layout of P V (16x16x16 MFMA, rows = heads, k = keys).  P enters as
// two bf16 terms (hi + lo, ~2^-17 relative).  V's B operand comes from the
// wave's LDS tile by a transposing read: lane m addresses 4 dims of row m / 4,
// and receives dims 16t + m % 16 of rows 4(m / 16) .. + 3.  o[t][i] is the
// output of head 4(l/16) + i, dim 16t + l % 16.  m_run, l_run belong to head
// l % 16 (l_run: this lane's keys only).
template <int D, int GP>
__device__ inline void compute_chunk(WaveBuf<D, GP>& wb, const ChunkBuf<D>& buf,
                                     const bf16x8_t* a_hi, const bf16x8_t* a_lo, int lane,
                                     float& m_run, float& l_run, f32x4_t (&o)[D / 16]) {
  constexpr int KSTEPS = D / 32, LPR = D / 8, RPI = kWave / LPR, VL = 16 / RPI;
  const int h = lane & 15, k0 = (lane >> 4) * 4;
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    const bf16x8_t kb = __builtin_bit_cast(bf16x8_t, buf.k[s]);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, a_hi[s], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, a_lo[s], acc, 0, 0, 0);
  }
  float cm = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t km = __shfl(buf.kmask, k0 + i, 64);   // key k0+i's head mask
    acc[i] = ((km >> h) & 1u) ? acc[i] : -INFINITY;
    cm = fmaxf(cm, acc[i]);
  }
  cm = fmaxf(cm, swz_xor<16>(cm));
  cm = fmaxf(cm, shfl_xor32(cm));
  const bool need = cm > m_run + kLazy;
  if (__ballot(need) != 0ull) {           // wave-uniform: raise some running maxima
    const float mnew = need ? cm : m_run;
    const float al = (mnew == -INFINITY) ? 1.0f : exp2f(m_run - mnew);
    l_run *= al;
    m_run = mnew;
    float ar[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ar[i] = __shfl(al, k0 + i, 64);   // heads of o's rows
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[t][i] *= ar[i];
  }
  bf16x4_t p_hi, p_lo;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float pv = (acc[i] == -INFINITY) ? 0.0f : exp2f(acc[i] - m_run);
    l_run += pv;
    const uint16_t hi = f32_to_bf16_rne(pv);
    p_hi[i] = (short)hi;
    p_lo[i] = (short)f32_to_bf16_rne(pv - __uint_as_float((uint32_t)hi << 16));
  }
  // the chunk's V rows into the tile; rows of keys nobody attends are zero
#pragma unroll
  for (int i = 0; i < VL; ++i) {
    const bool ok = (buf.vok >> i) & 1u;
    u32x4_t v = buf.v[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = ok ? v[j] : 0u;
    *(u32x4_t*)&wb.vt[RPI * i + lane / LPR][(lane % LPR) * 8] = v;
  }
  wave_lds_sync();
  typedef __attribute__((address_space(3))) __bf16 lds_bf16_t;
  typedef __bf16 bf16x4v_t __attribute__((__vector_size__(4 * sizeof(__bf16))));
  typedef __attribute__((address_space(3))) bf16x4v_t lds_bf16x4_t;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    lds_bf16x4_t* src = (lds_bf16x4_t*)(lds_bf16_t*)(&wb.vt[lane >> 2][16 * t + 4 * (lane & 3)]);
    const bf16x4_t vb = __builtin_bit_cast(bf16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(src));
    o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(p_hi, vb, o[t], 0, 0, 0);
    o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(p_lo, vb, o[t], 0, 0, 0);
  }
  wave_lds_sync();                        // the next chunk's rows overwrite the tile
}

// A wave's totals into its LDS state: l summed over the four key groups (o is
// already summed over the keys by the MFMA).
template <int D, int GP>
__device__ inline void wave_state_out(WaveBuf<D, GP>& wb, int lane, float m_run, float l_run,
                                      const f32x4_t (&o)[D / 16]) {
  float l = l_run;
  l += swz_xor<16>(l);
  l += shfl_xor32(l);
  if (lane < GP) { wb.state[lane][0] = m_run; wb.state[lane][1] = l; }
  const int h0 = (lane >> 4) * 4, c = lane & 15;
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (h0 + i < GP) wb.state[h0 + i][2 + 16 * t + c] = o[t][i];
}

template <int D, int GP, bool CONTIG>
__global__ void __launch_bounds__(256, 2)
attend_partial_bf16(AttendParams P) {
  touch_args(P);
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(GP == 4 || GP == 8 || GP == 16, "padded heads");
  constexpr int KSTEPS = D / 32;
  constexpr int LPR = D / 8;
  __shared__ AttendSmemB<D, GP> sm;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int BH = P.B * P.H_kv;
  const uint32_t full = (P.G >= 32) ? 0xffffffffu : ((1u << P.G) - 1u);
  const int cshift = __ffs(P.C) - 1;

  // work items of every group, prefix-summed into LDS
  int total;
  {
    const int per = (BH + blockDim.x - 1) / blockDim.x;
    const int g0 = threadIdx.x * per;
    int mine = 0;
    for (int k = 0; k < per; ++k)
      if (g0 + k < BH) mine += group_info(P, g0 + k).items;
    int acc = block_exclusive_scan<int>(mine, sm.scan, &total);
    for (int k = 0; k < per; ++k)
      if (g0 + k < BH) {
        sm.item_prefix[g0 + k] = acc;
        acc += group_info(P, g0 + k).items;
      }
    if (threadIdx.x == 0) sm.item_prefix[BH] = total;
    __syncthreads();
  }

  bf16x8_t a_hi[KSTEPS], a_lo[KSTEPS];
  const int item_keys = P.item_tiles * kTileKeys;   // <= kItemKeys
  const int span_max = (item_keys >> cshift) + 1;   // leaf entries an item can touch

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int gi = find_group(sm.item_prefix, BH, item);
    const int li = item - sm.item_prefix[gi];
    // Every load of the item's prologue goes out before any is waited on: the
    // group's geometry, the leaf entries the item could span (clamped to the
    // row; the ones past the list are dropped below) and the group's queries.
    const GroupRaw graw = group_raw(P, gi);
    const int64_t first0 = ((int64_t)li * item_keys) >> cshift;
    const bool one_pass = span_max <= (int)blockDim.x;
    int32_t e_id = 0;
    uint32_t e_m = 0u;
    if (P.leaf_ids != nullptr && one_pass && P.leaf_cap > 0) {
      const int64_t e = min(first0 + (int64_t)threadIdx.x, (int64_t)P.leaf_cap - 1);
      e_id = P.leaf_ids[(int64_t)gi * P.leaf_cap + e];
      e_m = P.leaf_mask[(int64_t)gi * P.leaf_cap + e];
    }
    const int row = lane & 15;
    const int kg = lane >> 4;
    const float* qrow = P.q + ((int64_t)gi * P.G + (row < P.G ? row : P.G - 1)) * D + kg * 8;
    float qx[KSTEPS][8];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) qx[s][j] = qrow[s * 32 + j];
    const GroupInfo g = group_info_from(P, graw);
    {
      const float f = row < P.G ? P.qscale : 0.0f;   // padding rows are zero
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        bf16x8_t hi, lo;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = qx[s][j] * f;
          const uint16_t h16 = f32_to_bf16_rne(x);
          const float r1 = x - __uint_as_float((uint32_t)h16 << 16);
          const uint16_t l16 = f32_to_bf16_rne(r1);
          hi[j] = __builtin_bit_cast(__bf16, h16);
          lo[j] = __builtin_bit_cast(__bf16, l16);
        }
        a_hi[s] = hi; a_lo[s] = lo;
      }
    }

    ItemView it;
    it.tail = (li == g.items - 1) ? 1 : 0;
    it.cshift = cshift;
    it.smask = 0u;
    it.first = 0;
    if (it.tail) {
      it.kbase = 0;
      it.nkeys = kTileKeys;
      it.smask = sink_mask_from(P, g, graw, full);
    } else {
      it.kbase = (int64_t)li * item_keys;
      const int64_t left = (int64_t)g.U * P.C - it.kbase;
      it.nkeys = (int)(left < item_keys ? left : item_keys);
      if (P.leaf_ids != nullptr) {
        it.first = first0;
        const int64_t last = (it.kbase + it.nkeys - 1) >> cshift;
        const int cnt = (int)(last - it.first + 1);
        if (one_pass) {
          if ((int)threadIdx.x < cnt) {
            int32_t leaf = e_id;
            uint32_t m = e_m & full;
            if (leaf < 0 || leaf >= g.n1) { leaf = 0; m = 0u; }
            sm.lid[threadIdx.x] = leaf;
            sm.lmask[threadIdx.x] = m;
          }
        } else {
          for (int i = threadIdx.x; i < cnt; i += blockDim.x) {
            const int64_t off = (int64_t)gi * P.leaf_cap + it.first + i;
            int32_t leaf = P.leaf_ids[off];
            uint32_t m = P.leaf_mask[off] & full;
            if (leaf < 0 || leaf >= g.n1) { leaf = 0; m = 0u; }
            sm.lid[i] = leaf;
            sm.lmask[i] = m;
          }
        }
      }
    }
    __syncthreads();

    float m_run = -INFINITY, l_run = 0.0f;
    f32x4_t o[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) o[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const int64_t kv_base = (int64_t)gi * P.T_cap;
    if constexpr (CONTIG) {
      // Chunks of consecutive rows.  Regular item: 16-key chunks of the list.
      // Tail item: chunk 0 is the sink row, then the open chunk in 16-row pieces.
      const int64_t open0 = (int64_t)g.n1 * P.C;
      const int open_len = (int)(g.T - open0);
      const int nchunks = it.tail ? 1 + (open_len + 15) / 16 : (it.nkeys + 15) / 16;
      const uint16_t* klane = (const uint16_t*)P.K + kv_base * D + (lane >> 4) * 8;
      const uint16_t* vlane = (const uint16_t*)P.V + kv_base * D + (lane % LPR) * 8;
      auto chunk_src = [&](int c, int64_t& row0, int& nv, uint32_t& hm) {
        if (it.tail) {
          if (c == 0) { row0 = 0; nv = 1; hm = it.smask; }
          else {
            row0 = open0 + 16 * (c - 1);
            nv = min(16, (int)(g.T - row0));
            hm = full;
          }
        } else {
          const int64_t gk = it.kbase + (int64_t)c * 16;
          nv = min(16, it.nkeys - 16 * c);   // partial only when C < 16 (dense)
          if (P.leaf_ids == nullptr) { row0 = gk; hm = full; }
          else {
            const int loc = (int)((gk >> cshift) - it.first);
            row0 = (int64_t)sm.lid[loc] * P.C + (gk & (P.C - 1));
            hm = sm.lmask[loc];
          }
        }
        row0 = __builtin_amdgcn_readfirstlane((int)row0);
        hm = __builtin_amdgcn_readfirstlane(hm);
      };
      // rotating buffer: chunk c+4's loads are in flight while chunk c computes
      ChunkBuf<D> cur, nxt;
      int64_t r0; int nv; uint32_t hm;
      int c = wave;
      if (c < nchunks) { chunk_src(c, r0, nv, hm); load_chunk_rows<D>(klane, vlane, lane, r0, nv, hm, cur); }
      for (; c < nchunks; c += kWavesPerWg) {
        const bool more = c + kWavesPerWg < nchunks;
        if (more) {
          chunk_src(c + kWavesPerWg, r0, nv, hm);
          load_chunk_rows<D>(klane, vlane, lane, r0, nv, hm, nxt);
        }
        compute_chunk<D, GP>(sm.wb[wave], cur, a_hi, a_lo, lane, m_run, l_run, o);
        if (more) cur = nxt;
      }
    } else {
      // gathered rows (leaves of C < 16 keys); the same rotating buffer: chunk
      // k+4's rows are in flight while chunk k computes
      const int nchunks = (it.nkeys + 15) / 16;
      ChunkBuf<D> cur, nxt;
      int k = wave;
      if (k < nchunks) load_chunk_any<D>(P, sm, g, it, k, full, kv_base, lane, cur);
      for (; k < nchunks; k += kWavesPerWg) {
        const bool more = k + kWavesPerWg < nchunks;
        if (more) load_chunk_any<D>(P, sm, g, it, k + kWavesPerWg, full, kv_base, lane, nxt);
        compute_chunk<D, GP>(sm.wb[wave], cur, a_hi, a_lo, lane, m_run, l_run, o);
        if (more) cur = nxt;
      }
    }

    wave_state_out<D, GP>(sm.wb[wave], lane, m_run, l_run, o);
    __syncthreads();
    write_partial_state<D>(P, [&](int w, int g, int c) { return sm.wb[w].state[g][c]; }, gi, li);
    __syncthreads();
  }
}

// ---------------------------------------------- bf16 path, pipelined over segments
//
// The contiguous-chunk kernel (dense, or leaves of C >= 16 keys).  Everything a
// segment needs besides its K/V rows is fetched while the previous segment is
// being computed, so a workgroup always has K/V loads in flight:
//   * per-group geometry (list length, leaf count, open-chunk length, sink mask)
//     and the chunk prefix are computed once per workgroup into LDS;
//   * the next segment's leaf entries and, when its group changes, its queries
//     are loaded into registers during the current segment's chunk loop and
//     moved to LDS after it (leaf entries into the other of two buffers);
//   * each wave issues the K/V loads of its first chunk of the next segment
//     before the current run's per-wave states are merged and written.

template <int D, int GP>
struct PipeSmem {
  int32_t chunk_prefix[kMaxGroups + 1];   // group-ordered offsets of the groups' chunks
  int32_t g_U[kMaxGroups];           // leaf-list entries (dense: complete leaves)
  int32_t g_n1[kMaxGroups];          // complete leaves
  int32_t g_open[kMaxGroups];        // open-chunk length T - C n1
  uint32_t g_smask[kMaxGroups];      // heads that take the sink from the tail
  int32_t scan[16];
  int32_t lid[2][kItemKeys / 16 + 2];    // leaf entries of the current / next segment (C >= 16)
  uint32_t lmask[2][kItemKeys / 16 + 2];
  float qs[GP * D];                  // the current group's queries, times scale*log2(e)
  WaveBuf<D, GP> wb[kWavesPerWg];
};

constexpr int kItemChunks = kItemKeys / 16;   // 16-key chunks of a work item

// One segment of a workgroup's range: chunks of one group inside one work item
// (1024 list keys), or of the group's tail (the sink chunk, then the open chunk
// in 16-row pieces).
struct PipeItem {
  int gi;
  int tail;          // 1: tail chunks
  int c0;            // tail: first tail chunk (0 is the sink)
  int64_t kbase;     // first list key (list segments)
  int nkeys;         // list keys in the segment
  int64_t first;     // first leaf entry of the segment
  int nent;          // leaf entries touched
  int nchunks;
};

// Chunks of group gi's leaf list (16 keys each; the last one may be partial).
template <int D, int GP>
__device__ inline int list_chunks(const PipeSmem<D, GP>& sm, int gi, int cshift) {
  return (int)((((int64_t)sm.g_U[gi] << cshift) + 15) / 16);
}

// The segment starting at global chunk cur, clipped to the range end c_end.
template <int D, int GP>
__device__ inline PipeItem pipe_seg(const AttendParams& P, const PipeSmem<D, GP>& sm, int BH,
                                    int cur, int c_end, int cshift) {
  PipeItem it;
  it.gi = find_group(sm.chunk_prefix, BH, cur);
  const int base = sm.chunk_prefix[it.gi];
  const int local = cur - base;
  const int lim = min(c_end, sm.chunk_prefix[it.gi + 1]) - base;   // local end in range
  const int nlist = list_chunks<D, GP>(sm, it.gi, cshift);
  it.kbase = 0; it.nkeys = 0; it.first = 0; it.nent = 0; it.c0 = 0;
  if (local >= nlist) {
    it.tail = 1;
    it.c0 = local - nlist;
    it.nchunks = lim - local;
  } else {
    it.tail = 0;
    const int iend = min((local / kItemChunks + 1) * kItemChunks, nlist);
    it.nchunks = min(iend, lim) - local;
    it.kbase = (int64_t)local * 16;
    const int64_t left = ((int64_t)sm.g_U[it.gi] << cshift) - it.kbase;
    const int64_t span = (int64_t)it.nchunks * 16;
    it.nkeys = (int)(left < span ? left : span);
    if (P.leaf_ids != nullptr) {
      it.first = it.kbase >> cshift;
      it.nent = (int)(((it.kbase + it.nkeys - 1) >> cshift) - it.first + 1);
    }
  }
  return it;
}

// Rows of chunk c of a segment: row0 .. row0+nv-1 of the group under head mask
// hm.  ent_id / ent_mask: the leaf entry covering the chunk (sparse list segments).
template <int D, int GP>
__device__ inline void pipe_chunk_rows(const AttendParams& P, const PipeSmem<D, GP>& sm,
                                       const PipeItem& it, int c, int cshift, uint32_t full,
                                       int32_t ent_id, uint32_t ent_mask,
                                       int64_t& row0, int& nv, uint32_t& hm) {
  if (it.tail) {
    const int tc = it.c0 + c;
    if (tc == 0) { row0 = 0; nv = 1; hm = sm.g_smask[it.gi]; }
    else {
      const int off = 16 * (tc - 1);
      row0 = ((int64_t)sm.g_n1[it.gi] << cshift) + off;
      nv = min(16, sm.g_open[it.gi] - off);
      hm = full;
    }
  } else {
    const int64_t gk = it.kbase + (int64_t)c * 16;
    nv = min(16, it.nkeys - 16 * c);     // partial only when C < 16 (dense)
    if (P.leaf_ids == nullptr) { row0 = gk; hm = full; }
    else { row0 = (int64_t)ent_id * P.C + (gk & (P.C - 1)); hm = ent_mask; }
  }
  row0 = __builtin_amdgcn_readfirstlane((int)row0);
  nv = __builtin_amdgcn_readfirstlane(nv);
  hm = __builtin_amdgcn_readfirstlane(hm);
}

// The pipelined kernel gives workgroup w the contiguous chunks
// [run_start(w), run_start(w + 1)) of the group-ordered chunk list (16 keys of a
// group's leaf list, or a piece of its tail; the grid is clamped to the chunk
// count, so no range is empty): the ranges differ by at most one chunk.
// Consecutive segments of one group fold into one running state, so a group's
// partials are one per workgroup whose range meets it: slot
// w - run_owner(first chunk of the group).
__device__ inline int run_start(int w, int total, int grid) {
  return (int)((int64_t)total * w / grid);
}
__device__ inline int run_owner(int chunk, int total, int grid) {
  return (int)(((int64_t)(chunk + 1) * grid - 1) / total);
}
// Workgroups that take a range: at most the launched ones, and few enough that
// every range holds at least kMinRunChunks chunks (which bounds a group's
// partials by the slots the workspace holds per head).
__device__ inline int run_grid(int launched, int total) {
  const int g = total / kMinRunChunks;
  return max(1, min(launched, g));
}

template <int D, int GP>
__global__ void __launch_bounds__(256, 2)
attend_partial_bf16_pipe(AttendParams P) {
  touch_args(P);
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(GP == 4 || GP == 8 || GP == 16, "padded heads");
  constexpr int KSTEPS = D / 32;
  constexpr int LPR = D / 8;
  constexpr int QPT = (GP * D + 255) / 256;    // query floats per thread when staging
  __shared__ PipeSmem<D, GP> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int BH = P.B * P.H_kv;
  const uint32_t full = (P.G >= 32) ? 0xffffffffu : ((1u << P.G) - 1u);
  const int cshift = __ffs(P.C) - 1;

  // ---- per-group geometry and the chunk prefix, once per workgroup
  int total;
  {
    const int per = (BH + blockDim.x - 1) / blockDim.x;
    const int g0 = tid * per;
    int mine = 0;
    for (int k = 0; k < per; ++k) {
      const int gi = g0 + k;
      if (gi < BH) {
        const GroupRaw r = group_raw(P, gi);
        const GroupInfo g = group_info_from(P, r);
        sm.g_U[gi] = g.U;
        sm.g_n1[gi] = g.n1;
        sm.g_open[gi] = (int)(g.T - (int64_t)g.n1 * P.C);
        sm.g_smask[gi] = sink_mask_from(P, g, r, full);
        mine += list_chunks<D, GP>(sm, gi, cshift) + 1 + (sm.g_open[gi] + 15) / 16;
      }
    }
    int acc = block_exclusive_scan<int>(mine, sm.scan, &total);
    for (int k = 0; k < per; ++k)
      if (g0 + k < BH) {
        sm.chunk_prefix[g0 + k] = acc;
        acc += list_chunks<D, GP>(sm, g0 + k, cshift) + 1 + (sm.g_open[g0 + k] + 15) / 16;
      }
    if (tid == 0) sm.chunk_prefix[BH] = total;
    __syncthreads();
  }
  const int gridp = run_grid((int)gridDim.x, total);
  if ((int)blockIdx.x >= gridp) return;
  if (blockIdx.x == 0)
    for (int k = tid; k <= BH; k += blockDim.x) P.prefix[k] = sm.chunk_prefix[k];
  int cur_c = run_start(blockIdx.x, total, gridp);
  const int c_end = run_start(blockIdx.x + 1, total, gridp);

  // ---- the first segment: staged synchronously
  PipeItem it = pipe_seg<D, GP>(P, sm, BH, cur_c, c_end, cshift);
  int pb = 0;   // leaf-entry buffer of the current segment
  if (!it.tail && P.leaf_ids != nullptr && tid < it.nent) {
    const int64_t off = (int64_t)it.gi * P.leaf_cap + it.first + tid;
    int32_t leaf = P.leaf_ids[off];
    uint32_t m = P.leaf_mask[off] & full;
    if (leaf < 0 || leaf >= sm.g_n1[it.gi]) { leaf = 0; m = 0u; }
    sm.lid[pb][tid] = leaf;
    sm.lmask[pb][tid] = m;
  }
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int idx = tid + 256 * k;
    if (idx < GP * D)
      sm.qs[idx] = (idx < P.G * D) ? P.q[(int64_t)it.gi * P.G * D + idx] * P.qscale : 0.0f;
  }
  __syncthreads();

  bf16x8_t a_hi[KSTEPS], a_lo[KSTEPS];
  auto convert_q = [&]() {
    const int row = lane & 15;
    const int kg = lane >> 4;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      bf16x8_t hi, lo;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = (row < GP) ? sm.qs[row * D + s * 32 + kg * 8 + j] : 0.0f;
        const uint16_t h16 = f32_to_bf16_rne(x);
        const float r1 = x - __uint_as_float((uint32_t)h16 << 16);
        const uint16_t l16 = f32_to_bf16_rne(r1);
        hi[j] = __builtin_bit_cast(__bf16, h16);
        lo[j] = __builtin_bit_cast(__bf16, l16);
      }
      a_hi[s] = hi; a_lo[s] = lo;
    }
  };
  convert_q();

  ChunkBuf<D> cur, nxt;
  {
    int64_t r0; int nv; uint32_t hm;
    if (wave < it.nchunks) {
      int32_t eid = 0; uint32_t em = 0u;
      if (!it.tail && P.leaf_ids != nullptr) {
        const int loc = (int)(((it.kbase + 16 * wave) >> cshift) - it.first);
        eid = sm.lid[pb][loc]; em = sm.lmask[pb][loc];
      }
      pipe_chunk_rows<D, GP>(P, sm, it, wave, cshift, full, eid, em, r0, nv, hm);
      const int64_t kv_base = (int64_t)it.gi * P.T_cap;
      load_chunk_rows<D>((const uint16_t*)P.K + kv_base * D + (lane >> 4) * 8,
                         (const uint16_t*)P.V + kv_base * D + (lane % LPR) * 8, lane, r0, nv, hm, cur);
    }
  }

  // running state of the current run of same-group segments
  float m_run = -INFINITY, l_run = 0.0f;
  f32x4_t o[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) o[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  for (;;) {
    // ---- prefetch what the next segment needs besides K/V
    const int next_c = cur_c + it.nchunks;
    const bool has_next = next_c < c_end;
    PipeItem nx = it;
    if (has_next) nx = pipe_seg<D, GP>(P, sm, BH, next_c, c_end, cshift);
    const bool new_q = has_next && nx.gi != it.gi;
    int32_t pf_id = 0;
    uint32_t pf_m = 0u;
    if (has_next && !nx.tail && P.leaf_ids != nullptr && tid < nx.nent) {
      const int64_t off = (int64_t)nx.gi * P.leaf_cap + nx.first + tid;
      pf_id = P.leaf_ids[off];
      pf_m = P.leaf_mask[off];
    }
    float pf_q[QPT];
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int idx = tid + 256 * k;
      pf_q[k] = (new_q && idx < P.G * D) ? P.q[(int64_t)nx.gi * P.G * D + idx] : 0.0f;
    }
    // this wave's first chunk of the next segment: its leaf entry
    int32_t nf_id = 0;
    uint32_t nf_m = 0u;
    if (has_next && !nx.tail && P.leaf_ids != nullptr && wave < nx.nchunks) {
      const int64_t e = (nx.kbase + 16 * wave) >> cshift;
      const int64_t off = (int64_t)nx.gi * P.leaf_cap + e;
      nf_id = P.leaf_ids[off];
      nf_m = P.leaf_mask[off] & full;
      if (nf_id < 0 || nf_id >= sm.g_n1[nx.gi]) { nf_id = 0; nf_m = 0u; }
    }

    // ---- the current segment's chunks: chunk c+4's loads in flight while c computes
    {
      const int64_t kv_base = (int64_t)it.gi * P.T_cap;
      const uint16_t* klane = (const uint16_t*)P.K + kv_base * D + (lane >> 4) * 8;
      const uint16_t* vlane = (const uint16_t*)P.V + kv_base * D + (lane % LPR) * 8;
      for (int c = wave; c < it.nchunks; c += kWavesPerWg) {
        const bool more = c + kWavesPerWg < it.nchunks;
        if (more) {
          int32_t eid = 0; uint32_t em = 0u;
          if (!it.tail && P.leaf_ids != nullptr) {
            const int loc = (int)(((it.kbase + 16 * (c + kWavesPerWg)) >> cshift) - it.first);
            eid = sm.lid[pb][loc]; em = sm.lmask[pb][loc];
          }
          int64_t r0; int nv; uint32_t hm;
          pipe_chunk_rows<D, GP>(P, sm, it, c + kWavesPerWg, cshift, full, eid, em, r0, nv, hm);
          load_chunk_rows<D>(klane, vlane, lane, r0, nv, hm, nxt);
        }
        compute_chunk<D, GP>(sm.wb[wave], cur, a_hi, a_lo, lane, m_run, l_run, o);
        if (more) cur = nxt;
      }
    }

    // ---- issue the next segment's first chunk before merging this one
    if (has_next && wave < nx.nchunks) {
      int64_t r0; int nv; uint32_t hm;
      pipe_chunk_rows<D, GP>(P, sm, nx, wave, cshift, full, nf_id, nf_m, r0, nv, hm);
      const int64_t kv_base = (int64_t)nx.gi * P.T_cap;
      load_chunk_rows<D>((const uint16_t*)P.K + kv_base * D + (lane >> 4) * 8,
                         (const uint16_t*)P.V + kv_base * D + (lane % LPR) * 8, lane, r0, nv, hm, cur);
    }
    // ---- the next segment's entries into the other buffer: nobody reads it
    // (its last readers, two segments back, passed the previous barrier)
    if (has_next && !nx.tail && P.leaf_ids != nullptr && tid < nx.nent) {
      if (pf_id < 0 || pf_id >= sm.g_n1[nx.gi]) { pf_id = 0; pf_m = 0u; }
      sm.lid[pb ^ 1][tid] = pf_id;
      sm.lmask[pb ^ 1][tid] = pf_m & full;
    }

    // ---- the run ends at a group change or at the range's end: the wave's
    // totals, then the workgroup's partial
    if (!has_next || new_q) {
      wave_state_out<D, GP>(sm.wb[wave], lane, m_run, l_run, o);
      __syncthreads();
      const int slot = blockIdx.x - run_owner(sm.chunk_prefix[it.gi], total, gridp);
      if (slot < P.split_cap)
        write_partial_state<D>(P, [&](int w, int g, int c) { return sm.wb[w].state[g][c]; },
                               it.gi, slot);
      else if (tid == 0)
        set_status(P.status, ZHA_ECAPACITY);
      m_run = -INFINITY;
      l_run = 0.0f;
#pragma unroll
      for (int t = 0; t < D / 16; ++t) o[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
    if (!has_next) break;
    // every wave is done with this segment (its LDS tiles, states and leaf
    // entries); the next segment's entries are visible after this barrier
    __syncthreads();
    if (new_q) {
      // a new group's queries: every wave is past the previous staging's reads
#pragma unroll
      for (int k = 0; k < QPT; ++k) {
        const int idx = tid + 256 * k;
        if (idx < GP * D) sm.qs[idx] = pf_q[k] * P.qscale;
      }
      __syncthreads();
      convert_q();
    }
    cur_c = next_c;
    it = nx;
    pb ^= 1;
  }
}

// ---------------------------------------------------------------- fp32 path
//
// fp32 K/V (exact-precision runs): VALU only.  Lane = key slot for the scores
// (q broadcast from LDS); lane = dims for P V.

template <int D, int GP>
__global__ void __launch_bounds__(256)
attend_partial_f32(AttendParams P) {
  touch_args(P);
  constexpr int DPL = D / kWave;            // dims per lane in P V
  __shared__ AttendSmem<D> sm;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int BH = P.B * P.H_kv;
  const int total = plan_items<D>(P, sm);
  const uint32_t full = (P.G >= 32) ? 0xffffffffu : ((1u << P.G) - 1u);
  const float* Kf = (const float*)P.K;
  const float* Vf = (const float*)P.V;

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int gi = find_group(sm.item_prefix, BH, item);
    const int li = item - sm.item_prefix[gi];
    const GroupRaw graw = group_raw(P, gi);
    const GroupInfo g = group_info_from(P, graw);
    for (int idx = threadIdx.x; idx < 16 * D; idx += blockDim.x) {
      const int hh = idx / D, c = idx % D;
      sm.qf[hh][c] = (hh < P.G) ? P.q[((int64_t)gi * P.G + hh) * D + c] * P.qscale : 0.0f;
    }
    __syncthreads();

    const bool tail = (li == g.items - 1);
    const uint32_t smask = tail ? sink_mask_from(P, g, graw, full) : 0u;
    int tile, t_end, t_step;
    if (tail) { tile = (wave == 0) ? -1 : 0; t_end = 0; t_step = 1; }
    else {
      tile = li * P.item_tiles + wave;
      t_end = min(g.tiles, (li + 1) * P.item_tiles);
      t_step = kWavesPerWg;
    }
    float m[GP], l[GP], o[GP][DPL];
#pragma unroll
    for (int hh = 0; hh < GP; ++hh) {
      m[hh] = -INFINITY; l[hh] = 0.0f;
#pragma unroll
      for (int j = 0; j < DPL; ++j) o[hh][j] = 0.0f;
    }
    const int64_t kv_base = (int64_t)gi * P.T_cap;
    for (; tile < t_end; tile += t_step) {
      const Slot my = slot_of(P, gi, g, tile, lane, full, smask);
      const float* krow = Kf + (kv_base + my.tok) * D;
      float sc[GP];
#pragma unroll
      for (int hh = 0; hh < GP; ++hh) sc[hh] = 0.0f;
      for (int c = 0; c < D; c += 4) {
        const f32x4_t k4 = *(const f32x4_t*)(krow + c);
#pragma unroll
        for (int hh = 0; hh < GP; ++hh) {
          const f32x4_t q4 = *(const f32x4_t*)&sm.qf[hh][c];
          sc[hh] += q4[0] * k4[0];
          sc[hh] += q4[1] * k4[1];
          sc[hh] += q4[2] * k4[2];
          sc[hh] += q4[3] * k4[3];
        }
      }
#pragma unroll
      for (int hh = 0; hh < GP; ++hh) {
        const bool ok = (my.mask >> hh) & 1u;
        const float s = ok ? sc[hh] : -INFINITY;
        const float mnew = fmaxf(m[hh], wave_max(s));
        const float alpha = (mnew == -INFINITY) ? 1.0f : exp2f(m[hh] - mnew);
        const float pv = ok ? exp2f(s - mnew) : 0.0f;
        l[hh] = l[hh] * alpha + pv;
        m[hh] = mnew;
        sm.p[wave][lane][hh] = pv;
#pragma unroll
        for (int j = 0; j < DPL; ++j) o[hh][j] *= alpha;
      }
      wave_lds_sync();
      for (int slot = 0; slot < kTileKeys; ++slot) {
        const int tok = __shfl(my.tok, slot, 64);
        const int ok = __shfl(my.mask != 0u ? 1 : 0, slot, 64);
        if (!ok) continue;  // wave-uniform
        const float* vrow = Vf + (kv_base + tok) * D;
        float v[DPL];
#pragma unroll
        for (int j = 0; j < DPL; ++j) v[j] = vrow[lane + j * kWave];
#pragma unroll
        for (int hh = 0; hh < GP; ++hh) {
          const float pv = sm.p[wave][slot][hh];
#pragma unroll
          for (int j = 0; j < DPL; ++j) o[hh][j] += pv * v[j];
        }
      }
      wave_lds_sync();
    }
#pragma unroll
    for (int hh = 0; hh < GP; ++hh) {
      const float lt = wave_sum(l[hh]);
      if (lane == 0) { sm.state[wave][hh][0] = m[hh]; sm.state[wave][hh][1] = lt; }
#pragma unroll
      for (int j = 0; j < DPL; ++j) sm.state[wave][hh][2 + lane + j * kWave] = o[hh][j];
    }
    __syncthreads();
    write_partial<D>(P, sm, gi, li);
    __syncthreads();
  }
}

// ---------------------------------------------------------------- merge
//
// [ASM] "방법론": lse = log sum_s Z_s, out = sum_s (Z_s / Z) a_s, evaluated in the
// log domain: the maximum of the partial maxima, then the rescaled sums.
constexpr int kMergeInFlight = 8;

// One query head's merge over its n partials at base, by NW waves: wave w takes
// partials w, w+NW, ..., lanes over dims, kMergeInFlight partials in flight per
// wave, the wave states added in a fixed order; writes out and lse.
// Deterministic.  When every partial fits one round of loads (n <= NW *
// kMergeInFlight, the usual case) they are loaded before the maximum is known
// and the maximum is taken over the loaded values, so the merge costs one memory
// round trip; otherwise a first pass finds the maximum.  Either way each
// partial is weighted by exp2(m - M) with the same M.
template <int D, int NW>
__device__ inline void merge_head(const float* base, int n, int head, float* out, float* lse) {
  constexpr int DPL = D / kWave;
  constexpr int U = kMergeInFlight;
  __shared__ float red[NW];
  __shared__ float acc_o[NW][D];
  __shared__ float acc_l[NW];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float l = 0.0f, o[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) o[j] = 0.0f;
  float M;
  if (n <= NW * U) {
    float mi[U], li[U], oi[U][DPL];
    float mloc = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = wave + u * NW;
      const float* pi = base + (int64_t)(i < n ? i : 0) * (D + 2);
      mi[u] = (i < n) ? pi[0] : -INFINITY;
      li[u] = pi[1];
#pragma unroll
      for (int j = 0; j < DPL; ++j) oi[u][j] = pi[2 + lane + j * kWave];
      mloc = fmaxf(mloc, mi[u]);
    }
    M = block_max_f<NW>(mloc, red);
    if (M != -INFINITY) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float w = exp2f(mi[u] - M);      // 0 for an empty or absent partial
        l += (w != 0.0f) ? li[u] * w : 0.0f;
#pragma unroll
        for (int j = 0; j < DPL; ++j) o[j] += (w != 0.0f) ? oi[u][j] * w : 0.0f;
      }
    }
  } else {
    M = -INFINITY;
    for (int i = threadIdx.x; i < n; i += blockDim.x) M = fmaxf(M, base[(int64_t)i * (D + 2)]);
    M = block_max_f<NW>(M, red);
    if (M != -INFINITY) {
      for (int i0 = wave; i0 < n; i0 += NW * U) {
        float mi[U], li[U], oi[U][DPL];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = i0 + u * NW;
          const float* pi = base + (int64_t)(i < n ? i : 0) * (D + 2);
          mi[u] = (i < n) ? pi[0] : -INFINITY;
          li[u] = pi[1];
#pragma unroll
          for (int j = 0; j < DPL; ++j) oi[u][j] = pi[2 + lane + j * kWave];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float w = exp2f(mi[u] - M);
          l += (w != 0.0f) ? li[u] * w : 0.0f;
#pragma unroll
          for (int j = 0; j < DPL; ++j) o[j] += (w != 0.0f) ? oi[u][j] * w : 0.0f;
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < DPL; ++j) acc_o[wave][lane + j * kWave] = o[j];
  if (lane == 0) acc_l[wave] = l;
  __syncthreads();
  float L = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) L += acc_l[w];
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    float Ov = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) Ov += acc_o[w][c];
    out[(int64_t)head * D + c] = (L > 0.0f) ? Ov / L : 0.0f;
  }
  if (threadIdx.x == 0) lse[head] = (L > 0.0f) ? (M + log2f(L)) * kLn2 : -INFINITY;
}

// Merge of the per-item kernels' partials (one per work item), one workgroup
// per query head.  One launch: a step's launches each cost a few microseconds
// whatever their work, and a head has at most a few hundred items.  Sixteen
// waves per head when the heads are few (the partials of a head then load in
// one round), four when they are many (rope_batch's 512 heads: 1024-thread
// workgroups made the launch 3 us slower).
constexpr int kMergeHeadsMany = 256;

template <int D, int NW>
__global__ void __launch_bounds__(64 * NW) attend_merge_items(AttendParams P, float* out,
                                                              float* lse) {
  touch_args(P);
  const int head = blockIdx.x;              // b * Hq + j
  const GroupInfo g = group_info(P, head / P.G);
  const int n = min(g.items, P.split_cap);
  merge_head<D, NW>(P.part + (int64_t)head * P.split_cap * (D + 2), n, head, out, lse);
}

// Merge after the pipelined kernel: one workgroup per query head over the
// partials of the runs (workgroup ranges) that met the head's group, in run
// order.
template <int D, int NW>
__global__ void __launch_bounds__(64 * NW) attend_merge_runs(AttendParams P, int grid, float* out,
                                                             float* lse) {
  touch_args(P);
  const int head = blockIdx.x;              // b * Hq + j
  const int gi = head / P.G;
  const int BH = P.B * P.H_kv;
  const int total = P.prefix[BH];
  const int gridp = run_grid(grid, total);
  const int n = min(run_owner(P.prefix[gi + 1] - 1, total, gridp) -
                    run_owner(P.prefix[gi], total, gridp) + 1, P.split_cap);
  merge_head<D, NW>(P.part + (int64_t)head * P.split_cap * (D + 2), n, head, out, lse);
}

// ---------------------------------------------------------------- host

// The pipelined kernel (bf16, dense or chunks of at least 16 keys) folds its
// items into runs and is merged by attend_merge_runs; the other kernels write
// one partial per item, merged by attend_merge_items.
inline bool pipelined(const AttendParams& P, int kv_dtype) {
  return kv_dtype == ZHA_BF16 && (P.leaf_ids == nullptr || P.C >= 16);
}

template <int D, int GP>
static void launch_partial(const AttendParams& P, int kv_dtype, int grid, hipStream_t s) {
  if (pipelined(P, kv_dtype))
    hipLaunchKernelGGL((attend_partial_bf16_pipe<D, GP>), dim3(grid), dim3(256), 0, s, P);
  else if (kv_dtype == ZHA_BF16)
    hipLaunchKernelGGL((attend_partial_bf16<D, GP, false>), dim3(grid), dim3(256), 0, s, P);
  else
    hipLaunchKernelGGL((attend_partial_f32<D, GP>), dim3(grid), dim3(256), 0, s, P);
}

template <int D>
static void launch_attend(const AttendParams& P, int kv_dtype, int grid, int BHq, float* out,
                          float* lse, hipStream_t s) {
  if (P.G <= 4) launch_partial<D, 4>(P, kv_dtype, grid, s);
  else if (P.G <= 8) launch_partial<D, 8>(P, kv_dtype, grid, s);
  else launch_partial<D, 16>(P, kv_dtype, grid, s);
  const bool few = BHq < kMergeHeadsMany;
  if (pipelined(P, kv_dtype)) {
    if (few)
      hipLaunchKernelGGL((attend_merge_runs<D, 16>), dim3(BHq), dim3(64 * 16), 0, s, P, grid, out, lse);
    else
      hipLaunchKernelGGL((attend_merge_runs<D, 4>), dim3(BHq), dim3(64 * 4), 0, s, P, grid, out, lse);
  } else {
    if (few)
      hipLaunchKernelGGL((attend_merge_items<D, 16>), dim3(BHq), dim3(64 * 16), 0, s, P, out, lse);
    else
      hipLaunchKernelGGL((attend_merge_items<D, 4>), dim3(BHq), dim3(64 * 4), 0, s, P, out, lse);
  }
}

// Checks of the arguments every attend call shares.
static int32_t check_attend(const zha_cfg* cfg, const float* q, const zha_kv* kv,
                            const int32_t* leaf_ids, const uint32_t* leaf_mask,
                            const int32_t* leaf_count, const float* out, const float* lse,
                            bool dense) {
  int32_t rc = zha_check_cfg(cfg);
  if (rc != ZHA_OK) return rc;
  if (cfg->G > 16) return ZHA_EUNSUPPORTED;
  if ((int64_t)cfg->B * cfg->H_kv > kMaxGroups) return ZHA_EUNSUPPORTED;
  if (q == nullptr || kv == nullptr || kv->K == nullptr || kv->V == nullptr ||
      kv->T == nullptr || out == nullptr || lse == nullptr)
    return ZHA_EINVAL;
  if (!dense && (leaf_ids == nullptr || leaf_mask == nullptr || leaf_count == nullptr ||
                 cfg->leaf_cap < 1))
    return ZHA_EINVAL;
  return ZHA_OK;
}

// The attend's scratch: split partials and the group
// chunk prefix, at the given addresses (256-byte aligned), with split_cap
// partial slots per query head; device-detected errors go to *status.
struct AttendScratch {
  float* part;
  float* seg;
  int32_t* prefix;
  int32_t* status;
  int32_t split_cap;
};

static int32_t launch_attend_call(const zha_cfg* cfg, const float* q, const zha_kv* kv,
                                  const int32_t* leaf_ids, const uint32_t* leaf_mask,
                                  const int32_t* leaf_count, float* out, float* lse,
                                  const AttendScratch& S, void* stream, bool dense) {
  AttendParams P;
  P.q = q; P.K = kv->K; P.V = kv->V; P.T = kv->T;
  P.leaf_ids = dense ? nullptr : leaf_ids;
  P.leaf_mask = dense ? nullptr : leaf_mask;
  P.leaf_count = dense ? nullptr : leaf_count;
  P.leaf_cap = cfg->leaf_cap;
  P.part = S.part;
  P.prefix = S.prefix;
  P.status = S.status;
  P.B = cfg->B; P.H_kv = cfg->H_kv; P.G = cfg->G; P.C = cfg->C;
  P.T_cap = cfg->T_cap;
  P.split_cap = S.split_cap;
  P.item_tiles = item_tiles(*cfg);
  P.qscale = cfg->scale * kLog2e;
  hipStream_t s = (hipStream_t)stream;
  const int64_t max_items = (int64_t)cfg->B * cfg->H_kv * split_capacity(*cfg);
  const int grid = (int)(max_items < kAttendGrid ? max_items : kAttendGrid);
  const int BHq = cfg->B * cfg->H_kv * cfg->G;
  if (cfg->d == 64)
    launch_attend<64>(P, cfg->kv_dtype, grid, BHq, out, lse, s);
  else
    launch_attend<128>(P, cfg->kv_dtype, grid, BHq, out, lse, s);
  return hipGetLastError() == hipSuccess ? ZHA_OK : ZHA_EHIP;
}

static int32_t run_attend(const zha_cfg* cfg, const float* q, const zha_kv* kv,
                          const int32_t* leaf_ids, const uint32_t* leaf_mask,
                          const int32_t* leaf_count, float* out, float* lse,
                          void* ws, size_t ws_bytes, void* stream, bool dense) {
  int32_t rc = check_attend(cfg, q, kv, leaf_ids, leaf_mask, leaf_count, out, lse, dense);
  if (rc != ZHA_OK) return rc;
  rc = zha_check_ws(cfg, dense ? ZHA_OP_DENSE : ZHA_OP_ATTEND, ws, ws_bytes);
  if (rc != ZHA_OK) return rc;
  const WsLayout w = ws_layout(*cfg);
  AttendScratch S;
  S.part = (float*)((char*)ws + w.attend_off);
  S.prefix = (int32_t*)((char*)ws + w.prefix_off);
  S.status = (int32_t*)ws;
  S.split_cap = w.split_cap;
  return launch_attend_call(cfg, q, kv, leaf_ids, leaf_mask, leaf_count, out, lse, S, stream,
                            dense);
}

// ---------------------------------------------------------------- no-allocation attend
//
// zha_attend_static keeps the attend's scratch in `scratch`, a buffer of
// kStaticScratchBytes that the library holds on every device it runs on.  In
// host code `scratch` names a host-side stand-in, never the device memory: the
// device address is looked up once per device (hipGetSymbolAddress, with that
// device current) at the first call there, kept in static_scratch_ptr, and only
// that address is handed to kernels.  Calls on one device share the buffer.
// No part of it needs to start at zero: every partial is written before it is
// read, and without a caller's status word the header
// word is a sink that nothing reads.

constexpr size_t kStaticScratchBytes = size_t(64) << 20;
constexpr int kStaticMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
static void* static_scratch_ptr[kStaticMaxDevices];
static std::mutex static_scratch_mu;

// Device address of this device's scratch, looked up at the first call.
static int32_t static_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kStaticMaxDevices) return ZHA_EHIP;
  std::lock_guard<std::mutex> lock(static_scratch_mu);
  if (static_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return ZHA_EHIP;
    static_scratch_ptr[dev] = p;
  }
  *ptr = static_scratch_ptr[dev];
  return ZHA_OK;
}

// Layout of the attend's scratch alone: [0, 256) a status sink, then partials
// and the chunk prefix.  Returns the bytes needed.
static size_t static_layout(const zha_cfg& c, char* base, AttendScratch* S) {
  const size_t BH = (size_t)c.B * c.H_kv, BHq = BH * c.G;
  const int32_t cap = run_capacity(c);
  size_t off = 256;
  const size_t part = off;
  off = align_up(off + BHq * (size_t)cap * (c.d + kPartPad) * 4, 256);
  const size_t prefix = off;
  off = align_up(off + (BH + 1) * 4, 256);
  if (S != nullptr) {
    S->part = (float*)(base + part);
    S->prefix = (int32_t*)(base + prefix);
    S->status = (int32_t*)base;
    S->split_cap = cap;
  }
  return off;
}

}  // namespace zha

extern "C" int32_t zha_attend(const zha_cfg* cfg, const float* q, const zha_kv* kv,
                              const int32_t* leaf_ids, const uint32_t* leaf_mask,
                              const int32_t* leaf_count, float* out, float* lse,
                              void* ws, size_t ws_bytes, void* stream) {
  return zha::run_attend(cfg, q, kv, leaf_ids, leaf_mask, leaf_count, out, lse, ws,
                         ws_bytes, stream, false);
}

extern "C" int32_t dense_attend(const zha_cfg* cfg, const float* q, const zha_kv* kv,
                                float* out, float* lse, void* ws, size_t ws_bytes,
                                void* stream) {
  return zha::run_attend(cfg, q, kv, nullptr, nullptr, nullptr, out, lse, ws, ws_bytes,
                         stream, true);
}

extern "C" int32_t zha_attend_static(const zha_cfg* cfg, const float* q, const zha_kv* kv,
                                     const int32_t* leaf_ids, const uint32_t* leaf_mask,
                                     const int32_t* leaf_count, float* out, float* lse,
                                     int32_t* status, void* stream) {
  using namespace zha;
  int32_t rc = check_attend(cfg, q, kv, leaf_ids, leaf_mask, leaf_count, out, lse, false);
  if (rc != ZHA_OK) return rc;
  if (static_layout(*cfg, nullptr, nullptr) > kStaticScratchBytes) return ZHA_EWORKSPACE;
  void* base = nullptr;
  rc = static_scratch(&base);
  if (rc != ZHA_OK) return rc;
  AttendScratch S;
  static_layout(*cfg, (char*)base, &S);
  if (status != nullptr) S.status = status;
  return launch_attend_call(cfg, q, kv, leaf_ids, leaf_mask, leaf_count, out, lse, S, stream,
                            false);
}
