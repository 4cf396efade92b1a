// Level-wise top-p routing down the summary tree.
//
// [ZHA] "전제와 한계" (premises and limits): at each level the candidate chunks are
// ordered by score and the shortest prefix holding fraction p of the estimated
// attention mass is kept; the kept nodes' children and the parentless nodes are
// the next level's candidates.  [ZHA] "무엇과 다른가": a node's estimated log-mass
// for a query is the maximum of its R tangent planes.
//
// Per level, one (sequence, KV head) group shares a "union list": every node that
// is a candidate of at least one of its G query heads, ascending, with a G-bit
// mask of the heads it is a candidate for.  Scoring reads each listed node's
// summary once and scores it for all G heads; each head then cuts its own
// candidates; the next level's union list is expanded from the OR of the heads'
// selections.  Everything stays on the device between levels.
//
// The top-p cut needs only the threshold, not a full sort.  Candidates are
// histogrammed (count and mass) over 2048 buckets of relative score
// floor((max s - s) * 64), which is monotone in the score, so every bucket holds
// a contiguous stretch of the descending order; a block scan finds the bucket
// where the running mass first reaches p * W, and only that bucket is sorted
// exactly by (score desc, id asc) to place the cut.  A bucket too large to sort
// (near-equal scores) falls back to an MSD radix select over the order-preserving
// 32-bit image of the scores, four 8-bit digits, ties taken by ascending id.
// Masses are w = exp(s - max s) in fp32, accumulated as 64-bit fixed point
// (w * 2^40) with integer atomics, so the cut is deterministic.
#include "zha_internal.hpp"

#include <float.h>
#include <type_traits>

namespace zha {

struct LevelParams {
  const float* q;              // [BHq][d]
  const float* khat;           // [BH][ncap][R][d]
  const float* bhat;           // [BH][ncap][R]
  int64_t ncap;
  const int32_t* uids;         // [BH][ucap] candidate union list, ascending
  const uint32_t* umask;       // [BH][ucap] head masks
  const int32_t* ucount;       // [BH]
  int64_t ucap;
  float* scores;               // [BHq][ucap]
  uint8_t* sel;                // [BHq][ucap]
  int32_t* kept;               // [BHq]
  uint32_t* selor;             // [BH][ucap] OR of kept bits, or null
  uint32_t* stage;             // [BHq][stage_cap][2] (key, w bits) for long lists
  int64_t stage_cap;
  int32_t* status;
  int32_t B, H_kv, G, d, R;
  float scale, p;
};

__device__ inline int clamp_count(int32_t u, int64_t cap) {
  if (u < 0) return 0;
  if (u > cap) return (int)cap;
  return u;
}

// ---------------------------------------------------------------- scoring (A3)
//
// One wave scores one node: the node's R x d summary (8 KiB at R=16, d=128) is
// read as 1 KiB contiguous rows per load instruction, with the non-temporal hint
// (summaries are streamed once per step; keeping them out of the caches measured
// ~10% faster).  Lane l holds rows
// r = RPI*s + l/LPR (s < NS) at dims (l%LPR)*4..+4 and the group's G query heads
// at the same dims.  The NS x GP partial dots are summed over the LPR lanes of a
// row by a transposing butterfly (each round halves the values a lane keeps),
// leaving GP/4 full dots per lane; the max over planes is a second butterfly.

template <int DELTA>
__device__ inline float xor_lane(float v) {
  if constexpr (DELTA == 32) return __shfl_xor(v, 32, 64);
  else return swz_xor<DELTA>(v);
}

template <int N, int DELTA>
__device__ inline void tr_round(float* a, int lane) {
  const bool upper = (lane & DELTA) != 0;
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const float lo = a[i], hi = a[i + N / 2];
    const float send = upper ? lo : hi;
    const float keep = upper ? hi : lo;
    a[i] = keep + xor_lane<DELTA>(send);
  }
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// The group's G queries at this lane's dims (t = lane % (D/4)), zero-padded to GP.
template <int D, int GP>
__device__ inline void load_group_queries(const LevelParams& P, int gi, int lane,
                                          float (&qv)[GP][4]) {
  const int t = lane % (D / 4);
#pragma unroll
  for (int g = 0; g < GP; ++g)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      qv[g][j] = (g < P.G) ? P.q[((int64_t)gi * P.G + g) * D + t * 4 + j] : 0.0f;
}

// One wave scores list entry u (tree node `node`) of group gi for all G heads.
template <int D, int GP>
__device__ inline void score_node(const LevelParams& P, int gi, int node, int u,
                                  const float (&qv)[GP][4], int lane) {
  constexpr int LPR = D / 4;           // lanes per summary row
  constexpr int RPI = kWave / LPR;     // rows per load instruction
  constexpr int NS = 16 / RPI;         // load instructions per node (R padded to 16)
  constexpr int V0 = NS * GP;          // partial dots per lane
  constexpr int J = GP / 4;            // full dots per lane after the butterfly
  static_assert(V0 / LPR == J, "butterfly shape");
  const int t = lane % LPR;
  if (P.selor != nullptr && lane == 0) P.selor[(int64_t)gi * P.ucap + u] = 0u;
  if (node < 0 || node >= P.ncap) {   // not a node of this tree: never selected
    if (lane < P.G) P.scores[((int64_t)gi * P.G + lane) * P.ucap + u] = -INFINITY;
    if (lane == 0) set_status(P.status, ZHA_EINVAL);
    return;
  }
  const float* base = P.khat + ((int64_t)gi * P.ncap + node) * P.R * D;
  // after the butterfly this lane holds row r = RPI*(t/4) + lane/LPR
  const int r_out = RPI * (t / 4) + lane / LPR;
  const float bh = (r_out < P.R) ? P.bhat[((int64_t)gi * P.ncap + node) * P.R + r_out] : 0.0f;
  float a[V0];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int r = RPI * s + lane / LPR;
    f32x4_t k4 = {0.f, 0.f, 0.f, 0.f};
    if (r < P.R) k4 = __builtin_nontemporal_load((const f32x4_t*)(base + r * D + t * 4));
#pragma unroll
    for (int g = 0; g < GP; ++g)
      a[s * GP + g] = qv[g][0] * k4[0] + qv[g][1] * k4[1] + qv[g][2] * k4[2] + qv[g][3] * k4[3];
  }
  // butterfly over the LPR lanes of a row: deltas LPR/2 .. 1
  if constexpr (LPR == 32) tr_round<V0, 16>(a, lane);
  if constexpr (LPR >= 16) tr_round<V0 * 16 / LPR, 8>(a, lane);
  tr_round<V0 * 8 / LPR, 4>(a, lane);
  tr_round<V0 * 4 / LPR, 2>(a, lane);
  tr_round<V0 * 2 / LPR, 1>(a, lane);
  // lane now holds dot(s = t/4, g = (t%4)*J + j) for row r_out
  float sc[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    float v = (r_out < P.R) ? fmaf(a[j], P.scale, bh) : -INFINITY;
    v = fmaxf(v, xor_lane<4>(v));
    v = fmaxf(v, xor_lane<8>(v));
    v = fmaxf(v, xor_lane<16>(v));
    v = fmaxf(v, xor_lane<32>(v));
    sc[j] = v;
  }
  if (lane < 4) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int g = lane * J + j;
      if (g < P.G) P.scores[((int64_t)gi * P.G + g) * P.ucap + u] = sc[j];
    }
  }
}

template <int D, int GP>
__global__ void __launch_bounds__(256) score_nodes(LevelParams P) {
  const int gi = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int U = clamp_count(P.ucount[gi], P.ucap);
  float qv[GP][4];
  load_group_queries<D, GP>(P, gi, lane, qv);
  const int nwaves = gridDim.x * (blockDim.x >> 6);
  const int32_t* ul = P.uids + (int64_t)gi * P.ucap;
  // the next node id is fetched one iteration ahead, so a wave's summary loads
  // never wait behind the id load that addresses them
  int u = blockIdx.x * (blockDim.x >> 6) + wave;
  int node_next = (u < U) ? ul[u] : 0;
  for (; u < U; u += nwaves) {
    const int node = node_next;
    if (u + nwaves < U) node_next = ul[u + nwaves];
    score_node<D, GP>(P, gi, node, u, qv, lane);
  }
}

// ---------------------------------------------------------------- top-p cut (A4)

constexpr int kCutThreads = 1024;
constexpr int kCutLds = 16384;         // entries staged in LDS; longer lists use the workspace
constexpr int kCutReg = 24;            // entries per thread held in registers (24576 per list)

// w * 2^40 truncated to an integer, for 0 <= w <= 1, from the fp32 bits: the
// 24-bit mantissa shifted by (exponent + 17).  Equal to (uint64)((double)w * 2^40).
__device__ inline uint64_t fixmass(float w) {
  const uint32_t b = __float_as_uint(w);
  const int sh = (int)(b >> 23) - 127 + 17;
  if (b == 0u || sh <= -24) return 0ull;
  const uint64_t m = (uint64_t)((b & 0x7fffffu) | 0x800000u);
  return sh >= 0 ? (m << sh) : (m >> (-sh));
}

// Estimated mass exp(s - max) on the hardware exp2.
__device__ inline float mass_of(float s, float mx) {
  return __builtin_amdgcn_exp2f((s - mx) * 1.4426950408889634f);
}

__device__ inline float sanitize(float s) { return isfinite(s) ? s : -FLT_MAX; }

__device__ inline uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m, 64);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

// Bitonic sort, descending, of the 64*NR values v[r] of lane l (entry r*64 + l).
template <int NR>
__device__ inline void wave_sort_desc(uint64_t (&v)[NR], int lane) {
  constexpr int N = 64 * NR;
#pragma unroll
  for (int k2 = 2; k2 <= N; k2 <<= 1) {
#pragma unroll
    for (int j = k2 >> 1; j > 0; j >>= 1) {
      if (j >= 64) {
        const int jr = j >> 6;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          if ((r & jr) == 0) {
            const int r2 = r | jr;
            const bool desc = ((r * 64) & k2) == 0;
            const uint64_t a = v[r], b = v[r2];
            const bool sw = desc ? (a < b) : (a > b);
            v[r] = sw ? b : a;
            v[r2] = sw ? a : b;
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const uint64_t a = v[r];
          const uint64_t b = shfl_xor_u64(a, j);
          const bool lower = (lane & j) == 0;
          const bool desc = ((r * 64 + lane) & k2) == 0;
          const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
          v[r] = (lower == desc) ? hi : lo;   // the lower entry of a descending pair keeps the larger
        }
      }
    }
  }
}

constexpr int kRelBuckets = 2048;
constexpr float kRelScale = 64.0f;     // buckets per unit of score
constexpr int kSortMax = 1024;         // largest crossing bucket sorted exactly

struct CutSmem {
  uint32_t key[kCutLds];
  float w[kCutLds];
  union {
    struct { uint32_t cnt[kRelBuckets]; unsigned long long mass[kRelBuckets]; } rel;
    struct { uint32_t cnt[256]; unsigned long long mass[256]; } rad;
    unsigned long long sortbuf[kSortMax];
  } u;
  float redf[16];
  unsigned long long redu[16];
  int32_t redi[16];
  uint32_t bucket;
  int32_t first;
  int32_t count;
  unsigned long long above;
};

__device__ inline float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ inline int rel_bucket(float s, float mx) {
  const float r = (mx - s) * kRelScale;
  return r >= (float)(kRelBuckets - 1) ? kRelBuckets - 1 : (int)r;
}

__global__ void __launch_bounds__(kCutThreads) cut_topp(LevelParams P) {
  __shared__ CutSmem sm;
  const int head = blockIdx.x;
  const int gi = head / P.G, g = head % P.G;
  const int tid = threadIdx.x;
  const int U = clamp_count(P.ucount[gi], P.ucap);
  const float* sc = P.scores + (int64_t)head * P.ucap;
  const uint32_t* mk = P.umask + (int64_t)gi * P.ucap;
  uint8_t* out = P.sel + (int64_t)head * P.ucap;
  const uint32_t bit = 1u << g;
  const bool lds = U <= kCutLds;
  uint32_t* skey = lds ? sm.key : P.stage + (int64_t)head * P.stage_cap * 2;
  float* sw = lds ? sm.w : (float*)(P.stage + (int64_t)head * P.stage_cap * 2 + P.stage_cap);

  uint32_t* selor = P.selor ? P.selor + (int64_t)gi * P.ucap : nullptr;
  // Lists that fit keep this thread's scores (entries j*1024 + tid) in registers
  // across every pass; all loads are issued before any is used.
  constexpr int PER = kCutReg;
  const bool reg = U <= PER * kCutThreads;
  float sv[PER];
  float mx = -INFINITY;
  int ncand = 0;
  if (reg) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int u = j * kCutThreads + tid;
      const int uu = u < U ? u : 0;         // in bounds: loads never wait on each other
      const uint32_t m = mk[uu];
      const float sj = sc[uu];
      sv[j] = (u < U && (m & bit)) ? sanitize(sj) : -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (sv[j] != -INFINITY) { mx = fmaxf(mx, sv[j]); ++ncand; }
  } else {
    for (int u = tid; u < U; u += kCutThreads)
      if (mk[u] & bit) { mx = fmaxf(mx, sanitize(sc[u])); ++ncand; }
  }
  constexpr int NW = kCutThreads / kWave;
  mx = block_max_f<NW>(mx, sm.redf);
  ncand = (int)block_sum<NW, uint32_t>((uint32_t)ncand, (uint32_t*)sm.redi);

  if (ncand == 0 || P.p >= 1.0f) {
    for (int u = tid; u < U; u += kCutThreads) {
      const bool s1 = P.p >= 1.0f && (mk[u] & bit);
      out[u] = s1 ? 1 : 0;
      if (s1 && selor) atomicOr(&selor[u], bit);
    }
    if (tid == 0) P.kept[head] = (P.p >= 1.0f) ? ncand : 0;
    return;
  }

  if (reg) {
    // ---- histogram of mass over relative-score buckets; W is its total
    for (int i = tid; i < kRelBuckets; i += kCutThreads) { sm.u.rel.cnt[i] = 0u; sm.u.rel.mass[i] = 0ull; }
    if (tid == 0) { sm.first = kRelBuckets; sm.count = 0; }
    __syncthreads();
    unsigned long long wsum = 0ull;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (sv[j] != -INFINITY) {
        const uint64_t fx = fixmass(mass_of(sv[j], mx));
        const int b = rel_bucket(sv[j], mx);
        wsum += fx;
        atomicAdd(&sm.u.rel.cnt[b], 1u);
        atomicAdd(&sm.u.rel.mass[b], (unsigned long long)fx);
      }
    }
    const unsigned long long W = block_sum<NW, unsigned long long>(wsum, sm.redu);
    const double target = (double)P.p * (double)W;
    // bucket b holds the scores just below those of buckets < b: running mass in
    // increasing b; thread t owns buckets 2t and 2t+1
    {
      const unsigned long long m0 = sm.u.rel.mass[2 * tid], m1 = sm.u.rel.mass[2 * tid + 1];
      unsigned long long tot;
      const unsigned long long pre = block_excl_scan<NW, unsigned long long>(m0 + m1, sm.redu, &tot);
      // exactly one bucket has its running mass cross p * W
      const bool c0 = (double)pre < target && (double)(pre + m0) >= target;
      const bool c1 = (double)(pre + m0) < target && (double)(pre + m0 + m1) >= target;
      if (c0) { sm.first = 2 * tid; sm.above = pre; }
      if (c1) { sm.first = 2 * tid + 1; sm.above = pre + m0; }
      __syncthreads();
    }
    const int bstar = sm.first;
    const unsigned long long above_b = sm.above;
    const int cstar = (bstar < kRelBuckets) ? (int)sm.u.rel.cnt[bstar] : kSortMax + 1;
    __syncthreads();
    if (cstar <= kSortMax) {
      // gather the crossing bucket as (key << 32 | ~u); sort descending: score
      // descending, then id ascending
      int n2 = 1;
      while (n2 < cstar) n2 <<= 1;
      for (int i = tid; i < n2; i += kCutThreads) sm.u.sortbuf[i] = 0ull;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        if (sv[j] != -INFINITY && rel_bucket(sv[j], mx) == bstar) {
          const int u = j * kCutThreads + tid;
          const int slot = atomicAdd(&sm.count, 1);
          sm.u.sortbuf[slot] = ((unsigned long long)order_key(sv[j]) << 32) | (uint32_t)(~(uint32_t)u);
        }
      }
      __syncthreads();
      const int lane = tid & 63;
      if (n2 <= 4 * kWave) {
        // one wave sorts in registers and scans; the others wait at the next barrier
        if (tid < kWave) {
          auto finish = [&](auto& v, auto nr_tag) {
            constexpr int NR = decltype(nr_tag)::value;
            wave_sort_desc<NR>(v, lane);
            int ic = -1;
            unsigned long long carry = 0ull;
#pragma unroll
            for (int r = 0; r < NR; ++r) {
              const uint64_t e = v[r];
              unsigned long long mi = 0ull;
              if ((uint32_t)(e >> 32) != 0u) mi = fixmass(mass_of(key_score((uint32_t)(e >> 32)), mx));
              const unsigned long long inc = wave_incl_scan<unsigned long long>(mi) + carry;
              const uint64_t reach = __ballot(mi != 0ull && (double)(above_b + inc) >= target);
              if (ic < 0 && reach != 0ull) ic = r * 64 + __ffsll((long long)reach) - 1;
              carry = rl64(inc, 63);
            }
            if (ic < 0 || ic > cstar - 1) ic = cstar - 1;
            // the cut entry, in sorted position ic, back to LDS for every wave
            const int r_ic = ic >> 6, l_ic = ic & 63;
            uint64_t ce = 0ull;
#pragma unroll
            for (int r = 0; r < NR; ++r)
              if (r == r_ic) ce = rl64(v[r], l_ic);
            if (lane == 0) { sm.count = 0; sm.u.sortbuf[0] = ce; }
          };
          if (n2 <= kWave) {
            uint64_t v[1] = {lane < n2 ? (uint64_t)sm.u.sortbuf[lane] : 0ull};
            finish(v, std::integral_constant<int, 1>());
          } else if (n2 <= 2 * kWave) {
            uint64_t v[2];
#pragma unroll
            for (int r = 0; r < 2; ++r) v[r] = (r * 64 + lane < n2) ? (uint64_t)sm.u.sortbuf[r * 64 + lane] : 0ull;
            finish(v, std::integral_constant<int, 2>());
          } else {
            uint64_t v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = (r * 64 + lane < n2) ? (uint64_t)sm.u.sortbuf[r * 64 + lane] : 0ull;
            finish(v, std::integral_constant<int, 4>());
          }
        }
      } else {
        for (int k2 = 2; k2 <= n2; k2 <<= 1) {
          for (int jj = k2 >> 1; jj > 0; jj >>= 1) {
            for (int i = tid; i < n2; i += kCutThreads) {
              const int ij = i ^ jj;
              if (ij > i) {
                const unsigned long long a = sm.u.sortbuf[i], b = sm.u.sortbuf[ij];
                const bool desc = (i & k2) == 0;
                if (desc ? (a < b) : (a > b)) { sm.u.sortbuf[i] = b; sm.u.sortbuf[ij] = a; }
              }
            }
            __syncthreads();
          }
        }
        // running mass in sorted order; the cut is the first element reaching p * W
        unsigned long long mi = 0ull;
        if (tid < n2) {
          const unsigned long long e = sm.u.sortbuf[tid];
          const uint32_t k = (uint32_t)(e >> 32);
          if (k != 0u) mi = fixmass(mass_of(key_score(k), mx));
        }
        unsigned long long tot2;
        const unsigned long long pre2 = block_excl_scan<NW, unsigned long long>(mi, sm.redu, &tot2);
        if (tid == 0) sm.count = kSortMax;
        __syncthreads();
        if (tid < n2 && mi != 0ull && (double)(above_b + pre2 + mi) >= target) atomicMin(&sm.count, tid);
        __syncthreads();
        if (tid == 0 && sm.count > cstar - 1) sm.count = cstar - 1;
      }
      __syncthreads();
      const int ic = sm.count;
      const unsigned long long ce = sm.u.sortbuf[ic];
      const uint32_t kap = (uint32_t)(ce >> 32);
      const int ukap = (int)(~(uint32_t)ce);
      uint32_t kept = 0;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int u = j * kCutThreads + tid;
        if (u < U) {
          uint8_t sel = 0;
          if (sv[j] != -INFINITY) {
            const uint32_t k = order_key(sv[j]);
            sel = (k > kap || (k == kap && u <= ukap)) ? 1 : 0;
          }
          out[u] = sel;
          kept += sel;
          if (sel && selor) atomicOr(&selor[u], bit);
        }
      }
      kept = block_sum<NW, uint32_t>(kept, (uint32_t*)sm.redi);
      if (tid == 0) P.kept[head] = (int32_t)kept;
      return;
    }
    __syncthreads();
  }

  // ---- general path: stage (key, w); non-candidates get key 0 and w 0
  unsigned long long wsum = 0;
  if (reg) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int u = j * kCutThreads + tid;
      uint32_t k = 0u;
      float w = 0.0f;
      if (sv[j] != -INFINITY) {
        k = order_key(sv[j]);
        w = mass_of(sv[j], mx);
        wsum += fixmass(w);
      }
      if (u < U) { skey[u] = k; sw[u] = w; }
    }
  } else {
    for (int u = tid; u < U; u += kCutThreads) {
      uint32_t k = 0u;
      float w = 0.0f;
      if (mk[u] & bit) {
        const float sc1 = sanitize(sc[u]);
        k = order_key(sc1);
        w = mass_of(sc1, mx);
        wsum += fixmass(w);
      }
      skey[u] = k;
      sw[u] = w;
    }
  }
  const unsigned long long W = block_reduce_sum<unsigned long long>(wsum, sm.redu);
  const double target = (double)P.p * (double)W;

  // MSD radix select of the threshold key over four 8-bit digits
  uint32_t prefix = 0u, pmask = 0u;
  unsigned long long above = 0ull;   // mass strictly above the current key range
  uint32_t tie_count = 0u;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kCutThreads) { sm.u.rad.cnt[i] = 0u; sm.u.rad.mass[i] = 0ull; }
    __syncthreads();
    // Scores cluster, so most lanes of a wave often hit one bucket: such waves
    // add one aggregated (count, mass) instead of 64 conflicting LDS atomics.
    const int lane = tid & 63;
    for (int base = 0; base < U; base += kCutThreads) {
      const int u = base + tid;
      const uint32_t k = (u < U) ? skey[u] : 0u;
      const bool in = k != 0u && (k & pmask) == prefix;
      const uint64_t act = __ballot(in);
      if (act == 0ull) continue;                       // wave-uniform
      const uint32_t bkt = in ? (k >> shift) & 255u : 0u;
      const unsigned long long ms = in ? (unsigned long long)fixmass(sw[u]) : 0ull;
      const int leader = __ffsll((long long)act) - 1;
      const uint32_t lb = __shfl(bkt, leader, 64);
      if (__ballot(in && bkt != lb) == 0ull) {
        unsigned long long tot = ms;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off, 64);
        if (lane == leader) {
          atomicAdd(&sm.u.rad.cnt[lb], (uint32_t)__popcll(act));
          atomicAdd(&sm.u.rad.mass[lb], tot);
        }
      } else if (in) {
        atomicAdd(&sm.u.rad.cnt[bkt], 1u);
        atomicAdd(&sm.u.rad.mass[bkt], ms);
      }
    }
    __syncthreads();
    if (tid < 64) {
      // lane owns buckets 4*lane .. 4*lane+3; suffix sums from the top bucket down
      unsigned long long own = 0ull;
#pragma unroll
      for (int i = 0; i < 4; ++i) own += sm.u.rad.mass[4 * tid + i];
      unsigned long long suf = own;   // sum over lanes >= tid
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const unsigned long long y = __shfl_down(suf, off, 64);
        if (tid + off < 64) suf += y;
      }
      const bool reach = (double)(above + suf) >= target;
      const unsigned long long ball = __ballot(reach);
      const int L = ball ? 63 - __clzll((long long)ball) : 0;   // highest lane that reaches
      if (tid == L) {
        unsigned long long run = above + (suf - own);  // mass of buckets above this lane's
        int bk = 4 * tid + 3;
        for (; bk > 4 * tid; --bk) {
          if ((double)(run + sm.u.rad.mass[bk]) >= target) break;
          run += sm.u.rad.mass[bk];
        }
        sm.bucket = (uint32_t)bk;
        sm.above = run;
      }
    }
    __syncthreads();
    const uint32_t bk = sm.bucket;
    above = sm.above;
    prefix |= bk << shift;
    pmask |= 255u << shift;
    tie_count = sm.u.rad.cnt[bk];
    __syncthreads();
  }
  // ties at the threshold key: all share one mass; take the first k by position
  const uint32_t kappa = prefix;
  __shared__ unsigned long long s_wk;
  for (int u = tid; u < U; u += kCutThreads)
    if (skey[u] == kappa) s_wk = fixmass(sw[u]);   // identical for every tie
  __syncthreads();
  const unsigned long long wk = s_wk;
  // the fewest ties k whose running mass above + k wk reaches p W, decided by the
  // same integer-to-double comparison as the sorted path
  double need = (target - (double)above) / (double)(wk == 0ull ? 1ull : wk);
  long long k_ties = (long long)ceil(need);
  if (k_ties < 1) k_ties = 1;
  if (k_ties > (long long)tie_count) k_ties = tie_count;
  while (k_ties > 1 && (double)(above + (unsigned long long)(k_ties - 1) * wk) >= target) --k_ties;
  while (k_ties < (long long)tie_count && (double)(above + (unsigned long long)k_ties * wk) < target) ++k_ties;

  // selection in list order; ties ranked by position with a block scan
  const int per = (U + kCutThreads - 1) / kCutThreads;
  const int u0 = tid * per, u1 = min(U, u0 + per);
  int my_ties = 0;
  for (int u = u0; u < u1; ++u) my_ties += (skey[u] == kappa) ? 1 : 0;
  int tot_ties = 0;
  int rank = block_exclusive_scan<int>(my_ties, sm.redi, &tot_ties);
  int kept = 0;
  for (int u = u0; u < u1; ++u) {
    const uint32_t k = skey[u];
    uint8_t s = 0;
    if (k > kappa) s = 1;
    else if (k == kappa) { s = (rank < k_ties) ? 1 : 0; ++rank; }
    out[u] = s;
    kept += s;
    if (s && selor) atomicOr(&selor[u], bit);
  }
  kept = block_reduce_sum<int>(kept, sm.redi);
  if (tid == 0) P.kept[head] = kept;
}

// ---------------------------------------------------------------- expansion (A5)
//
// One workgroup per group.  An entry of the union list is kept when any head
// kept it, its mask being the OR of the heads' bits (selor); kept entries are
// compacted in list order.  Kept parents are staged, then their children are
// written with consecutive threads on consecutive outputs, followed by the
// parentless nodes of the next level.  The final level writes the kept leaves
// themselves.  The top list (every level-L node) is built the same way with no
// parents; that launch also checks that the tree matches T.

struct ExpandParams {
  const int64_t* T;
  const int64_t* n_built;        // [L][B] (top launch only)
  const int32_t* uids; const uint32_t* umask; const int32_t* ucount; int64_t ucap;
  const uint32_t* selor;         // [BH][ucap] OR of the heads' kept bits
  int32_t* nids; uint32_t* nmask; int32_t* ncount; int64_t ncap;   // next list
  int32_t* xstage;               // [BH][xcap][2]
  int64_t xcap;
  int32_t* status;
  int32_t B, H_kv, G, C, L;
  int32_t level;                 // level of the input list; 0 = build the top list
  int32_t final_;                // 1: write the kept leaves (no children)
  int64_t span_next;             // C^(level-1): tokens per node of the next level
  int64_t T_cap;
};

constexpr int kExpandThreads = 1024;

constexpr int kExpandLds = 8192;   // kept parents staged in LDS; more use the workspace

__global__ void __launch_bounds__(kExpandThreads) expand_level(ExpandParams P) {
  constexpr int NW = kExpandThreads / kWave;
  __shared__ int32_t red[NW];
  __shared__ int32_t spid[kExpandLds];
  __shared__ uint32_t spm[kExpandLds];
  const int gi = blockIdx.x;
  const int b = gi / P.H_kv;
  const int tid = threadIdx.x;
  int64_t T = P.T[b];
  if (T < 0) T = 0;
  if (T > P.T_cap) T = P.T_cap;
  const uint32_t full = (P.G >= 32) ? 0xffffffffu : ((1u << P.G) - 1u);
  if (P.level == 0 && tid == 0 && (gi % P.H_kv) == 0) {
    int64_t span = 1;
    for (int l = 1; l <= P.L; ++l) {
      span *= P.C;
      if (P.n_built[(int64_t)(l - 1) * P.B + b] != T / span) set_status(P.status, ZHA_ESTALE);
    }
  }
  const int64_t n_next = T / P.span_next;                     // nodes at the next level
  const int64_t n_here = (P.level == 0) ? 0 : T / (P.span_next * P.C);
  const int U = (P.level == 0) ? 0 : clamp_count(P.ucount[gi], P.ucap);
  int32_t* ids = P.nids + (int64_t)gi * P.ncap;
  uint32_t* msk = P.nmask + (int64_t)gi * P.ncap;
  const uint32_t* so = P.selor ? P.selor + (int64_t)gi * P.ucap : nullptr;
  const int32_t* uid = P.uids ? P.uids + (int64_t)gi * P.ucap : nullptr;

  // Wave w owns the contiguous entries [w*R, (w+1)*R), read 64 at a time with
  // consecutive lanes on consecutive entries, kReg loads in flight per batch.
  // Kept entries are counted with ballots; one prefix over the wave counts gives
  // each wave's first output position; a second ballot pass places every kept
  // entry in list order (reusing the registers when one batch covers the range).
  const int lane = tid & 63, wave = tid >> 6;
  const int R = (((U + NW - 1) / NW) + 63) & ~63;
  const int nj = R / 64;
  const int w0 = wave * R;
  constexpr int kReg = 16;
  uint32_t mv[kReg];
  int32_t iv[kReg];
  auto load_batch = [&](int jb) {
#pragma unroll
    for (int j = 0; j < kReg; ++j) {
      const int u = w0 + (jb + j) * 64 + lane;
      const bool in = jb + j < nj && u < U;
      const int uu = in ? u : 0;
      const uint32_t m = so ? so[uu] : 0u;
      const int32_t id = uid ? uid[uu] : 0;
      mv[j] = in ? m : 0u;
      iv[j] = in ? id : 0;
    }
  };
  int cnt = 0;
  for (int jb = 0; jb < nj; jb += kReg) {
    load_batch(jb);
#pragma unroll
    for (int j = 0; j < kReg; ++j) cnt += __popcll(__ballot(mv[j] != 0u));
  }
  if (lane == 0) red[wave] = cnt;
  __syncthreads();
  int pos = 0, nsel = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int c = red[w];
    pos += (w < wave) ? c : 0;
    nsel += c;
  }
  const bool lds = nsel <= kExpandLds;
  int32_t* st = P.xstage + (int64_t)gi * P.xcap * 2;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));   // lanes below this one
  auto emit = [&](int p, int32_t id, uint32_t m) {
    if (P.final_) {
      if (p < P.ncap) { ids[p] = id; msk[p] = m; }
    } else if (lds) {
      spid[p] = id; spm[p] = m;
    } else {
      st[2 * p] = id; st[2 * p + 1] = (int32_t)m;
    }
  };
  for (int jb = 0; jb < nj; jb += kReg) {
    if (nj > kReg) load_batch(jb);
#pragma unroll
    for (int j = 0; j < kReg; ++j) {
      const uint64_t bal = __ballot(mv[j] != 0u);
      if (mv[j]) emit(pos + __popcll(bal & lt), iv[j], mv[j]);
      pos += __popcll(bal);
    }
  }
  int64_t n_orph = P.final_ ? 0 : (n_next - (int64_t)P.C * n_here);
  if (n_orph < 0) n_orph = 0;
  int64_t count = P.final_ ? nsel : (int64_t)nsel * P.C + n_orph;
  if (count > P.ncap) {
    if (tid == 0) set_status(P.status, ZHA_ECAPACITY);
    count = P.ncap;
  }
  if (!P.final_) {
    __syncthreads();   // staged parents visible to the whole block
    const int64_t nch = (int64_t)nsel * P.C;
    const int cshift = __ffs(P.C) - 1;   // C is a power of two
    for (int64_t o = tid; o < nch && o < count; o += kExpandThreads) {
      const int64_t pi = o >> cshift;
      const int32_t pid = lds ? spid[pi] : st[2 * pi];
      const uint32_t pm = lds ? spm[pi] : (uint32_t)st[2 * pi + 1];
      ids[o] = pid * P.C + (int32_t)(o & (P.C - 1));
      msk[o] = pm;
    }
    const int64_t first_orph = (int64_t)P.C * n_here;
    for (int64_t i = tid; i < n_orph; i += kExpandThreads) {
      const int64_t o = nch + i;
      if (o < count) { ids[o] = (int32_t)(first_orph + i); msk[o] = full; }
    }
  }
  if (tid == 0) P.ncount[gi] = (int32_t)count;
}

// ---------------------------------------------------------------- small levels
//
// A level whose list holds at most kSmallCap nodes per group is cut and expanded
// by one workgroup per group (route_small).  Each wave cuts one head: its
// candidates, keyed (score desc, id asc), are sorted in registers by a bitonic
// network; the masses exp(s - max) in that order, as the same 2^40 fixed point
// the large-list cut uses, give the running sums, and the cut is the first entry
// whose running mass reaches p W -- the same integers and the same comparisons
// as cut_topp, so both paths keep the same nodes.  The heads' kept bits are ORed
// in LDS and expanded exactly as expand_level does.  A level of at most kTinyCap
// nodes is also scored by that workgroup (one launch for the whole level);
// otherwise score_nodes runs first.  The top level's list (every level-L node,
// every head) is implicit.  Nothing is handed between workgroups inside a launch.

constexpr int kSmallCap = 256;
constexpr int kTinyCap = 16;
constexpr int kSmallThreads = 256;

struct SmallParams {
  int32_t top;                   // 1: the list is every level-L node (ids implicit)
  const int64_t* T;
  const int64_t* n_built;        // [L][B] (top launch: stale-tree check)
  int32_t* ucount_out;           // top launch: the level's list size, for diagnostics
  int32_t* nids; uint32_t* nmask; int32_t* ncount; int64_t ncap;   // next list
  int32_t final_;                // 1: write the kept leaves (no children)
  int32_t C, L;
  int64_t span_next;             // C^(level-1)
  int64_t T_cap;
};

// Top-p cut of one head over a list of U <= 64*NR entries, by one wave; ORs the
// head's bit into or_bits[u] of every kept entry and returns the kept count.
template <int NR>
__device__ inline int cut_head_wave(const float* sc, const uint32_t* cand_mask, uint32_t bit,
                                    int U, float p, uint32_t* or_bits, int lane) {
  uint64_t v[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int u = r * 64 + lane;
    uint64_t e = 0ull;
    if (u < U && (cand_mask[u] & bit))
      e = ((uint64_t)order_key(sanitize(sc[u])) << 32) | (uint32_t)(~(uint32_t)u);
    v[r] = e;
  }
  wave_sort_desc<NR>(v, lane);
  const uint64_t first = rl64(v[0], 0);
  if (first == 0ull) return 0;                       // no candidates
  const float mx = key_score((uint32_t)(first >> 32));
  uint64_t ms[NR];
  uint32_t nc = 0;
  uint64_t part = 0ull;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    ms[r] = (v[r] != 0ull) ? fixmass(mass_of(key_score((uint32_t)(v[r] >> 32)), mx)) : 0ull;
    part += ms[r];
    nc += __popcll(__ballot(v[r] != 0ull));
  }
  int ic;
  if (p >= 1.0f) {
    ic = (int)nc - 1;
  } else {
    const uint64_t W = wave_sum_u64(part);
    const double target = (double)p * (double)W;
    ic = -1;
    uint64_t carry = 0ull;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const uint64_t inc = wave_incl_scan<uint64_t>(ms[r]) + carry;
      const uint64_t reach = __ballot(ms[r] != 0ull && (double)inc >= target);
      if (ic < 0 && reach != 0ull) ic = r * 64 + __ffsll((long long)reach) - 1;
      carry = rl64(inc, 63);
    }
    if (ic < 0 || ic > (int)nc - 1) ic = (int)nc - 1;
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    if (v[r] != 0ull && r * 64 + lane <= ic) atomicOr(&or_bits[~(uint32_t)v[r]], bit);
  }
  return ic + 1;
}

template <int D, int GP, bool SCORE>
__global__ void __launch_bounds__(kSmallThreads) route_small(LevelParams P, SmallParams S) {
  constexpr int NW = kSmallThreads / kWave;
  __shared__ uint32_t s_cm[kSmallCap];    // candidate masks
  __shared__ int32_t s_id[kSmallCap];     // node ids
  __shared__ uint32_t s_or[kSmallCap];    // OR of the heads' kept bits
  __shared__ int32_t s_pid[kSmallCap];    // kept nodes in list order
  __shared__ uint32_t s_pm[kSmallCap];
  __shared__ int32_t s_red[NW];
  const int gi = blockIdx.x;
  const int b = gi / P.H_kv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int64_t T = S.T[b];
  if (T < 0) T = 0;
  if (T > S.T_cap) T = S.T_cap;
  const uint32_t full = (P.G >= 32) ? 0xffffffffu : ((1u << P.G) - 1u);
  const int64_t n_here = T / (S.span_next * S.C);      // nodes at this level
  int U;
  if (S.top) U = (int)(n_here < P.ucap ? n_here : P.ucap);
  else U = clamp_count(P.ucount[gi], P.ucap);
  if (U > kSmallCap) U = kSmallCap;
  const int32_t* ul = S.top ? nullptr : P.uids + (int64_t)gi * P.ucap;

  if constexpr (SCORE) {
    float qv[GP][4];
    load_group_queries<D, GP>(P, gi, lane, qv);
    for (int u = wave; u < U; u += NW) score_node<D, GP>(P, gi, S.top ? u : ul[u], u, qv, lane);
    __syncthreads();   // the scores are read back by other waves of this workgroup
  }

  for (int u = tid; u < kSmallCap; u += kSmallThreads) {
    s_or[u] = 0u;
    if (u < U) {
      s_id[u] = S.top ? u : ul[u];
      s_cm[u] = S.top ? full : P.umask[(int64_t)gi * P.ucap + u];
    }
  }
  __syncthreads();
  // ---- cut: wave w takes heads w, w + NW, ...
  for (int g = wave; g < P.G; g += NW) {
    const int64_t head = (int64_t)gi * P.G + g;
    const float* sc = P.scores + head * P.ucap;
    int kept;
    if (U <= 64) kept = cut_head_wave<1>(sc, s_cm, 1u << g, U, P.p, s_or, lane);
    else if (U <= 128) kept = cut_head_wave<2>(sc, s_cm, 1u << g, U, P.p, s_or, lane);
    else kept = cut_head_wave<4>(sc, s_cm, 1u << g, U, P.p, s_or, lane);
    if (lane == 0) P.kept[head] = kept;
  }
  __syncthreads();
  // ---- expand: kept entries in list order
  const uint32_t m = (tid < U) ? s_or[tid] : 0u;
  const uint64_t bal = __ballot(m != 0u);
  if (lane == 0) s_red[wave] = __popcll(bal);
  __syncthreads();
  int pos = 0, nsel = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    pos += (w < wave) ? s_red[w] : 0;
    nsel += s_red[w];
  }
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  pos += __popcll(bal & lt);
  if (m != 0u) { s_pid[pos] = s_id[tid]; s_pm[pos] = m; }
  __syncthreads();
  int32_t* ids = S.nids + (int64_t)gi * S.ncap;
  uint32_t* msk = S.nmask + (int64_t)gi * S.ncap;
  int64_t count;
  if (S.final_) {
    count = nsel;
    for (int i = tid; i < nsel && i < S.ncap; i += kSmallThreads) { ids[i] = s_pid[i]; msk[i] = s_pm[i]; }
  } else {
    const int64_t n_next = T / S.span_next;
    int64_t n_orph = n_next - (int64_t)S.C * n_here;
    if (n_orph < 0) n_orph = 0;
    const int64_t nch = (int64_t)nsel * S.C;
    count = nch + n_orph;
    const int64_t lim = count < S.ncap ? count : S.ncap;
    const int cshift = __ffs(S.C) - 1;   // C is a power of two
    for (int64_t o = tid; o < lim; o += kSmallThreads) {
      if (o < nch) {
        const int64_t pi = o >> cshift;
        ids[o] = s_pid[pi] * S.C + (int32_t)(o & (S.C - 1));
        msk[o] = s_pm[pi];
      } else {
        ids[o] = (int32_t)(S.C * n_here + (o - nch));
        msk[o] = full;
      }
    }
  }
  if (count > S.ncap) {
    if (tid == 0) set_status(P.status, ZHA_ECAPACITY);
    count = S.ncap;
  }
  if (tid == 0) {
    S.ncount[gi] = (int32_t)count;
    if (S.top) {
      S.ucount_out[gi] = U;
      if ((gi % P.H_kv) == 0) {
        int64_t span = 1;
        for (int l = 1; l <= S.L; ++l) {
          span *= S.C;
          if (S.n_built[(int64_t)(l - 1) * P.B + b] != T / span) set_status(P.status, ZHA_ESTALE);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- host

static void launch_score(const LevelParams& P, int64_t ucap, hipStream_t s) {
  const int BH = P.B * P.H_kv;
  int64_t gx = ceil_div(ucap, 4);
  int64_t lim = 2048 / BH;
  if (lim < 1) lim = 1;
  if (gx > lim) gx = lim;
  if (gx < 1) gx = 1;
  const dim3 grid((unsigned)gx, (unsigned)BH);
  const int GP = P.G <= 4 ? 4 : (P.G <= 8 ? 8 : 16);
  if (P.d == 128) {
    if (GP == 4) hipLaunchKernelGGL((score_nodes<128, 4>), grid, dim3(256), 0, s, P);
    else if (GP == 8) hipLaunchKernelGGL((score_nodes<128, 8>), grid, dim3(256), 0, s, P);
    else hipLaunchKernelGGL((score_nodes<128, 16>), grid, dim3(256), 0, s, P);
  } else {
    if (GP == 4) hipLaunchKernelGGL((score_nodes<64, 4>), grid, dim3(256), 0, s, P);
    else if (GP == 8) hipLaunchKernelGGL((score_nodes<64, 8>), grid, dim3(256), 0, s, P);
    else hipLaunchKernelGGL((score_nodes<64, 16>), grid, dim3(256), 0, s, P);
  }
}

template <bool SCORE>
static void launch_small_t(const LevelParams& P, const SmallParams& S, hipStream_t s) {
  const dim3 grid((unsigned)(P.B * P.H_kv));
  const int GP = P.G <= 4 ? 4 : (P.G <= 8 ? 8 : 16);
  if (P.d == 128) {
    if (GP == 4) hipLaunchKernelGGL((route_small<128, 4, SCORE>), grid, dim3(kSmallThreads), 0, s, P, S);
    else if (GP == 8) hipLaunchKernelGGL((route_small<128, 8, SCORE>), grid, dim3(kSmallThreads), 0, s, P, S);
    else hipLaunchKernelGGL((route_small<128, 16, SCORE>), grid, dim3(kSmallThreads), 0, s, P, S);
  } else {
    if (GP == 4) hipLaunchKernelGGL((route_small<64, 4, SCORE>), grid, dim3(kSmallThreads), 0, s, P, S);
    else if (GP == 8) hipLaunchKernelGGL((route_small<64, 8, SCORE>), grid, dim3(kSmallThreads), 0, s, P, S);
    else hipLaunchKernelGGL((route_small<64, 16, SCORE>), grid, dim3(kSmallThreads), 0, s, P, S);
  }
}

static int32_t check_route_common(const zha_cfg* cfg, const float* q, const zha_tree* tree,
                                  float p) {
  int32_t rc = zha_check_cfg(cfg);
  if (rc != ZHA_OK) return rc;
  if (cfg->G > 16) return ZHA_EUNSUPPORTED;
  if ((int64_t)cfg->B * cfg->H_kv > 65535) return ZHA_EUNSUPPORTED;
  if (q == nullptr || tree == nullptr) return ZHA_EINVAL;
  if (!(p > 0.0f) || !(p <= 1.0f)) return ZHA_EINVAL;
  int64_t span = 1;
  for (int l = 1; l <= cfg->L; ++l) {
    span *= cfg->C;
    if (tree->khat[l - 1] == nullptr || tree->bhat[l - 1] == nullptr) return ZHA_EINVAL;
    if (tree->n_cap[l - 1] < cfg->T_cap / span) return ZHA_EINVAL;
  }
  return ZHA_OK;
}

static LevelParams level_params(const zha_cfg* cfg, const float* q, const zha_tree* tree,
                                int level, float p, void* ws, const WsLayout& w) {
  LevelParams P;
  P.q = q;
  P.khat = tree->khat[level - 1];
  P.bhat = tree->bhat[level - 1];
  P.ncap = tree->n_cap[level - 1];
  P.stage = (uint32_t*)((char*)ws + w.stage);
  P.stage_cap = w.stage_cap;
  P.status = (int32_t*)ws;
  P.B = cfg->B; P.H_kv = cfg->H_kv; P.G = cfg->G; P.d = cfg->d; P.R = cfg->R;
  P.scale = cfg->scale; P.p = p;
  return P;
}

}  // namespace zha

extern "C" int32_t zha_route(const zha_cfg* cfg, const float* q, const zha_tree* tree,
                             const int64_t* T, float p, int32_t* leaf_ids,
                             uint32_t* leaf_mask, int32_t* leaf_count, void* ws,
                             size_t ws_bytes, void* stream) {
  using namespace zha;
  int32_t rc = check_route_common(cfg, q, tree, p);
  if (rc != ZHA_OK) return rc;
  if (T == nullptr || tree->n_built == nullptr || leaf_ids == nullptr ||
      leaf_mask == nullptr || leaf_count == nullptr)
    return ZHA_EINVAL;
  if ((int64_t)cfg->leaf_cap < cfg->T_cap / cfg->C || cfg->leaf_cap < 1) return ZHA_EINVAL;
  rc = zha_check_ws(cfg, ZHA_OP_ROUTE, ws, ws_bytes);
  if (rc != ZHA_OK) return rc;
  const WsLayout w = ws_layout(*cfg);
  hipStream_t s = (hipStream_t)stream;
  char* base = (char*)ws;
  const int BH = cfg->B * cfg->H_kv, BHq = BH * cfg->G, L = cfg->L;
  int64_t span[ZHA_MAX_L + 1];
  span[0] = 1;
  for (int l = 1; l <= L; ++l) span[l] = span[l - 1] * cfg->C;

  // Levels whose lists hold at most kSmallCap nodes run fused (score, cut and
  // expand in one launch); longer ones run score_nodes, cut_topp, expand_level.
  auto small = [&](int l) { return w.cap[l - 1] <= kSmallCap; };
  auto tiny = [&](int l) { return w.cap[l - 1] <= kTinyCap; };
  // an implicit top list needs the level scored in the same launch
  const bool top_implicit = tiny(L);
  ExpandParams E;
  E.T = T; E.status = (int32_t*)ws; E.n_built = tree->n_built;
  E.B = cfg->B; E.H_kv = cfg->H_kv; E.G = cfg->G; E.C = cfg->C; E.L = L; E.T_cap = cfg->T_cap;
  E.xstage = (int32_t*)(base + w.xstage); E.xcap = w.stage_cap;
  if (!top_implicit) {
    // top list: every level-L node, every head
    E.level = 0; E.final_ = 0;
    E.uids = nullptr; E.umask = nullptr; E.ucount = nullptr; E.ucap = 1; E.selor = nullptr;
    E.nids = (int32_t*)(base + w.uids[L - 1]);
    E.nmask = (uint32_t*)(base + w.umask[L - 1]);
    E.ncount = (int32_t*)(base + w.ucount[L - 1]);
    E.ncap = w.cap[L - 1];
    E.span_next = span[L];
    hipLaunchKernelGGL(expand_level, dim3(BH), dim3(kExpandThreads), 0, s, E);
  }

  for (int l = L; l >= 1; --l) {
    LevelParams P = level_params(cfg, q, tree, l, p, ws, w);
    P.uids = (const int32_t*)(base + w.uids[l - 1]);
    P.umask = (const uint32_t*)(base + w.umask[l - 1]);
    P.ucount = (const int32_t*)(base + w.ucount[l - 1]);
    P.ucap = w.cap[l - 1];
    P.scores = (float*)(base + w.scores[l - 1]);
    P.sel = (uint8_t*)(base + w.sel[l - 1]);
    P.kept = (int32_t*)(base + w.kept[l - 1]);
    int32_t* nids; uint32_t* nmask; int32_t* ncount; int64_t ncap;
    if (l > 1) {
      nids = (int32_t*)(base + w.uids[l - 2]);
      nmask = (uint32_t*)(base + w.umask[l - 2]);
      ncount = (int32_t*)(base + w.ucount[l - 2]);
      ncap = w.cap[l - 2];
    } else {
      nids = leaf_ids; nmask = leaf_mask; ncount = leaf_count; ncap = cfg->leaf_cap;
    }
    if (small(l)) {
      P.selor = nullptr;
      SmallParams S;
      S.top = (l == L && top_implicit) ? 1 : 0;
      S.T = T; S.n_built = tree->n_built;
      S.ucount_out = (int32_t*)(base + w.ucount[l - 1]);
      S.nids = nids; S.nmask = nmask; S.ncount = ncount; S.ncap = ncap;
      S.final_ = (l == 1) ? 1 : 0;
      S.C = cfg->C; S.L = L;
      S.span_next = span[l - 1];
      S.T_cap = cfg->T_cap;
      if (tiny(l)) {
        launch_small_t<true>(P, S, s);
      } else {
        launch_score(P, P.ucap, s);
        launch_small_t<false>(P, S, s);
      }
      continue;
    }
    P.selor = (uint32_t*)(base + w.selor[l - 1]);
    launch_score(P, P.ucap, s);
    hipLaunchKernelGGL(cut_topp, dim3(BHq), dim3(kCutThreads), 0, s, P);
    E.level = l;
    E.uids = P.uids; E.umask = P.umask; E.ucount = P.ucount; E.ucap = P.ucap;
    E.selor = P.selor;
    E.span_next = span[l - 1];
    E.final_ = (l == 1) ? 1 : 0;
    E.nids = nids; E.nmask = nmask; E.ncount = ncount; E.ncap = ncap;
    hipLaunchKernelGGL(expand_level, dim3(BH), dim3(kExpandThreads), 0, s, E);
  }
  return hipGetLastError() == hipSuccess ? ZHA_OK : ZHA_EHIP;
}

extern "C" int32_t zha_route_level(const zha_cfg* cfg, int32_t level, const float* q,
                                   const zha_tree* tree, float p, const int32_t* cand_ids,
                                   const uint32_t* cand_mask, const int32_t* cand_count,
                                   int32_t cand_cap, float* scores, uint8_t* sel,
                                   void* ws, size_t ws_bytes, void* stream) {
  using namespace zha;
  int32_t rc = check_route_common(cfg, q, tree, p);
  if (rc != ZHA_OK) return rc;
  if (level < 1 || level > cfg->L) return ZHA_EINVAL;
  if (cand_ids == nullptr || cand_mask == nullptr || cand_count == nullptr ||
      scores == nullptr || sel == nullptr || cand_cap < 1)
    return ZHA_EINVAL;
  rc = zha_check_ws(cfg, ZHA_OP_ROUTE, ws, ws_bytes);
  if (rc != ZHA_OK) return rc;
  const WsLayout w = ws_layout(*cfg);
  if ((int64_t)cand_cap > w.stage_cap) return ZHA_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  LevelParams P = level_params(cfg, q, tree, level, p, ws, w);
  P.uids = cand_ids; P.umask = cand_mask; P.ucount = cand_count; P.ucap = cand_cap;
  P.scores = scores; P.sel = sel;
  P.kept = (int32_t*)((char*)ws + w.kept[level - 1]);
  P.selor = nullptr;
  launch_score(P, cand_cap, s);
  hipLaunchKernelGGL(cut_topp, dim3(cfg->B * cfg->H_kv * cfg->G), dim3(kCutThreads), 0, s, P);
  return hipGetLastError() == hipSuccess ? ZHA_OK : ZHA_EHIP;
}

extern "C" int32_t zha_route_counts(const zha_cfg* cfg, const void* ws, int32_t* union_count,
                                    int32_t* kept_count, void* stream) {
  using namespace zha;
  int32_t rc = zha_check_cfg(cfg);
  if (rc != ZHA_OK) return rc;
  if (ws == nullptr || union_count == nullptr || kept_count == nullptr) return ZHA_EINVAL;
  const WsLayout w = ws_layout(*cfg);
  hipStream_t s = (hipStream_t)stream;
  const size_t BH = (size_t)cfg->B * cfg->H_kv, BHq = BH * cfg->G;
  for (int l = 1; l <= cfg->L; ++l) {
    if (hipMemcpyAsync(union_count + (l - 1) * BH, (const char*)ws + w.ucount[l - 1],
                       BH * sizeof(int32_t), hipMemcpyDeviceToDevice, s) != hipSuccess)
      return ZHA_EHIP;
    if (hipMemcpyAsync(kept_count + (l - 1) * BHq, (const char*)ws + w.kept[l - 1],
                       BHq * sizeof(int32_t), hipMemcpyDeviceToDevice, s) != hipSuccess)
      return ZHA_EHIP;
  }
  return ZHA_OK;
}
