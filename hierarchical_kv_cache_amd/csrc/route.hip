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
// candidates; the kept entries of all heads (a node kept by any head, with the
// OR of their bits) are compacted into the level's kept list.  The next level's
// union list is never written out: entry u is child u % C of kept node u / C, or,
// past the children, a parentless node; the top level's list is every level-L
// node.  (An explicit list can be given instead, for zha_route_level.)
// Everything stays on the device between levels.
//
// The top-p cut needs only the threshold, not a full sort.  Candidates are
// histogrammed by mass over 4096 buckets of relative score
// floor((max s - s) * 128), which is monotone in the score, so every bucket
// holds a contiguous stretch of the descending order; a block scan finds the
// bucket where the running mass first reaches p * W, and only that bucket (up to
// 1024 entries) is sorted exactly by (score desc, id asc), by one wave, to place
// the cut.  A larger bucket (near-equal scores) falls back to an MSD radix
// select over the order-preserving 32-bit image of the scores, four 8-bit
// digits, ties taken by ascending id.
// Masses are w = exp(s - max s) in fp32, accumulated as 64-bit fixed point
// (w * 2^40) with integer atomics, so the cut is deterministic.
#include "zha_internal.hpp"

#include <float.h>
#include <type_traits>

namespace zha {

// The candidate union list of one level, per group: explicit arrays, or implicit
// from the kept list of the level above (null kept list: every node, the top).
struct ListRef {
  const int32_t* ids;          // explicit: [BH][cap] ids, ascending (null: implicit)
  const uint32_t* mask;        // explicit: [BH][cap] head masks
  const int32_t* count;        // explicit: [BH]
  int64_t cap;
  const int32_t* pids;         // implicit: [BH][pcap] kept ids of the level above (null: top)
  const uint32_t* pmask;       // implicit: their OR'd head masks
  const int32_t* pcount;       // implicit: [BH]
  int64_t pcap;
  const int64_t* T;            // [B]
  int64_t T_cap;
  int64_t span;                // C^level: tokens per node of this level
  int32_t level_shift;         // log2 span (C is a power of two)
  int32_t C, cshift, H_kv;
  uint32_t full;               // every head's bit
  const int64_t* dummy;        // 8 readable bytes: stands in for an absent T or count
};

// The list's length inputs: the sequence length T and the count (explicit
// list, or kept parents of an implicit one).  Both loads are issued before
// either value is used (a missing one reads the dummy), so they cost one round
// trip; the geometry below is computed from them.
struct ListFetch {
  int64_t T;
  int32_t count;
};

__device__ inline ListFetch list_fetch(const ListRef& L, int gi) {
  const int64_t* tp = L.T != nullptr ? L.T + gi / L.H_kv : L.dummy;
  const int32_t* cp = L.ids != nullptr ? L.count + gi
                    : (L.pids != nullptr ? L.pcount + gi : (const int32_t*)L.dummy);
  ListFetch f;
  f.T = *tp;
  f.count = *cp;
  return f;
}

struct ListGeo {
  int U;          // entries
  int np;         // implicit: kept parents (children are entries [0, np*C))
  int64_t orph0;  // implicit: id of the first parentless node
};

__device__ inline ListGeo list_geo_from(const ListRef& L, const ListFetch& f, int64_t ucap) {
  ListGeo g{0, 0, 0};
  if (L.ids != nullptr) {
    const int32_t u = f.count;
    g.U = u < 0 ? 0 : (u > L.cap ? (int)L.cap : u);
  } else {
    int64_t T = f.T;
    if (T < 0) T = 0;
    if (T > L.T_cap) T = L.T_cap;
    const int64_t n_here = T >> L.level_shift;
    int64_t U;
    if (L.pids != nullptr) {
      int32_t np = f.count;
      np = np < 0 ? 0 : (np > L.pcap ? (int)L.pcap : np);
      g.np = np;
      g.orph0 = (T >> (L.level_shift + L.cshift)) << L.cshift;
      const int64_t orph = n_here - g.orph0;
      U = (int64_t)np * L.C + (orph > 0 ? orph : 0);
    } else {
      U = n_here;
    }
    g.U = (int)(U < ucap ? U : ucap);
  }
  return g;
}

__device__ inline ListGeo list_geo(const ListRef& L, int gi, int64_t ucap) {
  return list_geo_from(L, list_fetch(L, gi), ucap);
}

// Node id and head mask of entry u (< U) of group gi's list.
__device__ inline void list_entry(const ListRef& L, const ListGeo& g, int gi, int u,
                                  int32_t& id, uint32_t& mask) {
  if (L.ids != nullptr) {
    id = L.ids[(int64_t)gi * L.cap + u];
    mask = L.mask[(int64_t)gi * L.cap + u];
  } else if (u < g.np * L.C) {
    const int64_t pi = (int64_t)gi * L.pcap + (u >> L.cshift);
    id = L.pids[pi] * L.C + (u & (L.C - 1));
    mask = L.pmask[pi];
  } else {
    id = (int32_t)(g.orph0 + (u - (int64_t)g.np * L.C));
    mask = L.full;
  }
}

// Node id of entry u, with the kept parents' ids staged in LDS (spid) when given.
__device__ inline int32_t list_id(const ListRef& L, const ListGeo& g, int gi, int u,
                                  const int32_t* spid) {
  if (L.ids != nullptr) return L.ids[(int64_t)gi * L.cap + u];
  if (u < g.np * L.C) {
    const int pi = u >> L.cshift;
    const int32_t pid = spid ? spid[pi] : L.pids[(int64_t)gi * L.pcap + pi];
    return pid * L.C + (u & (L.C - 1));
  }
  return (int32_t)(g.orph0 + (u - (int64_t)g.np * L.C));
}

// Node id and head mask of entry u, with the kept parents' ids and masks
// staged in LDS (spid, spm) when given.
__device__ inline void list_entry_staged(const ListRef& L, const ListGeo& g, int gi, int u,
                                         const int32_t* spid, const uint32_t* spm,
                                         int32_t& id, uint32_t& mask) {
  if (spid == nullptr || L.ids != nullptr || u >= g.np * L.C) {
    list_entry(L, g, gi, u, id, mask);
    return;
  }
  const int pi = u >> L.cshift;
  id = spid[pi] * L.C + (u & (L.C - 1));
  mask = spm[pi];
}

struct LevelParams {
  const float* q;              // [BHq][d]
  const float* khat;           // [BH][ncap][R][d]
  const float* bhat;           // [BH][ncap][R]
  const uint16_t* khat16;      // [BH][ncap][R][d] bf16 copy of khat, read instead when set
  int64_t ncap;
  ListRef list;                // this level's candidate union list
  int32_t* ucount_out;         // [BH] list length (diagnostics), or null
  int64_t ucap;
  float* scores;               // [BHq][ucap]
  uint8_t* sel;                // [BHq][ucap]
  int32_t* kept;               // [BHq]
  uint64_t* selbits;           // [BHq][nwcap] kept bits per head, 64 entries a word, or null
  int64_t nwcap;
  uint32_t* stage;             // [BHq][stage_cap][2] (key, w bits) for long lists
  int64_t stage_cap;
  int32_t* status;
  int32_t B, H_kv, G, d, R;
  float scale, p;
  int32_t topk;                // > 0: keep this many nodes per head instead of top-p
  const int64_t* n_built;      // [L][B]: checked against T by the first launch of a route
  int32_t check_stale, L;
  // Compaction of the parent level (the level whose kept nodes' children this
  // list holds), done by this level's scoring instead of a launch of its own:
  // every workgroup compacts it into LDS, workgroup 0 also writes it out.
  int32_t fused;
  const uint64_t* fbits;       // parent level's kept bits [BHq][fnwcap]
  int64_t fnwcap;
  ListRef flist;               // parent level's candidate list
  int64_t fucap;
  int32_t* fkids; uint32_t* fkmask; int32_t* fkcount; int64_t fkcap;   // its kept list out
};

// Parent levels of at most this many nodes are compacted by the next level's
// scoring (their kept list fits the scoring kernel's LDS staging).
constexpr int64_t kFuseCap = 4096;

// The first launch of a route checks that every level was built for the current
// T: one wave, lane l holding level l + 1's built count (loaded by
// stale_count, issued with the prologue's other loads), compared once T is in.
__device__ inline int64_t stale_count(const LevelParams& P, int gi, int lane, bool chk) {
  return (chk && lane < P.L) ? P.n_built[(int64_t)lane * P.B + gi / P.H_kv] : 0;
}
__device__ inline void stale_check(const LevelParams& P, int64_t T, int64_t nb, int lane, bool chk) {
  if (T < 0) T = 0;
  if (T > P.list.T_cap) T = P.list.T_cap;
  const bool bad = chk && lane < P.L && nb != (T >> ((lane + 1) * P.list.cshift));
  if (__ballot(bad) != 0ull && lane == 0) set_status(P.status, ZHA_ESTALE);
}

__device__ inline int clamp_count(int32_t u, int64_t cap) {
  if (u < 0) return 0;
  if (u > cap) return (int)cap;
  return u;
}

// ---------------------------------------------------------------- scoring (A3)
//
// One wave scores one node: the node's R x d summary (8 KiB at R=16, d=128 in
// fp32; half that from a bf16 copy) is read as 1 KiB contiguous rows per load
// instruction (16 bytes per lane), with the non-temporal hint (summaries are
// streamed once per step; keeping them out of the caches measured ~10% faster).
// A lane holds EPL values of a row (4 fp32, or 8 bf16 widened to fp32): lane l
// holds rows r = RPI*s + l/LPR (s < NS) at dims (l%LPR)*EPL..+EPL and the
// group's G query heads at the same dims.  The NS x GP partial dots are summed
// over the LPR lanes of a row by a transposing butterfly (each round halves the
// values a lane keeps), leaving GP/4 full dots per lane; the max over planes is
// a second butterfly.

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
typedef uint32_t u32x4s_t __attribute__((ext_vector_type(4)));

// k_hat values per lane and load: 16 bytes of fp32 or of the bf16 copy.
template <bool H16>
constexpr int epl() { return H16 ? 8 : 4; }

// The group's G queries, zero-padded to GP: at this lane's EPL dims (t = lane %
// (D/EPL)) in registers when the scorer keeps them there, else into the
// workgroup's LDS copy qlds ([GP][D]; the caller synchronises the workgroup
// before it is read).
template <int D, int GP, int EPL, bool QLDS>
__device__ inline void load_group_queries(const LevelParams& P, int gi, int lane,
                                          float (&qv)[GP][EPL], float* qlds) {
  if constexpr (QLDS) {
    for (int i = threadIdx.x; i < GP * D; i += blockDim.x)
      qlds[i] = (i / D < P.G) ? P.q[(int64_t)gi * P.G * D + i] : 0.0f;
  } else {
    const int t = lane % (D / EPL);
#pragma unroll
    for (int g = 0; g < GP; ++g)
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        qv[g][j] = (g < P.G) ? P.q[((int64_t)gi * P.G + g) * D + t * EPL + j] : 0.0f;
  }
}

// One wave scores list entry u (tree node `node`) of group gi for all G heads,
// from the fp32 k_hat or (H16) its bf16 copy.  A head outside the entry's mask
// gets -inf (not its candidate); a candidate's non-finite score is stored as
// -FLT_MAX, so -inf marks exactly the non-candidates for the cut.  QLDS: the
// queries come from the workgroup's LDS copy instead of registers.
template <int D, int GP, bool H16, bool QLDS>
__device__ inline void score_node(const LevelParams& P, int gi, int node, uint32_t mask, int u,
                                  const float (&qv)[GP][epl<H16>()], const float* qlds, int lane) {
  constexpr int EPL = epl<H16>();
  constexpr int LPR = D / EPL;         // lanes per summary row
  constexpr int RPI = kWave / LPR;     // rows per load instruction
  constexpr int NS = 16 / RPI;         // load instructions per node (R padded to 16)
  constexpr int V0 = NS * 4;           // partial dots per lane and quad of heads
  static_assert(V0 == LPR, "butterfly shape");
  const int t = lane % LPR;
  if (node < 0 || node >= P.ncap) {   // not a node of this tree: never selected
    if (lane < P.G) P.scores[((int64_t)gi * P.G + lane) * P.ucap + u] = -INFINITY;
    if (lane == 0) set_status(P.status, ZHA_EINVAL);
    return;
  }
  const int64_t row0 = ((int64_t)gi * P.ncap + node) * P.R;
  // after the butterfly this lane holds row r = RPI*(t/4) + lane/LPR
  const int r_out = RPI * (t / 4) + lane / LPR;
  const float bh = (r_out < P.R) ? P.bhat[row0 + r_out] : 0.0f;
  float k[NS][EPL];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int r = RPI * s + lane / LPR;
    if constexpr (H16) {
      u32x4s_t v = u32x4s_t{0u, 0u, 0u, 0u};
      if (r < P.R) v = __builtin_nontemporal_load((const u32x4s_t*)(P.khat16 + (row0 + r) * D + t * EPL));
#pragma unroll
      for (int j = 0; j < 4; ++j) {       // bf16 -> fp32 is exact: the bits move up
        k[s][2 * j] = __uint_as_float(v[j] << 16);
        k[s][2 * j + 1] = __uint_as_float(v[j] & 0xffff0000u);
      }
    } else {
      f32x4_t v = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (r < P.R) v = __builtin_nontemporal_load((const f32x4_t*)(P.khat + (row0 + r) * D + t * EPL));
#pragma unroll
      for (int j = 0; j < 4; ++j) k[s][j] = v[j];
    }
  }
  // The heads go four at a time over the summary held in registers; the
  // scheduling barrier keeps one quad's partial dots live at a time.  With more
  // than four heads the queries come from the workgroup's LDS copy (qlds,
  // [GP][D]), which keeps the kernel at four waves per SIMD.
#pragma unroll
  for (int hq = 0; hq < GP / 4; ++hq) {
    if (hq > 0) __builtin_amdgcn_sched_barrier(0);
    float q[4][EPL];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if constexpr (QLDS) {
#pragma unroll
        for (int j4 = 0; j4 < EPL / 4; ++j4) {
          const f32x4_t x = *(const f32x4_t*)(qlds + (4 * hq + g) * D + t * EPL + 4 * j4);
#pragma unroll
          for (int j = 0; j < 4; ++j) q[g][4 * j4 + j] = x[j];
        }
      } else {
#pragma unroll
        for (int j = 0; j < EPL; ++j) q[g][j] = qv[4 * hq + g][j];
      }
    }
    float a[V0];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float acc = q[g][0] * k[s][0];
#pragma unroll
        for (int j = 1; j < EPL; ++j) acc = fmaf(q[g][j], k[s][j], acc);
        a[s * 4 + g] = acc;
      }
    // butterfly over the LPR lanes of a row: deltas LPR/2 .. 1
    if constexpr (LPR == 32) tr_round<V0, 16>(a, lane);
    if constexpr (LPR >= 16) tr_round<V0 * 16 / LPR, 8>(a, lane);
    tr_round<V0 * 8 / LPR, 4>(a, lane);
    tr_round<V0 * 4 / LPR, 2>(a, lane);
    tr_round<V0 * 2 / LPR, 1>(a, lane);
    // lane now holds dot(s = t/4, head 4 hq + t%4) for row r_out
    float v = (r_out < P.R) ? fmaf(a[0], P.scale, bh) : -INFINITY;
    v = fmaxf(v, xor_lane<4>(v));
    v = fmaxf(v, xor_lane<8>(v));
    v = fmaxf(v, xor_lane<16>(v));
    v = fmaxf(v, xor_lane<32>(v));
    const int g = 4 * hq + lane;
    if (lane < 4 && g < P.G)
      P.scores[((int64_t)gi * P.G + g) * P.ucap + u] =
          ((mask >> g) & 1u) ? (isfinite(v) ? v : -FLT_MAX) : -INFINITY;
  }
}

template <int D, int GP, bool FUSED, int NT, bool H16>
__global__ void __launch_bounds__(NT) score_nodes(LevelParams P) {
  touch_args(P);
  constexpr int kPidLds = 4096;
  constexpr int kPre = 4;              // parents per thread loaded with the prologue
  __shared__ int32_t s_pid[kPidLds];   // the group's kept parents (implicit lists)
  __shared__ uint32_t s_pm[kPidLds];   // and their head masks
  const int gi = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // ---- prologue: every load that does not wait on another is issued first --
  // the queries, the list's length inputs, the stale check's counts and the
  // first kPre * blockDim.x kept parents (the list's capacity bounds their number) --
  // so they cost one round trip; only longer parent lists need a second.
  __shared__ __attribute__((aligned(16))) float s_q[GP > 4 ? GP * D : 4];
  float qv[GP][epl<H16>()];
  load_group_queries<D, GP, epl<H16>(), (GP > 4)>(P, gi, lane, qv, s_q);
  const bool chk = P.check_stale && blockIdx.x == 0 && wave == 0 && (gi % P.H_kv) == 0;
  const int64_t nb = stale_count(P, gi, lane, chk);
  // fused: the length and the grandparents' count (the parent level's list),
  // and the parent level's bitmap rows (every row the capacity allows)
  const ListFetch lf = list_fetch(FUSED ? P.flist : P.list, gi);
  uint64_t fw[FUSED ? ZHA_MAX_G : 1];
  if constexpr (FUSED) {
#pragma unroll
    for (int g = 0; g < ZHA_MAX_G; ++g) {
      fw[g] = 0ull;
      if (wave == 0 && g < P.G && lane < P.fnwcap)
        fw[g] = P.fbits[((int64_t)gi * P.G + g) * P.fnwcap + lane];
    }
  }
  const bool implicit = P.list.ids == nullptr && P.list.pids != nullptr;
  int32_t pre_id[kPre];
  uint32_t pre_m[kPre];
#pragma unroll
  for (int k = 0; k < kPre; ++k) {
    const int i = threadIdx.x + blockDim.x * k;
    pre_id[k] = 0;
    pre_m[k] = 0u;
    if (implicit && !FUSED && i < P.list.pcap) {
      pre_id[k] = P.list.pids[(int64_t)gi * P.list.pcap + i];
      pre_m[k] = P.list.pmask[(int64_t)gi * P.list.pcap + i];
    }
  }
  ListGeo geo;
  bool staged;
  if constexpr (FUSED) {
    // the parent level's kept list, compacted here from its heads' bitmaps: rows
    // of 64 list entries, the kept entries (any head's bit) in list order
    __shared__ uint64_t s_w[ZHA_MAX_G][kFuseCap / 64];   // heads' words per row
    __shared__ uint64_t s_any[kFuseCap / 64];
    __shared__ int32_t s_off[kFuseCap / 64];
    __shared__ int32_t s_np;
    const ListGeo pg = list_geo_from(P.flist, lf, P.fucap);
    const int prow = (pg.U + 63) >> 6;                      // <= kFuseCap / 64
    if (wave == 0) {
      uint64_t any = 0ull;
      if (lane < prow) {
        const int valid = pg.U - lane * 64;
        const uint64_t vmask = valid >= 64 ? ~0ull : ((1ull << valid) - 1ull);
#pragma unroll
        for (int g = 0; g < ZHA_MAX_G; ++g) {
          const uint64_t wd = fw[g] & vmask;
          if (g < P.G) s_w[g][lane] = wd;
          any |= wd;
        }
        s_any[lane] = any;
      }
      const int c = __popcll(any);
      const int inc = wave_incl_scan<int>(c);
      if (lane < prow) s_off[lane] = inc - c;
      if (lane == kWave - 1) s_np = inc;
    }
    __syncthreads();
    const int np_all = s_np;
    const int np = np_all < P.fkcap ? np_all : (int)P.fkcap;
    for (int u = threadIdx.x; u < prow * 64; u += blockDim.x) {
      const int r = u >> 6, bpos = u & 63;
      const uint64_t any = s_any[r];
      if ((any >> bpos) & 1ull) {
        const int pos = s_off[r] + __popcll(any & ((1ull << bpos) - 1ull));
        uint32_t m = 0u;
        for (int g = 0; g < P.G; ++g) m |= (uint32_t)((s_w[g][r] >> bpos) & 1ull) << g;
        if (pos < np) {
          s_pid[pos] = list_id(P.flist, pg, gi, u, nullptr);
          s_pm[pos] = m;
        }
      }
    }
    ListFetch own;
    own.T = lf.T;
    own.count = np;
    geo = list_geo_from(P.list, own, P.ucap);
    staged = true;
    __syncthreads();
    if (blockIdx.x == 0) {
      for (int i = threadIdx.x; i < np; i += blockDim.x) {
        P.fkids[(int64_t)gi * P.fkcap + i] = s_pid[i];
        P.fkmask[(int64_t)gi * P.fkcap + i] = s_pm[i];
      }
      if (threadIdx.x == 0) {
        if (np_all > P.fkcap) set_status(P.status, ZHA_ECAPACITY);
        P.fkcount[gi] = np;
      }
    }
  } else {
    geo = list_geo_from(P.list, lf, P.ucap);
    staged = implicit && geo.np <= kPidLds;
  }
  stale_check(P, lf.T, nb, lane, chk);
  const int U = geo.U;
  if (staged && !FUSED) {
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
      const int i = threadIdx.x + blockDim.x * k;
      if (i < geo.np) { s_pid[i] = pre_id[k]; s_pm[i] = pre_m[k]; }
    }
    for (int i = threadIdx.x + blockDim.x * kPre; i < geo.np; i += blockDim.x) {
      s_pid[i] = P.list.pids[(int64_t)gi * P.list.pcap + i];
      s_pm[i] = P.list.pmask[(int64_t)gi * P.list.pcap + i];
    }
  }
  __syncthreads();
  const int32_t* spid = staged ? s_pid : nullptr;
  const uint32_t* spm = staged ? s_pm : nullptr;
  const int nwaves = gridDim.x * (blockDim.x >> 6);
  // Logical workgroup xl takes entries 4 xl + wave, + nwaves, ...: the 8
  // writers of one 128-byte line of a head's scores share an XCD (its L2).
  const int xl = xcd_grouped_x();
  // the next entry is fetched one iteration ahead, so a wave's summary loads
  // never wait behind the id load that addresses them
  int u = xl * (blockDim.x >> 6) + wave;
  int32_t node_next = 0;
  uint32_t mask_next = 0u;
  if (u < U) list_entry_staged(P.list, geo, gi, u, spid, spm, node_next, mask_next);
  for (; u < U; u += nwaves) {
    const int node = node_next;
    const uint32_t mask = mask_next;
    if (u + nwaves < U) list_entry_staged(P.list, geo, gi, u + nwaves, spid, spm, node_next, mask_next);
    score_node<D, GP, H16, (GP > 4)>(P, gi, node, mask, u, qv, s_q, lane);
  }
}

// ---------------------------------------------------------------- top-p cut (A4)

constexpr int kCutThreads = 1024;
constexpr int kCutLds = 16384;         // general path: entries staged in LDS; longer lists use the workspace
constexpr int kCutStage = 24;          // entries per thread staged in LDS by the main path (24576 per list)

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

// The weight a candidate carries into the cut: its estimated mass exp(s - max)
// for top-p, or 1 for a fixed budget of topk nodes (the cut then falls on the
// topk-th node in order).
__device__ inline float cut_mass(float s, float mx, int topk) {
  return topk > 0 ? 1.0f : mass_of(s, mx);
}

// The running weight at which the cut falls: p W for top-p; for a budget of topk
// nodes, topk unit weights (2^40 each), or every candidate when fewer.
__device__ inline double cut_target(float p, int topk, unsigned long long W) {
  if (topk > 0) {
    const double k = (double)topk * 1099511627776.0;
    return k < (double)W ? k : (double)W;
  }
  return (double)p * (double)W;
}

// The value of lane (lane ^ J), J < 64: DPP row operations for J <= 8 (quad
// permutes; row shifts by 4 selected per lane; row rotate by 8), a swizzle for
// J = 16 and a permute across the 32-lane halves for J = 32.
template <int J>
__device__ inline uint32_t xor_partner32(uint32_t v, int lane) {
  if constexpr (J == 1) return dpp32<0xB1>(v);
  else if constexpr (J == 2) return dpp32<0x4E>(v);
  else if constexpr (J == 4) {
    const uint32_t up = dpp32<0x104>(v);    // row_shl:4: the value of lane + 4
    const uint32_t dn = dpp32<0x114>(v);    // row_shr:4: the value of lane - 4
    return (lane & 4) ? dn : up;
  } else if constexpr (J == 8) return dpp32<0x128>(v);   // row_ror:8
  else if constexpr (J == 16) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (16 << 10) | 0x1f);
  else return (uint32_t)__shfl_xor((int)v, 32, 64);
}
template <int J>
__device__ inline uint64_t xor_partner64(uint64_t v, int lane) {
  return ((uint64_t)xor_partner32<J>((uint32_t)(v >> 32), lane) << 32) |
         xor_partner32<J>((uint32_t)v, lane);
}

// Bitonic network, descending, over the 64 NR values of a wave held blocked:
// entry i = NR lane + r is v[r] of lane `lane`.  Exchanges between entries fewer
// than NR apart stay in a lane's registers; the others pair lanes J/NR apart.
template <int NR, int K2, int J>
__device__ inline void bitonic_stage(uint64_t (&v)[NR], int lane) {
  if constexpr (J < NR) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      if ((r & J) == 0) {
        const int r2 = r | J;
        const bool desc = ((NR * lane + r) & K2) == 0;
        const uint64_t a = v[r], b = v[r2];
        const bool sw = (a < b) == desc;   // a descending pair puts the larger first
        v[r] = sw ? b : a;
        v[r2] = sw ? a : b;
      }
    }
  } else {
    constexpr int JL = J / NR;
    const bool lower = (lane & JL) == 0;
    const bool desc = ((NR * lane) & K2) == 0;   // K2 > J >= NR: r stays below bit K2
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const uint64_t a = v[r];
      const uint64_t b = xor_partner64<JL>(a, lane);
      // the lower entry of a descending pair keeps the larger, and so on
      v[r] = ((b > a) == (lower == desc)) ? b : a;
    }
  }
  if constexpr (J > 1) bitonic_stage<NR, K2, J / 2>(v, lane);
}

template <int NR, int K2, int KMAX>
__device__ inline void bitonic_merge_all(uint64_t (&v)[NR], int lane) {
  bitonic_stage<NR, K2, K2 / 2>(v, lane);
  if constexpr (K2 < KMAX) bitonic_merge_all<NR, K2 * 2, KMAX>(v, lane);
}

// Sorts the blocked entries descending.  With KMAX < 64 NR only the networks of
// KMAX entries run: the first KMAX entries come out sorted when every later one
// is zero (a shorter list padded with zeros).
template <int NR, int KMAX = 64 * NR>
__device__ inline void wave_sort_desc(uint64_t (&v)[NR], int lane) {
  static_assert(KMAX >= 2 && KMAX <= 64 * NR && (KMAX & (KMAX - 1)) == 0, "power-of-two network");
  bitonic_merge_all<NR, 2, KMAX>(v, lane);
}

constexpr int kRelBuckets = 4096;
constexpr float kRelScale = 128.0f;    // buckets per unit of score (32 units in all)
constexpr int kSortMax = 1024;         // largest crossing bucket sorted exactly
// Lists of at most this many entries are cut by one wave sorting them whole.
// Longer ones take the buckets: a one-wave sort of 278 entries took 11.1 us
// against 8.0 us bucketed, of 787 entries 19.9 us against 7.9 us.
constexpr int kWaveCutMax = 64;
static_assert(kSortMax == kCutThreads, "the crossing-bucket buffer is cleared one entry per thread");
static_assert(kRelBuckets == 4 * kCutThreads, "each thread scans four buckets");

// ---------------------------------------------------------------- compaction (A5)
//
// After the cut.  An entry of the level's union list is kept when any head kept
// it, its mask being the OR of the heads' bits, read from the heads' bitmaps
// (one 64-bit word per row of 64 entries); kept entries are written in list
// order (ascending ids) as the level's kept list -- the leaf list at level 1,
// otherwise the parents of the next level's implicit list.  Workgroup x of a
// group places rows [x R, x R + R), R = kCompactRows; it finds its first output
// position by counting the kept entries of the rows before it itself, so the
// workgroups never wait for one another.

struct CompactParams {
  ListRef list;                  // this level's union list
  int64_t ucap;
  const uint64_t* selbits;       // [BHq][nwcap]
  int64_t nwcap;
  int32_t G;
  int32_t* kids; uint32_t* kmask; int32_t* kcount; int64_t kcap;   // kept list out
  int32_t* status;
};

constexpr int kCompactThreads = 256;
constexpr int kCompactRows = 16;     // rows of 64 entries placed per workgroup

// Entries of row r kept by at least one head (bit l: entry 64 r + l; U entries).
__device__ inline uint64_t kept_row(const uint64_t* hb, int64_t nwcap, int G, int r, int U) {
  const int valid = U - r * 64;
  const uint64_t vmask = valid >= 64 ? ~0ull : ((1ull << valid) - 1ull);
  uint64_t any = 0ull;
  for (int g = 0; g < G; ++g) any |= hb[(int64_t)g * nwcap + r];
  return any & vmask;
}

struct CutSmem {
  union {
    struct {                                      // staged path
      float sc[kCutStage * kCutThreads];            // the head's scores (-inf past U)
      unsigned long long relmass[kRelBuckets];    // mass per relative-score bucket
      unsigned long long ent[kSortMax];           // crossing bucket: key << 32 | ~u, 0 past it
      unsigned long long kbits[kCutStage * kCutThreads / 64];   // kept bits, 64 entries a word
    } h;
    struct {                                      // general path
      uint32_t key[kCutLds];
      float w[kCutLds];
      uint32_t cnt[256];
      unsigned long long mass[256];
    } g;
  } u;
  float redf[16];
  unsigned long long scan[16];
  unsigned long long redu[16];
  int32_t redi[16];
  uint32_t bucket;
  int32_t first;
  int32_t count;       // crossing-bucket entries gathered
  int32_t nabove;      // candidates in buckets above the crossing one
  int32_t ic;          // sorted position of the cut entry within the crossing bucket
  unsigned long long above;
};

__device__ inline float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ inline int rel_bucket(float s, float mx) {
  const float r = (mx - s) * kRelScale;
  return r >= (float)(kRelBuckets - 1) ? kRelBuckets - 1 : (int)r;
}

// One wave places the cut inside the crossing bucket: its entries (key << 32 |
// ~u, zero past the last), at most KMAX of them, are sorted by score descending
// then id ascending; their masses are run in that order from `above`, the mass
// of every bucket before it; the first entry whose running mass reaches target
// is the cut.  Sets sm.ic (its position) and sets the kept entries' bits in
// sm.u.h.kbits.
template <int NR, int KMAX = 64 * NR>
__device__ inline void cut_in_bucket(CutSmem& sm, int cstar, float mx, int topk,
                                     unsigned long long above, double target, int lane) {
  uint64_t v[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) v[r] = (uint64_t)sm.u.h.ent[NR * lane + r];
  wave_sort_desc<NR, KMAX>(v, lane);
  // running mass in sorted order: this lane's entries follow those of lower lanes
  unsigned long long mi[NR], own = 0ull;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const uint64_t e = v[r];
    mi[r] = 0ull;
    if ((uint32_t)(e >> 32) != 0u) mi[r] = fixmass(cut_mass(key_score((uint32_t)(e >> 32)), mx, topk));
    own += mi[r];
  }
  unsigned long long run = above + wave_incl_scan<unsigned long long>(own) - own;
  int rf = NR;   // this lane's first entry whose running mass reaches target
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    run += mi[r];
    if (rf == NR && mi[r] != 0ull && (double)run >= target) rf = r;
  }
  const uint64_t reach = __ballot(rf < NR);
  int ic = -1;
  if (reach != 0ull) {
    const int l = __ffsll((long long)reach) - 1;
    ic = NR * l + (int)rl32((uint32_t)rf, l);
  }
  if (ic < 0 || ic > cstar - 1) ic = cstar - 1;
  // the bucket's entries up to the cut are kept
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    if (v[r] != 0ull && NR * lane + r <= ic) {
      const uint32_t u = ~(uint32_t)v[r];
      atomicOr(&sm.u.h.kbits[u >> 6], 1ull << (u & 63));
    }
  }
  if (lane == 0) sm.ic = ic;
}

// A list of at most kWaveCutMax entries: one wave sorts the head's candidates whole
// in registers (key << 32 | ~u, blocked NR per lane) and runs their masses in
// that order; the first entry whose running mass reaches the target is the cut.
// The same integers and comparisons as the bucketed path, without its passes.
// The kept bits go through the wave's LDS words (wbits, NR of them) to the
// head's bitmap rows.
template <int NR, int KMAX = 64 * NR>
__device__ inline void cut_list_wave(const LevelParams& P, const float* sc, int U, int head,
                                     uint8_t* out, uint64_t* bits, uint64_t* wbits, int lane) {
  uint64_t v[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int u = NR * lane + r;
    uint64_t e = 0ull;
    if (u < U) {
      const float x = sc[u];
      if (x != -INFINITY) e = ((uint64_t)order_key(x) << 32) | (uint32_t)(~(uint32_t)u);
    }
    v[r] = e;
  }
  wave_sort_desc<NR, KMAX>(v, lane);
  const uint64_t first = rl64(v[0], 0);
  int ic = -1;   // sorted position of the last kept entry; -1: no candidates
  if (first != 0ull) {
    const float mx = key_score((uint32_t)(first >> 32));
    uint64_t ms[NR];
    uint32_t nc = 0;
    uint64_t own = 0ull;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      ms[r] = (v[r] != 0ull) ? fixmass(cut_mass(key_score((uint32_t)(v[r] >> 32)), mx, P.topk)) : 0ull;
      own += ms[r];
      nc += __popcll(__ballot(v[r] != 0ull));
    }
    if (P.topk == 0 && P.p >= 1.0f) {
      ic = (int)nc - 1;
    } else {
      const uint64_t inc = wave_incl_scan<uint64_t>(own);
      const double target = cut_target(P.p, P.topk, rl64(inc, 63));
      uint64_t run = inc - own;
      int rf = NR;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        run += ms[r];
        if (rf == NR && ms[r] != 0ull && (double)run >= target) rf = r;
      }
      const uint64_t reach = __ballot(rf < NR);
      if (reach != 0ull) {
        const int l = __ffsll((long long)reach) - 1;
        ic = NR * l + (int)rl32((uint32_t)rf, l);
      }
      if (ic < 0 || ic > (int)nc - 1) ic = (int)nc - 1;
    }
  }
  const int nrow = (U + 63) >> 6;
  if (lane < NR) wbits[lane] = 0ull;
  wave_lds_sync();
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    if (v[r] != 0ull && NR * lane + r <= ic) {
      const uint32_t u = ~(uint32_t)v[r];
      atomicOr((unsigned long long*)&wbits[u >> 6], 1ull << (u & 63));
    }
  }
  wave_lds_sync();
  if (bits && lane < nrow) bits[lane] = wbits[lane];
  if (out)
    for (int u = lane; u < U; u += kWave) out[u] = (uint8_t)((wbits[u >> 6] >> (u & 63)) & 1ull);
  if (lane == 0) P.kept[head] = ic + 1;
}

// One workgroup cuts one query head.  The head's kept entries are written as a
// bitmap (bit u % 64 of word u / 64; a wave's 64 consecutive entries are one
// ballot) and, when sel is given, as bytes.
//
// The kernel runs once per level right after the scoring pass has streamed the
// summaries through the caches, so its instructions are fetched cold: every
// phase after the loads is a rolled loop over the scores staged in LDS, which
// keeps the code that runs small.
__device__ inline void cut_head(const LevelParams& P, CutSmem& sm) {
  constexpr int NW = kCutThreads / kWave;
  constexpr int PER = kCutStage;
  const int head = blockIdx.x;
  const int gi = head / P.G, g = head % P.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* sc = P.scores + (int64_t)head * P.ucap;
  // The scores are loaded up to the list's capacity before its length is known,
  // so these loads do not wait on the length's; entries past it are dropped.
  // The scores mark this head's non-candidates with -inf (candidates are finite).
  const int ucap = (int)(P.ucap < (int64_t)PER * kCutThreads ? P.ucap : (int64_t)PER * kCutThreads);
  float v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    v[j] = -INFINITY;
    if (j * kCutThreads < ucap) v[j] = sc[min(j * kCutThreads + tid, ucap - 1)];
  }
  const ListGeo geo = list_geo(P.list, gi, P.ucap);
  const int U = geo.U;
  if (g == 0 && tid == 0 && P.ucount_out != nullptr) P.ucount_out[gi] = U;
  uint8_t* out = P.sel ? P.sel + (int64_t)head * P.ucap : nullptr;
  uint64_t* bits = P.selbits ? P.selbits + (int64_t)head * P.nwcap : nullptr;
  if (U <= kWaveCutMax) {
    // short list: one wave, no histogram; the other waves leave
    if (wave == 0) {
      uint64_t* wbits = (uint64_t*)sm.u.h.relmass;
      if (U <= 16) cut_list_wave<1, 16>(P, sc, U, head, out, bits, wbits, lane);
      else cut_list_wave<1>(P, sc, U, head, out, bits, wbits, lane);
    }
    return;
  }
  const int nrow = (U + 63) >> 6;
  const bool staged = U <= PER * kCutThreads;
  const int nj = (U + kCutThreads - 1) / kCutThreads;   // rows of kCutThreads entries
  if (tid == 0) { sm.nabove = 0; sm.count = 0; sm.first = kRelBuckets; sm.ic = kSortMax; }
  float mx = -INFINITY;
  if (staged) {
    for (int i = tid; i < kRelBuckets; i += kCutThreads) sm.u.h.relmass[i] = 0ull;
    sm.u.h.ent[tid] = 0ull;   // kSortMax == kCutThreads
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int u = j * kCutThreads + tid;
      const float x = u < U ? v[j] : -INFINITY;
      sm.u.h.sc[u] = x;
      mx = fmaxf(mx, x);
    }
  } else {
    for (int u = tid; u < U; u += kCutThreads) mx = fmaxf(mx, sc[u]);
  }
  mx = wave_max_fast(mx);
  if (lane == 0) sm.redf[wave] = mx;
  __syncthreads();
  for (int w = 0; w < NW; ++w) mx = fmaxf(mx, sm.redf[w]);   // -inf: the head has no candidates

  if (mx == -INFINITY || (P.topk == 0 && P.p >= 1.0f)) {
    // p >= 1 keeps every candidate; no candidates keeps nothing
    int kept = 0;
    for (int j0 = 0; j0 < U; j0 += kCutThreads) {
      const int u = j0 + tid;
      const bool s1 = mx != -INFINITY && u < U && sc[u] != -INFINITY;
      const uint64_t b = __ballot(s1);
      if (out && u < U) out[u] = s1 ? 1 : 0;
      const int row = (j0 >> 6) + wave;
      if (bits && lane == 0 && row < nrow) bits[row] = b;
      kept += __popcll(b);
    }
    if (lane == 0) atomicAdd(&sm.nabove, kept);
    __syncthreads();
    if (tid == 0) P.kept[head] = sm.nabove;
    return;
  }

  if (staged) {
    const float* ss = sm.u.h.sc;
    // ---- mass per bucket of relative score floor((max - s) * kRelScale)
#pragma unroll 4
    for (int j = 0; j < nj; ++j) {
      const float x = ss[j * kCutThreads + tid];
      if (x != -INFINITY)
        atomicAdd(&sm.u.h.relmass[rel_bucket(x, mx)], (unsigned long long)fixmass(cut_mass(x, mx, P.topk)));
    }
    __syncthreads();
    // ---- running mass in increasing bucket order (bucket b holds the scores
    // just below those of buckets < b); thread t owns buckets 4t .. 4t+3.  The
    // total is W, the sum of every candidate's mass.
    unsigned long long m[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) m[i] = sm.u.h.relmass[4 * tid + i];
    const unsigned long long own = (m[0] + m[1]) + (m[2] + m[3]);
    const unsigned long long inc = wave_incl_scan<unsigned long long>(own);
    if (lane == 63) sm.scan[wave] = inc;
    __syncthreads();
    unsigned long long run = inc - own, W = 0ull;
    for (int w = 0; w < NW; ++w) {
      const unsigned long long t = sm.scan[w];
      run += (w < wave) ? t : 0ull;
      W += t;
    }
    const double target = cut_target(P.p, P.topk, W);
    // exactly one bucket has its running mass cross p W
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if ((double)run < target && (double)(run + m[i]) >= target) { sm.first = 4 * tid + i; sm.above = run; }
      run += m[i];
    }
    __syncthreads();
    const int bstar = sm.first;
    const unsigned long long above_b = sm.above;
    // ---- gather the crossing bucket; count the candidates above it
    // (one slot reservation per wave and row: the lanes in the bucket take
    // consecutive slots in lane order)
    int nab = 0;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));   // lanes below this one
    for (int j = 0; j < nj; ++j) {
      const int u = j * kCutThreads + tid;
      const float x = ss[u];
      const int b = x != -INFINITY ? rel_bucket(x, mx) : kRelBuckets;
      nab += b < bstar ? 1 : 0;
      // row u / 64 = j NW + wave: every entry of a bucket above the crossing one is kept
      const uint64_t above_row = __ballot(b < bstar);
      if (lane == 0) sm.u.h.kbits[j * NW + wave] = above_row;
      const uint64_t inb = __ballot(b == bstar);
      if (inb != 0ull) {                                  // uniform over the wave
        const int leader = __ffsll((long long)inb) - 1;
        int base = 0;
        if (lane == leader) base = atomicAdd(&sm.count, __popcll(inb));
        base = __shfl(base, leader, 64);
        const int slot = base + __popcll(inb & lt);
        if (b == bstar && slot < kSortMax)
          sm.u.h.ent[slot] = ((unsigned long long)order_key(x) << 32) | (uint32_t)(~(uint32_t)u);
      }
    }
    nab = (int)wave_sum_u32((uint32_t)nab);
    if (lane == 0) atomicAdd(&sm.nabove, nab);
    __syncthreads();
    const int cstar = (bstar < kRelBuckets) ? sm.count : kSortMax + 1;
    if (cstar <= kSortMax) {
      // one wave sorts the bucket in registers; the others wait at the barrier
      if (tid < kWave) {
        if (cstar <= 16) cut_in_bucket<1, 16>(sm, cstar, mx, P.topk, above_b, target, lane);
        else if (cstar <= kWave) cut_in_bucket<1>(sm, cstar, mx, P.topk, above_b, target, lane);
        else if (cstar <= 2 * kWave) cut_in_bucket<2>(sm, cstar, mx, P.topk, above_b, target, lane);
        else if (cstar <= 4 * kWave) cut_in_bucket<4>(sm, cstar, mx, P.topk, above_b, target, lane);
        else if (cstar <= 8 * kWave) cut_in_bucket<8>(sm, cstar, mx, P.topk, above_b, target, lane);
        else cut_in_bucket<16>(sm, cstar, mx, P.topk, above_b, target, lane);
      }
      __syncthreads();
      // the kept bits: rows above the crossing bucket from the gather, the
      // bucket's kept entries from the sort
      if (bits)
        for (int r = tid; r < nrow; r += kCutThreads) bits[r] = sm.u.h.kbits[r];
      if (out)
        for (int u = tid; u < U; u += kCutThreads) out[u] = (uint8_t)((sm.u.h.kbits[u >> 6] >> (u & 63)) & 1ull);
      if (tid == 0) P.kept[head] = sm.nabove + sm.ic + 1;
      return;
    }
    __syncthreads();   // the general path's staging overlays the staged scores
  }

  // ---- general path: stage (key, w); non-candidates get key 0 and w 0
  const bool lds = U <= kCutLds;
  uint32_t* skey = lds ? sm.u.g.key : P.stage + (int64_t)head * P.stage_cap * 2;
  float* sw = lds ? sm.u.g.w : (float*)(P.stage + (int64_t)head * P.stage_cap * 2 + P.stage_cap);
  unsigned long long wsum = 0;
  for (int u = tid; u < U; u += kCutThreads) {
    uint32_t k = 0u;
    float w = 0.0f;
    const float sc1 = sc[u];
    if (sc1 != -INFINITY) {
      k = order_key(sc1);
      w = cut_mass(sc1, mx, P.topk);
      wsum += fixmass(w);
    }
    skey[u] = k;
    sw[u] = w;
  }
  if (bits)
    for (int r = tid; r < nrow; r += kCutThreads) bits[r] = 0ull;
  const unsigned long long W = block_reduce_sum<unsigned long long>(wsum, sm.redu);
  const double target = cut_target(P.p, P.topk, W);

  // MSD radix select of the threshold key over four 8-bit digits
  uint32_t prefix = 0u, pmask = 0u;
  unsigned long long above = 0ull;   // mass strictly above the current key range
  uint32_t tie_count = 0u;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kCutThreads) { sm.u.g.cnt[i] = 0u; sm.u.g.mass[i] = 0ull; }
    __syncthreads();
    // Scores cluster, so most lanes of a wave often hit one bucket: such waves
    // add one aggregated (count, mass) instead of 64 conflicting LDS atomics.
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
          atomicAdd(&sm.u.g.cnt[lb], (uint32_t)__popcll(act));
          atomicAdd(&sm.u.g.mass[lb], tot);
        }
      } else if (in) {
        atomicAdd(&sm.u.g.cnt[bkt], 1u);
        atomicAdd(&sm.u.g.mass[bkt], ms);
      }
    }
    __syncthreads();
    if (tid < 64) {
      // lane owns buckets 4*lane .. 4*lane+3; suffix sums from the top bucket down
      unsigned long long own = 0ull;
#pragma unroll
      for (int i = 0; i < 4; ++i) own += sm.u.g.mass[4 * tid + i];
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
          if ((double)(run + sm.u.g.mass[bk]) >= target) break;
          run += sm.u.g.mass[bk];
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
    tie_count = sm.u.g.cnt[bk];
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
    uint8_t s1 = 0;
    if (k > kappa) s1 = 1;
    else if (k == kappa) { s1 = (rank < k_ties) ? 1 : 0; ++rank; }
    if (out) out[u] = s1;
    kept += s1;
    if (s1 && bits) atomicOr((unsigned long long*)&bits[u >> 6], 1ull << (u & 63));
  }
  kept = block_reduce_sum<int>(kept, sm.redi);
  if (tid == 0) P.kept[head] = kept;
}

__global__ void __launch_bounds__(kCutThreads) cut_topp(LevelParams P) {
  touch_args(P);
  __shared__ CutSmem sm;
  cut_head(P, sm);
}

// grid (ceil(nwcap / kCompactRows), groups).
__global__ void __launch_bounds__(kCompactThreads) compact_level(CompactParams P) {
  touch_args(P);
  constexpr int NW = kCompactThreads / kWave;
  constexpr int RW = kCompactRows;
  __shared__ uint64_t s_words[ZHA_MAX_G][RW];   // this workgroup's rows, per head
  __shared__ int32_t s_cnt[RW];                  // kept entries per row
  __shared__ int32_t s_red[2][NW];
  const int gi = blockIdx.y, x = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const ListGeo geo = list_geo(P.list, gi, P.ucap);
  const int U = geo.U, nrow = (U + 63) >> 6;
  const int r0 = x * RW;
  if (x > 0 && r0 >= nrow) return;              // no rows here (uniform over the block)
  const int nr = min(RW, nrow - r0);            // < 1 only for workgroup 0 of an empty list
  const uint64_t* hb = P.selbits + (int64_t)gi * P.G * P.nwcap;
  // kept entries in rows [0, r0); workgroup 0 counts every row for the total
  const int rlim = (x == 0) ? nrow : r0;
  uint32_t before = 0u, all = 0u;
  for (int r = tid; r < rlim; r += kCompactThreads) {
    const uint32_t c = (uint32_t)__popcll(kept_row(hb, P.nwcap, P.G, r, U));
    all += c;
    before += (r < r0) ? c : 0u;
  }
  if (tid < RW) {
    int c = 0;
    if (tid < nr) {
      const int r = r0 + tid;
      const int valid = U - r * 64;
      const uint64_t vmask = valid >= 64 ? ~0ull : ((1ull << valid) - 1ull);
      uint64_t any = 0ull;
      for (int g = 0; g < P.G; ++g) {
        const uint64_t w = hb[(int64_t)g * P.nwcap + r] & vmask;
        s_words[g][tid] = w;
        any |= w;
      }
      c = __popcll(any);
    }
    s_cnt[tid] = c;
  }
  before = wave_sum_u32(before);
  all = wave_sum_u32(all);
  if (lane == 0) { s_red[0][wave] = (int32_t)before; s_red[1][wave] = (int32_t)all; }
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) { base += s_red[0][w]; tot += s_red[1][w]; }
  if (x == 0 && tid == 0) {
    if (tot > P.kcap) set_status(P.status, ZHA_ECAPACITY);
    P.kcount[gi] = tot > P.kcap ? (int32_t)P.kcap : tot;
  }
  // first output position of row i: lane i of the exclusive scan of the counts
  const int ci = lane < RW ? s_cnt[lane] : 0;
  const int rowoff = base + wave_incl_scan<int>(ci) - ci;
  int32_t* ids = P.kids + (int64_t)gi * P.kcap;
  uint32_t* msk = P.kmask + (int64_t)gi * P.kcap;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));   // lanes below this one
  for (int i = wave; i < nr; i += NW) {
    uint32_t m = 0u;
    for (int g = 0; g < P.G; ++g) m |= (uint32_t)((s_words[g][i] >> lane) & 1ull) << g;
    const uint64_t bal = __ballot(m != 0u);
    const int p = __shfl(rowoff, i) + __popcll(bal & lt);
    if (m != 0u && p < P.kcap) {
      ids[p] = list_id(P.list, geo, gi, (r0 + i) * 64 + lane, nullptr);
      msk[p] = m;
    }
  }
}

// ---------------------------------------------------------------- small levels
//
// A list of at most kSmallCap entries is cut by one wave per head: its
// candidates, keyed (score desc, id asc), are sorted in registers by a bitonic
// network; the masses exp(s - max) in that order, as the same 2^40 fixed point
// cut_topp uses, give the running sums, and the cut is the first entry whose
// running mass reaches p W -- the same integers and the same comparisons as
// cut_topp, so both paths keep the same nodes.  The heads' kept bits are ORed in
// LDS and the kept entries compacted in list order.

constexpr int kSmallCap = 256;
// cut_upper runs one wave per query head of the group, and at least one thread
// per list entry.
template <int GP>
constexpr int small_threads() { return 64 * GP > kSmallCap ? 64 * GP : kSmallCap; }

// Top-p cut of one head over a list of U <= KMAX entries, by one wave; ORs the
// head's bit into or_bits[u] of every kept entry and returns the kept count.
template <int NR, int KMAX = 64 * NR>
__device__ inline int cut_head_wave(const float* sc, const uint32_t* cand_mask, uint32_t bit,
                                    int U, float p, int topk, uint32_t* or_bits, int lane) {
  uint64_t v[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int u = NR * lane + r;
    uint64_t e = 0ull;
    if (u < U && (cand_mask[u] & bit))
      e = ((uint64_t)order_key(sanitize(sc[u])) << 32) | (uint32_t)(~(uint32_t)u);
    v[r] = e;
  }
  wave_sort_desc<NR, KMAX>(v, lane);
  const uint64_t first = rl64(v[0], 0);
  if (first == 0ull) return 0;                       // no candidates
  const float mx = key_score((uint32_t)(first >> 32));
  uint64_t ms[NR];
  uint32_t nc = 0;
  uint64_t own = 0ull;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    ms[r] = (v[r] != 0ull) ? fixmass(cut_mass(key_score((uint32_t)(v[r] >> 32)), mx, topk)) : 0ull;
    own += ms[r];
    nc += __popcll(__ballot(v[r] != 0ull));
  }
  int ic;
  if (topk == 0 && p >= 1.0f) {
    ic = (int)nc - 1;
  } else {
    // running mass in sorted order: this lane's entries follow those of lower lanes
    const uint64_t inc = wave_incl_scan<uint64_t>(own);
    const uint64_t W = rl64(inc, 63);
    const double target = cut_target(p, topk, W);
    uint64_t run = inc - own;
    int rf = NR;   // this lane's first entry whose running mass reaches target
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      run += ms[r];
      if (rf == NR && ms[r] != 0ull && (double)run >= target) rf = r;
    }
    const uint64_t reach = __ballot(rf < NR);
    ic = -1;
    if (reach != 0ull) {
      const int l = __ffsll((long long)reach) - 1;
      ic = NR * l + (int)rl32((uint32_t)rf, l);
    }
    if (ic < 0 || ic > (int)nc - 1) ic = (int)nc - 1;
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    if (v[r] != 0ull && NR * lane + r <= ic) atomicOr(&or_bits[~(uint32_t)v[r]], bit);
  }
  return ic + 1;
}

// The small top levels: every node of every level in the run is scored by one
// launch (score_upper; these levels hold at most kSmallCap nodes each, a few MB
// of summaries per group), then one workgroup per group (cut_upper) walks the
// levels top-down -- cut each head, compact the kept nodes in LDS, take their
// children plus the parentless nodes as the next level's list, gathering that
// list's scores by node id -- and writes the lowest level's kept list.  Scoring
// nodes whose parent was not kept reads summaries the route never uses, but the
// scores of the nodes it does use are the same numbers, so the selection is
// unchanged.

struct UpperLevel {
  const float* khat;           // [BH][ncap][R][d]
  const float* bhat;           // [BH][ncap][R]
  const uint16_t* khat16;      // bf16 copy of khat, read instead when set
  int64_t ncap;
  float* scores;               // [BHq][cap], by node id
  int64_t cap;
  int64_t span;                // C^level
  int32_t shift;               // log2 span
  int32_t* kept;               // [BHq] kept per head (diagnostics)
  int32_t* ucount;             // [BH] candidates per group (diagnostics)
  float p;                     // this level's top-p
  int32_t topk;                // > 0: this level's node budget instead
};

struct UpperParams {
  UpperLevel lv[ZHA_MAX_L];    // lv[0]: level L, lv[k]: level L-k
  int32_t nlev;
  LevelParams base;            // q, geometry, p, status, stale check
  int32_t* kids; uint32_t* kmask; int32_t* kcount; int64_t kcap;   // lowest level's kept list
};

__device__ inline LevelParams upper_level_params(const UpperParams& U, int k) {
  LevelParams P = U.base;
  P.khat = U.lv[k].khat;
  P.bhat = U.lv[k].bhat;
  P.khat16 = U.lv[k].khat16;
  P.ncap = U.lv[k].ncap;
  P.scores = U.lv[k].scores;
  P.ucap = U.lv[k].cap;
  return P;
}

__device__ inline int64_t upper_nodes(const UpperParams& U, int k, int64_t T) {
  const int64_t n = T >> U.lv[k].shift;
  return n < U.lv[k].cap ? n : U.lv[k].cap;
}

template <int D, int GP>
__global__ void __launch_bounds__(256) score_upper(UpperParams U) {
  touch_args(U);
  constexpr int NW = 256 / kWave;
  const int gi = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the queries and the length are loaded together (one round trip); the
  // queries go to LDS for every group size, since the levels of the run may
  // score from fp32 k_hat or from its bf16 copy, whose lanes hold different dims
  __shared__ __attribute__((aligned(16))) float s_q[GP * D];
  float qv[GP][4], qv16[GP][8];
  load_group_queries<D, GP, 4, true>(U.base, gi, lane, qv, s_q);
  int64_t T = U.base.list.T[gi / U.base.H_kv];
  if (T < 0) T = 0;
  if (T > U.base.list.T_cap) T = U.base.list.T_cap;
  int total = 0;
  for (int k = 0; k < U.nlev; ++k) total += (int)upper_nodes(U, k, T);
  __syncthreads();
  // node t's score lines are shared by 8 neighbouring workgroups: one XCD runs them
  for (int t = xcd_grouped_x() * NW + wave; t < total; t += gridDim.x * NW) {
    int k = 0, node = t;
    while (node >= (int)upper_nodes(U, k, T)) { node -= (int)upper_nodes(U, k, T); ++k; }
    const LevelParams P = upper_level_params(U, k);
    if (P.khat16 != nullptr) score_node<D, GP, true, true>(P, gi, node, 0xffffffffu, node, qv16, s_q, lane);
    else score_node<D, GP, false, true>(P, gi, node, 0xffffffffu, node, qv, s_q, lane);
  }
}

template <int GP>
__global__ void __launch_bounds__(small_threads<GP>()) cut_upper(UpperParams U) {
  touch_args(U);
  constexpr int NT = small_threads<GP>();
  constexpr int NW = NT / kWave;
  __shared__ int32_t s_id[kSmallCap];     // this level's list: node ids
  __shared__ uint32_t s_cm[kSmallCap];    //   head masks
  __shared__ float s_sc[GP][kSmallCap];   //   scores per head
  __shared__ uint32_t s_or[kSmallCap];    //   OR of the heads' kept bits
  __shared__ int32_t s_kid[kSmallCap];    // kept list of the level above / this level
  __shared__ uint32_t s_km[kSmallCap];
  __shared__ int32_t s_red[NW];
  const LevelParams& B = U.base;
  const int gi = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // The first two levels' scores of every node and head (scored whole, by
  // node id), loaded with the length: their addresses need neither the length
  // nor the level above's cut, so the walk reads them from LDS.
  constexpr int kPreLv = 2;
  constexpr int kPerT = GP * kSmallCap / NT;
  __shared__ float s_pre[kPreLv][GP][kSmallCap];
  float pre[kPreLv][kPerT];
#pragma unroll
  for (int k = 0; k < kPreLv; ++k) {
    const bool have = k < U.nlev;   // otherwise level 0's (valid) scores are read and unused
    const float* sb = have ? U.lv[k].scores : U.lv[0].scores;
    const int64_t capk = have ? U.lv[k].cap : U.lv[0].cap;
#pragma unroll
    for (int i = 0; i < kPerT; ++i) {
      const int idx = tid + i * NT, g = idx / kSmallCap, u = idx % kSmallCap;
      const int gg = g < B.G ? g : B.G - 1;
      const int64_t uu = u < capk ? u : capk - 1;
      pre[k][i] = sb[((int64_t)gi * B.G + gg) * capk + uu];
    }
  }
  const bool chk = B.check_stale && wave == 0 && (gi % B.H_kv) == 0;
  const int64_t nb = stale_count(B, gi, lane, chk);   // with the length: one round trip
  int64_t T = B.list.T[gi / B.H_kv];
#pragma unroll
  for (int k = 0; k < kPreLv; ++k)
#pragma unroll
    for (int i = 0; i < kPerT; ++i) {
      const int idx = tid + i * NT;
      s_pre[k][idx / kSmallCap][idx % kSmallCap] = pre[k][i];
    }
  __syncthreads();
  stale_check(B, T, nb, lane, chk);
  if (T < 0) T = 0;
  if (T > B.list.T_cap) T = B.list.T_cap;
  const int C = B.list.C, cshift = B.list.cshift;
  const uint32_t full = B.list.full;
  int np = 0;   // kept nodes of the level above
  for (int k = 0; k < U.nlev; ++k) {
    const UpperLevel& lv = U.lv[k];
    const int64_t n_here = upper_nodes(U, k, T);
    int cnt;
    int64_t orph0 = 0;
    if (k == 0) {
      cnt = (int)n_here;
    } else {
      orph0 = (T >> (lv.shift + cshift)) << cshift;
      const int64_t orph = n_here - orph0;
      cnt = np * C + (int)(orph > 0 ? orph : 0);
    }
    if (cnt > kSmallCap) cnt = kSmallCap;
    for (int u = tid; u < kSmallCap; u += NT) {
      s_or[u] = 0u;
      if (u < cnt) {
        int32_t id;
        uint32_t m;
        if (k == 0) { id = u; m = full; }
        else if (u < np * C) { id = s_kid[u >> cshift] * C + (u & (C - 1)); m = s_km[u >> cshift]; }
        else { id = (int32_t)(orph0 + (u - np * C)); m = full; }
        s_id[u] = id;
        s_cm[u] = m;
        if (k < kPreLv)
          for (int g = 0; g < B.G; ++g) s_sc[g][u] = s_pre[k][g][id];
        else
          for (int g = 0; g < B.G; ++g) s_sc[g][u] = lv.scores[((int64_t)gi * B.G + g) * lv.cap + id];
      }
    }
    __syncthreads();
    for (int g = wave; g < B.G; g += NW) {
      int kept;
      if (cnt <= 16) kept = cut_head_wave<1, 16>(s_sc[g], s_cm, 1u << g, cnt, lv.p, lv.topk, s_or, lane);
      else if (cnt <= 64) kept = cut_head_wave<1>(s_sc[g], s_cm, 1u << g, cnt, lv.p, lv.topk, s_or, lane);
      else if (cnt <= 128) kept = cut_head_wave<2>(s_sc[g], s_cm, 1u << g, cnt, lv.p, lv.topk, s_or, lane);
      else kept = cut_head_wave<4>(s_sc[g], s_cm, 1u << g, cnt, lv.p, lv.topk, s_or, lane);
      if (lane == 0) lv.kept[(int64_t)gi * B.G + g] = kept;
    }
    __syncthreads();
    // kept entries in list order become the kept list of this level
    const uint32_t m = (tid < cnt) ? s_or[tid] : 0u;
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
    if (m != 0u) { s_kid[pos] = s_id[tid]; s_km[pos] = m; }
    if (tid == 0) lv.ucount[gi] = cnt;
    np = nsel;
    __syncthreads();
  }
  const int nout = np < U.kcap ? np : (int)U.kcap;
  for (int i = tid; i < nout; i += NT) {
    U.kids[(int64_t)gi * U.kcap + i] = s_kid[i];
    U.kmask[(int64_t)gi * U.kcap + i] = s_km[i];
  }
  if (tid == 0) {
    if (np > U.kcap) set_status(B.status, ZHA_ECAPACITY);
    U.kcount[gi] = nout;
  }
}

// ---------------------------------------------------------------- quality forward
//
// [ZHA] "어떻게 쓰나": the reference queries are fit so that the estimated node
// distribution follows the true one.  Per level and query head this computes
// KL(p || p_hat) over the level's complete nodes, p = softmax_n F_n(q) with F_n
// the exact log-mass of the node's keys, p_hat = softmax_n of the routing score.
// F of the leaves comes from the keys (leaf_logmass), F of a parent is the LSE of
// its children's F (parent_logmass), the scores from score_nodes over every node.

struct QualityParams {
  const float* q;              // [BHq][d]
  const void* K;               // [BH][T_cap][d]
  const int64_t* T;            // [B]
  int64_t T_cap;
  float* F;                    // [BHq][cap] this level's log-mass
  const float* Fc;             // [BHq][ccap] the level below (parent_logmass)
  int64_t cap, ccap;
  int64_t span;                // C^level
  int32_t B, H_kv, G, C, kv_dtype;
  float scale;
};

__device__ inline int64_t clamp_T(const int64_t* Tp, int b, int64_t T_cap) {
  int64_t T = Tp[b];
  if (T < 0) T = 0;
  return T > T_cap ? T_cap : T;
}

// 256 threads per block of 64 keys: thread t takes key t / 4 of the block and a
// quarter of its dims; the quarter dots are summed across the four threads, the
// block's scores staged in LDS, and each (head, leaf) takes the LSE of its C.
template <int D>
__global__ void __launch_bounds__(256) leaf_logmass(QualityParams P) {
  constexpr int DQ = D / 4;
  __shared__ float qs[ZHA_MAX_G][D];
  __shared__ float z[ZHA_MAX_G][64];
  const int gi = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t T = clamp_T(P.T, gi / P.H_kv, P.T_cap);
  const int64_t n1 = T / P.C;
  const int64_t nblk = (n1 * P.C + 63) / 64;
  for (int i = tid; i < P.G * D; i += 256)
    qs[i / D][i % D] = P.q[((int64_t)gi * P.G + i / D) * D + i % D] * P.scale;
  __syncthreads();
  const int kk = tid >> 2, qt = tid & 3;
  for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    const int64_t key = blk * 64 + kk;
    const bool ok = key < n1 * P.C;
    float kv[DQ];
    const int64_t row = ((int64_t)gi * P.T_cap + (ok ? key : 0)) * D + qt * DQ;
    if (P.kv_dtype == ZHA_BF16) {
      const uint16_t* kp = (const uint16_t*)P.K + row;
#pragma unroll
      for (int j = 0; j < DQ; ++j) kv[j] = __uint_as_float((uint32_t)kp[j] << 16);
    } else {
      const float* kp = (const float*)P.K + row;
#pragma unroll
      for (int j = 0; j < DQ; ++j) kv[j] = kp[j];
    }
    for (int g = 0; g < P.G; ++g) {
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < DQ; ++j) acc = fmaf(qs[g][qt * DQ + j], kv[j], acc);
      acc += __shfl_xor(acc, 1, 64);
      acc += __shfl_xor(acc, 2, 64);
      if (qt == 0) z[g][kk] = ok ? acc : -INFINITY;
    }
    __syncthreads();
    const int per = 64 / P.C;                      // leaves in the block
    for (int i = tid; i < per * P.G; i += 256) {
      const int g = i / per, lf = i % per;
      const int64_t leaf = blk * per + lf;
      if (leaf < n1) {
        float m = -INFINITY;
        for (int j = 0; j < P.C; ++j) m = fmaxf(m, z[g][lf * P.C + j]);
        float sum = 0.0f;
        for (int j = 0; j < P.C; ++j) sum += expf(z[g][lf * P.C + j] - m);
        P.F[((int64_t)gi * P.G + g) * P.cap + leaf] = m + logf(sum);
      }
    }
    __syncthreads();
  }
}

__global__ void __launch_bounds__(256) parent_logmass(QualityParams P) {
  const int head = blockIdx.y;
  const int gi = head / P.G;
  const int64_t T = clamp_T(P.T, gi / P.H_kv, P.T_cap);
  const int64_t n = T / P.span;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float* fc = P.Fc + (int64_t)head * P.ccap + i * P.C;
    float m = -INFINITY;
    for (int c = 0; c < P.C; ++c) m = fmaxf(m, fc[c]);
    float sum = 0.0f;
    for (int c = 0; c < P.C; ++c) sum += expf(fc[c] - m);
    P.F[(int64_t)head * P.cap + i] = m + logf(sum);
  }
}

// KL(softmax F || softmax s) over the level's n nodes, one workgroup per head.
__global__ void __launch_bounds__(1024) level_kl(QualityParams P, const float* S, float* kl) {
  constexpr int NW = 1024 / kWave;
  __shared__ float red[NW];
  const int head = blockIdx.x;
  const int gi = head / P.G;
  const int64_t T = clamp_T(P.T, gi / P.H_kv, P.T_cap);
  const int64_t n = T / P.span;
  const float* f = P.F + (int64_t)head * P.cap;
  const float* s = S + (int64_t)head * P.cap;
  if (n == 0) {
    if (threadIdx.x == 0) kl[head] = NAN;
    return;
  }
  float mf = -INFINITY, ms = -INFINITY;
  for (int64_t i = threadIdx.x; i < n; i += 1024) { mf = fmaxf(mf, f[i]); ms = fmaxf(ms, s[i]); }
  mf = block_max_f<NW>(mf, red);
  ms = block_max_f<NW>(ms, red);
  float zf = 0.0f, zs = 0.0f, e = 0.0f;
  for (int64_t i = threadIdx.x; i < n; i += 1024) {
    const float wf = expf(f[i] - mf);
    zf += wf;
    zs += expf(s[i] - ms);
    e += wf * (f[i] - s[i]);
  }
  // fixed-order block sums (no atomics): deterministic
  auto bsum = [&](float v) {
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += red[w];
    __syncthreads();
    return t;
  };
  zf = bsum(zf);
  zs = bsum(zs);
  e = bsum(e);
  if (threadIdx.x == 0) {
    const float lse_f = mf + logf(zf), lse_s = ms + logf(zs);
    kl[head] = e / zf - lse_f + lse_s;
  }
}

// ---------------------------------------------------------------- host

// Scoring grid: one wave per node, at most 128 workgroups per group and about
// 8192 in all (more than stay resident; they are dispatched group by group).
// Measured caps per group of 32, 64, 128, 256 and 512, and none: 128 is best or
// level with the best on every workload (deep 270 -> 195 us per route, gqa128k
// 60 -> 53 us, long1m and rope_batch unchanged); with more, a wave scores too
// few nodes to repay its workgroup's start.
template <int D, int GP, int NT>
static void launch_score_g(const LevelParams& P, dim3 grid, hipStream_t s) {
  const dim3 block(NT);
  const bool h16 = P.khat16 != nullptr;
  if (P.fused) {
    if (h16) hipLaunchKernelGGL((score_nodes<D, GP, true, NT, true>), grid, block, 0, s, P);
    else hipLaunchKernelGGL((score_nodes<D, GP, true, NT, false>), grid, block, 0, s, P);
  } else {
    if (h16) hipLaunchKernelGGL((score_nodes<D, GP, false, NT, true>), grid, block, 0, s, P);
    else hipLaunchKernelGGL((score_nodes<D, GP, false, NT, false>), grid, block, 0, s, P);
  }
}

template <int NT>
static void launch_score_nt(const LevelParams& P, dim3 grid, hipStream_t s) {
  const int GP = P.G <= 4 ? 4 : (P.G <= 8 ? 8 : 16);
  if (P.d == 128) {
    if (GP == 4) launch_score_g<128, 4, NT>(P, grid, s);
    else if (GP == 8) launch_score_g<128, 8, NT>(P, grid, s);
    else launch_score_g<128, 16, NT>(P, grid, s);
  } else {
    if (GP == 4) launch_score_g<64, 4, NT>(P, grid, s);
    else if (GP == 8) launch_score_g<64, 8, NT>(P, grid, s);
    else launch_score_g<64, 16, NT>(P, grid, s);
  }
}

static void launch_score(const LevelParams& P, int64_t ucap, hipStream_t s) {
  const int BH = P.B * P.H_kv;
  int64_t gx = ceil_div(ucap, 4);
  int64_t lim = 8192 / BH;
  if (lim > 128) lim = 128;
  if (lim >= 8) lim = lim / 8 * 8;   // whole rounds of the XCDs
  if (lim < 1) lim = 1;
  if (gx > lim) gx = lim;
  if (gx < 1) gx = 1;
  const dim3 grid((unsigned)gx, (unsigned)BH);
  // few groups (the per-group cap leaves under 1024 workgroups) and lists long
  // enough to keep them busy: eight waves per workgroup instead of four, so the
  // GPU holds as many waves in flight (deep's levels 3 to 1: 62 -> 48 us at
  // level 1; its 1024-node level 4 was 1.2 us slower with them)
  if (gx * BH < 1024 && ucap >= 2048) launch_score_nt<512>(P, grid, s);
  else launch_score_nt<256>(P, grid, s);
}

static void launch_upper(const UpperParams& U, hipStream_t s) {
  const int BH = U.base.B * U.base.H_kv;
  int64_t nodes = 0;
  for (int k = 0; k < U.nlev; ++k) nodes += U.lv[k].cap;
  int64_t gx = ceil_div(nodes, 4);   // one node per wave
  gx = (gx + 7) / 8 * 8;              // whole rounds of the XCDs
  if (gx < 1) gx = 1;
  const dim3 grid((unsigned)gx, (unsigned)BH);
  const int GP = U.base.G <= 4 ? 4 : (U.base.G <= 8 ? 8 : 16);
  if (U.base.d == 128) {
    if (GP == 4) hipLaunchKernelGGL((score_upper<128, 4>), grid, dim3(256), 0, s, U);
    else if (GP == 8) hipLaunchKernelGGL((score_upper<128, 8>), grid, dim3(256), 0, s, U);
    else hipLaunchKernelGGL((score_upper<128, 16>), grid, dim3(256), 0, s, U);
  } else {
    if (GP == 4) hipLaunchKernelGGL((score_upper<64, 4>), grid, dim3(256), 0, s, U);
    else if (GP == 8) hipLaunchKernelGGL((score_upper<64, 8>), grid, dim3(256), 0, s, U);
    else hipLaunchKernelGGL((score_upper<64, 16>), grid, dim3(256), 0, s, U);
  }
  if (GP == 4) hipLaunchKernelGGL((cut_upper<4>), dim3(BH), dim3(small_threads<4>()), 0, s, U);
  else if (GP == 8) hipLaunchKernelGGL((cut_upper<8>), dim3(BH), dim3(small_threads<8>()), 0, s, U);
  else hipLaunchKernelGGL((cut_upper<16>), dim3(BH), dim3(small_threads<16>()), 0, s, U);
}

// Top-p masses are summed as w 2^40 (w <= 1) in 64 bits, so a cut pool of n
// entries sums to at most n 2^40, which fits while n < 2^24.  The largest pool
// a route cuts is level 1's union list, at most T_cap / C entries; an explicit
// list of zha_route_level holds at most cand_cap.
constexpr int64_t kMaxCutPool = (int64_t(1) << 24) - 1;

static int32_t check_route_common(const zha_cfg* cfg, const float* q, const zha_tree* tree,
                                  const float* p, int np) {
  int32_t rc = zha_check_cfg(cfg);
  if (rc != ZHA_OK) return rc;
  if (cfg->G > 16) return ZHA_EUNSUPPORTED;
  if ((int64_t)cfg->B * cfg->H_kv > 65535) return ZHA_EUNSUPPORTED;
  if (level_cap(*cfg, 1) > kMaxCutPool) return ZHA_EUNSUPPORTED;
  if (q == nullptr || tree == nullptr || p == nullptr) return ZHA_EINVAL;
  for (int i = 0; i < np; ++i)
    if (!(p[i] > 0.0f) || !(p[i] <= 1.0f)) return ZHA_EINVAL;
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
  P.khat16 = tree->khat16[level - 1];
  P.ncap = tree->n_cap[level - 1];
  P.stage = (uint32_t*)((char*)ws + w.stage);
  P.stage_cap = w.stage_cap;
  P.status = (int32_t*)ws;
  P.B = cfg->B; P.H_kv = cfg->H_kv; P.G = cfg->G; P.d = cfg->d; P.R = cfg->R;
  P.scale = cfg->scale; P.p = p;
  P.topk = 0;
  P.ucount_out = nullptr;
  P.sel = nullptr;
  P.selbits = nullptr;
  P.nwcap = 0;
  P.n_built = tree->n_built;
  P.check_stale = 0;
  P.L = cfg->L;
  P.fused = 0;
  P.fbits = nullptr; P.fnwcap = 0; P.fucap = 0;
  P.fkids = nullptr; P.fkmask = nullptr; P.fkcount = nullptr; P.fkcap = 0;
  ListRef& L = P.list;
  L.ids = nullptr; L.mask = nullptr; L.count = nullptr; L.cap = 0;
  L.pids = nullptr; L.pmask = nullptr; L.pcount = nullptr; L.pcap = 0;
  L.T = nullptr; L.T_cap = cfg->T_cap;
  int64_t span = 1;
  for (int i = 0; i < level; ++i) span *= cfg->C;
  L.span = span;
  L.C = cfg->C;
  L.cshift = __builtin_ctz((unsigned)cfg->C);
  L.level_shift = level * L.cshift;
  L.dummy = (const int64_t*)((const char*)ws + 8);   // inside the 256-byte header
  L.H_kv = cfg->H_kv;
  L.full = (cfg->G >= 32) ? 0xffffffffu : ((1u << cfg->G) - 1u);
  return P;
}

static int32_t route_impl(const zha_cfg* cfg, const float* q, const zha_tree* tree,
                          const int64_t* T, const float* pl, const int32_t* kl, int32_t* leaf_ids,
                          uint32_t* leaf_mask, int32_t* leaf_count, void* ws,
                          size_t ws_bytes, void* stream) {
  int32_t rc = check_route_common(cfg, q, tree, pl, cfg->L);
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

  auto kept_list = [&](int l, int32_t*& kids, uint32_t*& kmask, int32_t*& kcount, int64_t& kcap) {
    if (l > 1) {
      kids = (int32_t*)(base + w.kids[l - 1]);
      kmask = (uint32_t*)(base + w.kmask[l - 1]);
      kcount = (int32_t*)(base + w.kcount[l - 1]);
      kcap = w.cap[l - 1];
    } else {
      kids = leaf_ids; kmask = leaf_mask; kcount = leaf_count; kcap = cfg->leaf_cap;
    }
  };
  // The run of small levels from the top (at most kSmallCap nodes each) is scored
  // in one launch and cut in another; each lower level runs score_nodes,
  // cut_topp and compact_level on the list implied by the level above.
  int lo = L + 1;
  if (w.cap[L - 1] <= kSmallCap) {
    lo = L;
    while (lo > 1 && w.cap[lo - 2] <= kSmallCap) --lo;
    UpperParams U;
    U.base = level_params(cfg, q, tree, L, pl[L - 1], ws, w);
    U.base.list.T = T;
    U.base.check_stale = 1;
    U.nlev = L - lo + 1;
    for (int k = 0; k < U.nlev; ++k) {
      const int l = L - k;
      UpperLevel& v = U.lv[k];
      v.khat = tree->khat[l - 1];
      v.bhat = tree->bhat[l - 1];
      v.khat16 = tree->khat16[l - 1];
      v.ncap = tree->n_cap[l - 1];
      v.scores = (float*)(base + w.scores[l - 1]);
      v.cap = w.cap[l - 1];
      int64_t span = 1;
      for (int i = 0; i < l; ++i) span *= cfg->C;
      v.span = span;
      v.shift = l * __builtin_ctz((unsigned)cfg->C);
      v.kept = (int32_t*)(base + w.kept[l - 1]);
      v.ucount = (int32_t*)(base + w.ucount[l - 1]);
      v.p = pl[l - 1];
      v.topk = kl ? kl[l - 1] : 0;
    }
    kept_list(lo, U.kids, U.kmask, U.kcount, U.kcap);
    launch_upper(U, s);
  }
  // A level of at most kFuseCap nodes (other than the leaves) is compacted by
  // the next level's scoring: one launch fewer per such level.
  bool pend = false;           // the level above awaits its compaction
  ListRef pend_list;
  for (int l = lo - 1; l >= 1; --l) {
    LevelParams P = level_params(cfg, q, tree, l, pl[l - 1], ws, w);
    P.topk = kl ? kl[l - 1] : 0;
    P.list.T = T;
    if (pend) {
      P.fused = 1;
      P.fbits = (const uint64_t*)(base + w.selbits[l]);
      P.fnwcap = w.nwcap[l];
      P.flist = pend_list;
      P.fucap = w.cap[l];
      P.fkids = (int32_t*)(base + w.kids[l]);
      P.fkmask = (uint32_t*)(base + w.kmask[l]);
      P.fkcount = (int32_t*)(base + w.kcount[l]);
      P.fkcap = w.cap[l];
    }
    if (l < L) {   // children of the kept nodes of level l+1, then the parentless nodes
      P.list.pids = (const int32_t*)(base + w.kids[l]);
      P.list.pmask = (const uint32_t*)(base + w.kmask[l]);
      P.list.pcount = (const int32_t*)(base + w.kcount[l]);
      P.list.pcap = w.cap[l];
    }
    P.ucap = w.cap[l - 1];
    P.ucount_out = (int32_t*)(base + w.ucount[l - 1]);
    P.scores = (float*)(base + w.scores[l - 1]);
    P.kept = (int32_t*)(base + w.kept[l - 1]);
    P.check_stale = (l == L) ? 1 : 0;
    P.selbits = (uint64_t*)(base + w.selbits[l - 1]);
    P.nwcap = w.nwcap[l - 1];
    CompactParams X;
    X.list = P.list; X.ucap = P.ucap; X.selbits = P.selbits; X.nwcap = P.nwcap; X.G = cfg->G;
    kept_list(l, X.kids, X.kmask, X.kcount, X.kcap);
    X.status = (int32_t*)ws;
    launch_score(P, P.ucap, s);
    P.check_stale = 0;
    P.fused = 0;
    hipLaunchKernelGGL(cut_topp, dim3(BHq), dim3(kCutThreads), 0, s, P);
    pend = l >= 2 && w.cap[l - 1] <= kFuseCap;
    if (pend) {
      pend_list = P.list;
    } else {
      const int64_t cx = ceil_div(X.nwcap, kCompactRows);
      hipLaunchKernelGGL(compact_level, dim3((unsigned)(cx < 1 ? 1 : cx), (unsigned)BH),
                         dim3(kCompactThreads), 0, s, X);
    }
  }
  return hipGetLastError() == hipSuccess ? ZHA_OK : ZHA_EHIP;
}

}  // namespace zha

extern "C" int32_t zha_route(const zha_cfg* cfg, const float* q, const zha_tree* tree,
                             const int64_t* T, float p, int32_t* leaf_ids,
                             uint32_t* leaf_mask, int32_t* leaf_count, void* ws,
                             size_t ws_bytes, void* stream) {
  if (cfg == nullptr) return ZHA_EINVAL;
  float pl[ZHA_MAX_L];
  const int L = (cfg->L >= 1 && cfg->L <= ZHA_MAX_L) ? cfg->L : 1;
  for (int i = 0; i < L; ++i) pl[i] = p;
  return zha::route_impl(cfg, q, tree, T, pl, nullptr, leaf_ids, leaf_mask, leaf_count, ws,
                         ws_bytes, stream);
}

extern "C" int32_t zha_route_sched(const zha_cfg* cfg, const float* q, const zha_tree* tree,
                                   const int64_t* T, const float* p_levels, int32_t* leaf_ids,
                                   uint32_t* leaf_mask, int32_t* leaf_count, void* ws,
                                   size_t ws_bytes, void* stream) {
  return zha::route_impl(cfg, q, tree, T, p_levels, nullptr, leaf_ids, leaf_mask, leaf_count,
                         ws, ws_bytes, stream);
}

extern "C" int32_t zha_route_topk(const zha_cfg* cfg, const float* q, const zha_tree* tree,
                                  const int64_t* T, const int32_t* k_levels, int32_t* leaf_ids,
                                  uint32_t* leaf_mask, int32_t* leaf_count, void* ws,
                                  size_t ws_bytes, void* stream) {
  if (cfg == nullptr || k_levels == nullptr) return ZHA_EINVAL;
  const int L = (cfg->L >= 1 && cfg->L <= ZHA_MAX_L) ? cfg->L : 1;
  float pl[ZHA_MAX_L];
  for (int i = 0; i < L; ++i) {
    if (k_levels[i] < 1) return ZHA_EINVAL;
    pl[i] = 1.0f;
  }
  return zha::route_impl(cfg, q, tree, T, pl, k_levels, leaf_ids, leaf_mask, leaf_count, ws,
                         ws_bytes, stream);
}

extern "C" int32_t zha_route_level(const zha_cfg* cfg, int32_t level, const float* q,
                                   const zha_tree* tree, float p, const int32_t* cand_ids,
                                   const uint32_t* cand_mask, const int32_t* cand_count,
                                   int32_t cand_cap, float* scores, uint8_t* sel,
                                   void* ws, size_t ws_bytes, void* stream) {
  using namespace zha;
  int32_t rc = check_route_common(cfg, q, tree, &p, 1);
  if (rc != ZHA_OK) return rc;
  if (level < 1 || level > cfg->L) return ZHA_EINVAL;
  if (cand_ids == nullptr || cand_mask == nullptr || cand_count == nullptr ||
      scores == nullptr || sel == nullptr || cand_cap < 1)
    return ZHA_EINVAL;
  rc = zha_check_ws(cfg, ZHA_OP_ROUTE, ws, ws_bytes);
  if (rc != ZHA_OK) return rc;
  const WsLayout w = ws_layout(*cfg);
  if ((int64_t)cand_cap > w.stage_cap) return ZHA_EINVAL;
  if ((int64_t)cand_cap > kMaxCutPool) return ZHA_EUNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  LevelParams P = level_params(cfg, q, tree, level, p, ws, w);
  P.list.ids = cand_ids; P.list.mask = cand_mask; P.list.count = cand_count;
  P.list.cap = cand_cap;
  P.ucap = cand_cap;
  P.scores = scores; P.sel = sel;
  P.kept = (int32_t*)((char*)ws + w.kept[level - 1]);
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

extern "C" int32_t zha_route_quality(const zha_cfg* cfg, const float* q, const zha_kv* kv,
                                     const zha_tree* tree, float* kl, void* ws, size_t ws_bytes,
                                     void* stream) {
  using namespace zha;
  const float one = 1.0f;
  int32_t rc = check_route_common(cfg, q, tree, &one, 1);
  if (rc != ZHA_OK) return rc;
  if (kv == nullptr || kv->K == nullptr || kv->T == nullptr || kl == nullptr) return ZHA_EINVAL;
  rc = zha_check_ws(cfg, ZHA_OP_ROUTE, ws, ws_bytes);
  if (rc != ZHA_OK) return rc;
  const WsLayout w = ws_layout(*cfg);
  hipStream_t s = (hipStream_t)stream;
  char* base = (char*)ws;
  const int BH = cfg->B * cfg->H_kv, BHq = BH * cfg->G, L = cfg->L;
  QualityParams Q;
  Q.q = q; Q.K = kv->K; Q.T = kv->T; Q.T_cap = cfg->T_cap;
  Q.B = cfg->B; Q.H_kv = cfg->H_kv; Q.G = cfg->G; Q.C = cfg->C; Q.kv_dtype = cfg->kv_dtype;
  Q.scale = cfg->scale;
  int64_t span = 1;
  for (int l = 1; l <= L; ++l) {
    span *= cfg->C;
    Q.F = (float*)(base + w.logmass[l - 1]);
    Q.cap = w.cap[l - 1];
    Q.span = span;
    if (l == 1) {
      int64_t gx = ceil_div(cfg->T_cap, 64);
      if (gx > 1024) gx = 1024;
      if (gx < 1) gx = 1;
      if (cfg->d == 128) hipLaunchKernelGGL(leaf_logmass<128>, dim3((unsigned)gx, (unsigned)BH), dim3(256), 0, s, Q);
      else hipLaunchKernelGGL(leaf_logmass<64>, dim3((unsigned)gx, (unsigned)BH), dim3(256), 0, s, Q);
    } else {
      Q.Fc = (const float*)(base + w.logmass[l - 2]);
      Q.ccap = w.cap[l - 2];
      int64_t gx = ceil_div(w.cap[l - 1], 256);
      if (gx < 1) gx = 1;
      if (gx > 64) gx = 64;
      hipLaunchKernelGGL(parent_logmass, dim3((unsigned)gx, (unsigned)BHq), dim3(256), 0, s, Q);
    }
    // the routing score of every node of the level (an implicit list of them all)
    LevelParams P = level_params(cfg, q, tree, l, 1.0f, ws, w);
    P.list.T = kv->T;
    P.ucap = w.cap[l - 1];
    P.scores = (float*)(base + w.scores[l - 1]);
    launch_score(P, P.ucap, s);
    hipLaunchKernelGGL(level_kl, dim3(BHq), dim3(1024), 0, s, Q, (const float*)P.scores,
                       kl + (size_t)(l - 1) * BHq);
  }
  return hipGetLastError() == hipSuccess ? ZHA_OK : ZHA_EHIP;
}
