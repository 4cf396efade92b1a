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
// The top-p cut needs only the threshold, not a full sort: an MSD radix pass
// over the order-preserving 32-bit image of the fp32 scores histograms count and
// mass per 8-bit digit and keeps the digit where the running mass (from the top)
// first reaches p * W; four passes fix the threshold score, ties at it are taken
// in ascending id order.  Masses are w = exp(s - max s) in fp32, accumulated as
// 64-bit fixed point (w * 2^40) with integer atomics, so the cut is deterministic.
#include "zha_internal.hpp"

#include <float.h>

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
// read as 1 KiB contiguous rows per load instruction.  Lane l holds rows
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

template <int D, int GP>
__global__ void __launch_bounds__(256) score_nodes(LevelParams P) {
  constexpr int LPR = D / 4;           // lanes per summary row
  constexpr int RPI = kWave / LPR;     // rows per load instruction
  constexpr int NS = 16 / RPI;         // load instructions per node (R padded to 16)
  constexpr int V0 = NS * GP;          // partial dots per lane
  constexpr int J = GP / 4;            // full dots per lane after the butterfly
  static_assert(V0 / LPR == J, "butterfly shape");
  const int gi = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int U = clamp_count(P.ucount[gi], P.ucap);
  const int t = lane % LPR;

  // the group's queries at this lane's dims
  float qv[GP][4];
#pragma unroll
  for (int g = 0; g < GP; ++g)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      qv[g][j] = (g < P.G) ? P.q[((int64_t)gi * P.G + g) * D + t * 4 + j] : 0.0f;

  const int nwaves = gridDim.x * (blockDim.x >> 6);
  for (int u = blockIdx.x * (blockDim.x >> 6) + wave; u < U; u += nwaves) {
    const int node = P.uids[(int64_t)gi * P.ucap + u];
    if (node < 0 || node >= P.ncap) {   // not a node of this tree: never selected
      if (lane < P.G) P.scores[((int64_t)gi * P.G + lane) * P.ucap + u] = -INFINITY;
      if (lane == 0) set_status(P.status, ZHA_EINVAL);
      continue;
    }
    const float* base = P.khat + ((int64_t)gi * P.ncap + node) * P.R * D;
    float a[V0];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int r = RPI * s + lane / LPR;
      float4 k4 = make_float4(0.f, 0.f, 0.f, 0.f);
      if (r < P.R) k4 = *(const float4*)(base + r * D + t * 4);
#pragma unroll
      for (int g = 0; g < GP; ++g)
        a[s * GP + g] = qv[g][0] * k4.x + qv[g][1] * k4.y + qv[g][2] * k4.z + qv[g][3] * k4.w;
    }
    // butterfly over the LPR lanes of a row: deltas LPR/2 .. 1
    if constexpr (LPR == 32) tr_round<V0, 16>(a, lane);
    if constexpr (LPR >= 16) tr_round<V0 * 16 / LPR, 8>(a, lane);
    tr_round<V0 * 8 / LPR, 4>(a, lane);
    tr_round<V0 * 4 / LPR, 2>(a, lane);
    tr_round<V0 * 2 / LPR, 1>(a, lane);
    // lane now holds dot(s = t/4, g = (t%4)*J + j) for row r = RPI*(t/4) + lane/LPR
    const int r = RPI * (t / 4) + lane / LPR;
    const float bh = (r < P.R) ? P.bhat[((int64_t)gi * P.ncap + node) * P.R + r] : 0.0f;
    float sc[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      float v = (r < P.R) ? fmaf(a[j], P.scale, bh) : -INFINITY;
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
}

// ---------------------------------------------------------------- top-p cut (A4)

constexpr int kCutThreads = 1024;
constexpr int kCutLds = 16384;         // entries staged in LDS; longer lists use the workspace
constexpr double kFix = 1099511627776.0;  // 2^40

__device__ inline uint64_t fixmass(float w) { return (uint64_t)((double)w * kFix); }

__device__ inline float sanitize(float s) { return isfinite(s) ? s : -FLT_MAX; }

struct CutSmem {
  uint32_t key[kCutLds];
  float w[kCutLds];
  uint32_t cnt[256];
  unsigned long long mass[256];
  float redf[16];
  unsigned long long redu[16];
  int32_t redi[16];
  uint32_t bucket;
  unsigned long long above;
};

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

  // max score and candidate count of this head
  float mx = -FLT_MAX;
  int ncand = 0;
  for (int u = tid; u < U; u += kCutThreads)
    if (mk[u] & bit) { mx = fmaxf(mx, sanitize(sc[u])); ++ncand; }
  mx = block_reduce_max<float>(mx, sm.redf);
  ncand = block_reduce_sum<int>(ncand, sm.redi);

  if (ncand == 0 || P.p >= 1.0f) {
    for (int u = tid; u < U; u += kCutThreads) out[u] = (P.p >= 1.0f && (mk[u] & bit)) ? 1 : 0;
    if (tid == 0) P.kept[head] = (P.p >= 1.0f) ? ncand : 0;
    return;
  }

  // stage (key, w); non-candidates get w = 0 and key 0 (never above the threshold)
  unsigned long long wsum = 0;
  for (int u = tid; u < U; u += kCutThreads) {
    uint32_t k = 0u;
    float w = 0.0f;
    if (mk[u] & bit) {
      const float s = sanitize(sc[u]);
      k = order_key(s);
      w = expf(s - mx);
      wsum += fixmass(w);
    }
    skey[u] = k;
    sw[u] = w;
  }
  const unsigned long long W = block_reduce_sum<unsigned long long>(wsum, sm.redu);
  const double target = (double)P.p * (double)W;

  // MSD radix select of the threshold key over four 8-bit digits
  uint32_t prefix = 0u, pmask = 0u;
  unsigned long long above = 0ull;   // mass strictly above the current key range
  uint32_t tie_count = 0u;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kCutThreads) { sm.cnt[i] = 0u; sm.mass[i] = 0ull; }
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
          atomicAdd(&sm.cnt[lb], (uint32_t)__popcll(act));
          atomicAdd(&sm.mass[lb], tot);
        }
      } else if (in) {
        atomicAdd(&sm.cnt[bkt], 1u);
        atomicAdd(&sm.mass[bkt], ms);
      }
    }
    __syncthreads();
    if (tid < 64) {
      // lane owns buckets 4*lane .. 4*lane+3; suffix sums from the top bucket down
      unsigned long long own = 0ull;
#pragma unroll
      for (int i = 0; i < 4; ++i) own += sm.mass[4 * tid + i];
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
          if ((double)(run + sm.mass[bk]) >= target) break;
          run += sm.mass[bk];
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
    tie_count = sm.cnt[bk];
    __syncthreads();
  }
  // ties at the threshold key: all share one mass; take the first k by position
  const uint32_t kappa = prefix;
  __shared__ unsigned long long s_wk;
  for (int u = tid; u < U; u += kCutThreads)
    if (skey[u] == kappa) s_wk = fixmass(sw[u]);   // identical for every tie
  __syncthreads();
  const unsigned long long wk = s_wk;
  double need = (target - (double)above) / (double)(wk == 0ull ? 1ull : wk);
  long long k_ties = (long long)ceil(need);
  if (k_ties < 1) k_ties = 1;
  if (k_ties > (long long)tie_count) k_ties = tie_count;

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
  }
  kept = block_reduce_sum<int>(kept, sm.redi);
  if (tid == 0) P.kept[head] = kept;
}

// ---------------------------------------------------------------- expansion (A5)
//
// One workgroup per group.  The union list is walked in tiles of 1024 entries
// (thread t takes entry tile*1024 + t, so the selection bytes load coalesced);
// an entry is kept when any head kept it, its mask being the OR of the heads'
// bits; a block scan per tile gives its position in list order.  Kept parents
// are staged, then their children are written with consecutive threads on
// consecutive outputs, followed by the parentless nodes of the next level.  The
// final level writes the kept leaves themselves.  The top list (every level-L
// node) is built the same way with no parents; that launch also checks that the
// tree matches T.

struct ExpandParams {
  const int64_t* T;
  const int64_t* n_built;        // [L][B] (top launch only)
  const int32_t* uids; const uint32_t* umask; const int32_t* ucount; int64_t ucap;
  const uint8_t* sel;            // [BHq][ucap]
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

__global__ void __launch_bounds__(kExpandThreads) expand_level(ExpandParams P) {
  __shared__ int32_t red[16];
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
  int32_t* st = P.xstage + (int64_t)gi * P.xcap * 2;
  int32_t* ids = P.nids + (int64_t)gi * P.ncap;
  uint32_t* msk = P.nmask + (int64_t)gi * P.ncap;

  // kept entries in list order
  int nsel = 0;
  for (int base = 0; base < U; base += kExpandThreads) {
    const int u = base + tid;
    uint32_t m = 0u;
    if (u < U)
      for (int g = 0; g < P.G; ++g)
        m |= (P.sel[((int64_t)gi * P.G + g) * P.ucap + u] ? 1u : 0u) << g;
    int tot = 0;
    const int pos = nsel + block_exclusive_scan<int>(m ? 1 : 0, red, &tot);
    if (m) {
      const int32_t id = P.uids[(int64_t)gi * P.ucap + u];
      if (P.final_) {
        if (pos < P.ncap) { ids[pos] = id; msk[pos] = m; }
      } else {
        st[2 * pos] = id;
        st[2 * pos + 1] = (int32_t)m;
      }
    }
    nsel += tot;
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
      ids[o] = st[2 * pi] * P.C + (int32_t)(o & (P.C - 1));
      msk[o] = (uint32_t)st[2 * pi + 1];
    }
    const int64_t first_orph = (int64_t)P.C * n_here;
    for (int64_t i = tid; i < n_orph; i += kExpandThreads) {
      const int64_t o = nch + i;
      if (o < count) { ids[o] = (int32_t)(first_orph + i); msk[o] = full; }
    }
  }
  if (tid == 0) P.ncount[gi] = (int32_t)count;
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

  // top list: every level-L node, every head
  ExpandParams E;
  E.T = T; E.status = (int32_t*)ws; E.n_built = tree->n_built;
  E.B = cfg->B; E.H_kv = cfg->H_kv; E.G = cfg->G; E.C = cfg->C; E.L = L; E.T_cap = cfg->T_cap;
  E.xstage = (int32_t*)(base + w.xstage); E.xcap = w.stage_cap;
  E.level = 0; E.final_ = 0;
  E.uids = nullptr; E.umask = nullptr; E.ucount = nullptr; E.ucap = 1; E.sel = nullptr;
  E.nids = (int32_t*)(base + w.uids[L - 1]);
  E.nmask = (uint32_t*)(base + w.umask[L - 1]);
  E.ncount = (int32_t*)(base + w.ucount[L - 1]);
  E.ncap = w.cap[L - 1];
  E.span_next = span[L];
  hipLaunchKernelGGL(expand_level, dim3(BH), dim3(kExpandThreads), 0, s, E);

  for (int l = L; l >= 1; --l) {
    LevelParams P = level_params(cfg, q, tree, l, p, ws, w);
    P.uids = (const int32_t*)(base + w.uids[l - 1]);
    P.umask = (const uint32_t*)(base + w.umask[l - 1]);
    P.ucount = (const int32_t*)(base + w.ucount[l - 1]);
    P.ucap = w.cap[l - 1];
    P.scores = (float*)(base + w.scores[l - 1]);
    P.sel = (uint8_t*)(base + w.sel[l - 1]);
    P.kept = (int32_t*)(base + w.kept[l - 1]);
    launch_score(P, P.ucap, s);
    hipLaunchKernelGGL(cut_topp, dim3(BHq), dim3(kCutThreads), 0, s, P);
    E.level = l;
    E.uids = P.uids; E.umask = P.umask; E.ucount = P.ucount; E.ucap = P.ucap;
    E.sel = P.sel;
    E.span_next = span[l - 1];
    if (l > 1) {
      E.final_ = 0;
      E.nids = (int32_t*)(base + w.uids[l - 2]);
      E.nmask = (uint32_t*)(base + w.umask[l - 2]);
      E.ncount = (int32_t*)(base + w.ucount[l - 2]);
      E.ncap = w.cap[l - 2];
    } else {
      E.final_ = 1;
      E.nids = leaf_ids; E.nmask = leaf_mask; E.ncount = leaf_count;
      E.ncap = cfg->leaf_cap;
    }
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
