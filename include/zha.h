/*
 * zha.h -- C ABI of libzha: tree-summarised (ZHA) decode attention on gfx950.
 *
 * Sources (the pages; cited by title and section):
 *   [ZHA] "ZHA는 KV 캐시를 트리로 요약해 어텐션 비용을 준(sub)이차로 낮춘다"
 *         (onedev.kr/papers/1556), sections "어떻게 동작하나" (how it works),
 *         "무엇과 다른가" (how it differs), "전제와 한계" (premises and limits).
 *   [ATT] "Attention" (zzong2006.github.io/machine_learning/nlp/attention-function),
 *         sections on the scaled dot-product equation, the KV cache at decode time,
 *         and the FlashAttention family (online softmax, Flash-Decoding).
 *   [ASM] "효율적인 긴 컨텍스트 생성을 위한 컨텍스트 기억화" (aitrends.kr/articles/59378),
 *         section "방법론" (the (a, Z) merge of attention states).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  * B sequences, H_kv KV heads, G query heads per KV head (Hq = H_kv * G; query
 *    head j reads KV head j / G), head dim d, chunk size C, L tree levels, R
 *    reference queries.  Node n of level l covers keys [n C^l, (n+1) C^l); only
 *    complete nodes exist, so a sequence of length T has n_l = T / C^l nodes at
 *    level l and its open chunk is [C n_1, T).  The tree shape is implicit in T:
 *    no child pointers are stored.
 *  * All pointers are DEVICE pointers unless marked (host).  Every buffer is
 *    allocated and freed by the caller; the library allocates nothing, keeps no
 *    pointer after a call returns and holds no global state.  Calls are
 *    asynchronous on ``stream`` (a hipStream_t; NULL = the null stream) and,
 *    except zha_ws_status, never synchronise the host.  Calls on different
 *    streams with disjoint outputs and workspaces may run concurrently.
 *  * Stream capture: every entry point except zha_ws_status (a host
 *    synchronisation) and zha_route_counts (device copies) only launches kernels
 *    on ``stream``, so it can be recorded into a graph and replayed; its scalar
 *    arguments (p, level, topk, max_new_tokens) are fixed at capture.
 *  * Layouts are row-major and dense:
 *      K, V   [B][H_kv][T_cap][d]   fp32 or bf16 (cfg.kv_dtype), keys post-RoPE
 *      T      [B] int64             current length of each sequence (device)
 *      qref   [H_kv][R][d] fp32     reference queries, shared by all levels
 *      khat_l [B][H_kv][n_cap_l][R][d] fp32, bhat_l [B][H_kv][n_cap_l][R] fp32
 *      q      [B][Hq][d] fp32       decode queries, post-RoPE (rotated at T-1)
 *      out    [B][Hq][d] fp32, lse [B][Hq] fp32 (natural log of the partition sum)
 *  * Leaf list (route output, attend input), one per (b, h_kv) group:
 *      leaf_ids  [B][H_kv][leaf_cap] int32   leaf (level-1 node) ids, ascending
 *      leaf_mask [B][H_kv][leaf_cap] uint32  bit g set: query head h_kv*G+g selected it
 *      leaf_count[B][H_kv] int32             valid entries
 *    A group's K/V chunk is read once for all of its query heads that selected it.
 *  * Return value: ZHA_OK or a positive ZHA_E* code.  Arguments are checked on the
 *    host before anything is launched; a failed check launches nothing.  Errors
 *    only the device can see (a stale tree, a capacity overflow) set bits in the
 *    workspace status word, read with zha_ws_status().
 *  * Results are deterministic for fixed inputs: fixed reduction orders, integer
 *    atomics only, no floating-point atomics.
 */
#ifndef ZHA_H
#define ZHA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZHA_MAX_L 8      /* deepest tree supported */
#define ZHA_MAX_G 16     /* query heads per KV head (leaf_mask bits used) */

enum zha_status {
  ZHA_OK = 0,
  ZHA_EINVAL = 1,        /* null pointer, bad shape, p not in (0,1], bad level */
  ZHA_EUNSUPPORTED = 2,  /* d not in {64,128}, C not a power of two in [2,64], dtype;
                            routing: a cut pool above 2^24 - 1 entries (T_cap / C) */
  ZHA_EWORKSPACE = 3,    /* ws_bytes smaller than zha_workspace_bytes() */
  ZHA_ECAPACITY = 4,     /* a list would exceed its capacity (device-detected) */
  ZHA_EHIP = 5,          /* a HIP launch or runtime call failed */
  ZHA_ESTALE = 6         /* tree levels do not match T (device-detected) */
};

enum zha_dtype { ZHA_F32 = 0, ZHA_BF16 = 1 };

enum zha_sched {          /* depth schedules, see zha_p_schedule */
  ZHA_SCHED_UNIFORM = 0, ZHA_SCHED_ROOT = 1, ZHA_SCHED_POWER = 2
};

enum zha_op {             /* workspace sizing, see zha_workspace_bytes */
  ZHA_OP_BUILD = 0, ZHA_OP_ROUTE = 1, ZHA_OP_ATTEND = 2, ZHA_OP_DENSE = 3,
  ZHA_OP_ALL = 4
};

/* Problem geometry (host struct, read during the call only). */
typedef struct zha_cfg {
  int32_t B, H_kv, G, d;
  int32_t C;             /* chunk size: keys per leaf and children per node */
  int32_t L;             /* tree levels, 1..ZHA_MAX_L */
  int32_t R;             /* reference queries per tree, 1..16 */
  float scale;           /* score scale, normally 1/sqrt(d) ([ATT] SDPA equation) */
  int32_t rope;          /* 0: NoPE; 1: reference queries rotated (rotate-half) */
  float rope_base;       /* RoPE base when rope = 1, e.g. 1e6 */
  int32_t kv_dtype;      /* enum zha_dtype */
  int32_t leaf_cap;      /* capacity of a group's leaf list (entries) */
  int64_t T_cap;         /* cache capacity per (b, h_kv) in tokens */
} zha_cfg;

/* KV cache view (host struct holding device pointers). */
typedef struct zha_kv {
  const void* K;         /* [B][H_kv][T_cap][d] */
  const void* V;         /* [B][H_kv][T_cap][d] */
  const int64_t* T;      /* [B] current lengths, 0 <= T <= T_cap */
} zha_kv;

/* Tree storage (host struct holding device pointers); entry l-1 is level l.
 * Zero-initialise it (zha_tree t = {0};) so the optional pointers are NULL. */
typedef struct zha_tree {
  float* khat[ZHA_MAX_L];     /* [B][H_kv][n_cap[l-1]][R][d] */
  float* bhat[ZHA_MAX_L];     /* [B][H_kv][n_cap[l-1]][R] */
  int64_t n_cap[ZHA_MAX_L];   /* node capacity per level, >= T_cap / C^l */
  int64_t* n_built;           /* [L][B] int64 nodes built per level and sequence */
  /* Optional bf16 copy of a level's k_hat (same layout as khat, each value
   * rounded to nearest even), or NULL.  When set, zha_build_level and zha_append
   * write it beside khat, and every routing call scores that level from it
   * instead of khat: half the bytes per node, each k_hat value to 2^-9 relative,
   * b_hat and all arithmetic still fp32.  A level's copy must be set when the
   * level is built and appended, or the route reads stale values. */
  uint16_t* khat16[ZHA_MAX_L];
} zha_tree;

/*
 * Bytes of workspace the given operation needs for this geometry.  A workspace
 * must be zero-filled before its first use (it holds the status word and the
 * append's arrival counters).  Calls that share a workspace must not overlap
 * (use one stream per workspace).  A ZHA_OP_ALL workspace serves every call.
 */
size_t zha_workspace_bytes(const zha_cfg* cfg, int32_t op);

/* Human-readable name of a status code (static string). */
const char* zha_status_str(int32_t status);

/*
 * zha_build_level -- [ZHA] "무엇과 다른가": summarise every complete node of one level.
 *
 * level 1 (leaves): for node n and plane r, with q_hat = qref[h][r] (rotated to
 * position n C when cfg.rope), z_j = scale q_hat.k_j over the node's C keys,
 * F = LSE z, k_hat = sum softmax(z)_j k_j, b_hat = F - scale q_hat.k_hat.
 * level >= 2: the same formula over the node's C children, whose logits are the
 * children's planes r evaluated at the parent's reference query,
 * s_c = scale q_hat_P.k_hat_{r,c} + b_hat_{r,c} (this equals the child's own
 * tangent value plus the RoPE correction 1/sqrt(d) <k_hat_{r,c}, q_hat_P - q_hat_c>),
 * and whose compressed keys k_hat_{r,c} play the keys.
 * Builds nodes [0, T[b] / C^level) of every (b, h_kv) and sets n_built[level-1][b].
 * Level l-1 must be built first.  For prefill.
 */
int32_t zha_build_level(const zha_cfg* cfg, int32_t level, const zha_kv* kv,
                        const float* qref, const zha_tree* tree,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * zha_append -- [ZHA] "무엇과 다른가": incremental growth.  A level-1 summary is
 * added every C decode steps and a level-2 one every C^2 steps; this builds, level
 * by level, every node in [n_built[l-1][b], T[b] / C^l) and advances n_built.
 * max_new_tokens (host) bounds the growth of T since the tree was last current;
 * any growth is handled.  With max_new_tokens <= C (a decode step: at most one
 * new node per level and tree) the whole cascade runs as one launch, one
 * workgroup per (b, h_kv) tree, and the summaries are bit for bit those of
 * zha_build_level (with RoPE and C >= 16, equal to rounding: the prefill advances
 * its rotation angle from leaf to leaf).  Larger growth runs one launch per level.
 * ws: at least zha_workspace_bytes(cfg, ZHA_OP_BUILD) bytes, zero-filled before
 * its first use; the one-launch cascade keeps a per-sequence arrival counter
 * there and returns it to zero.
 */
int32_t zha_append(const zha_cfg* cfg, const zha_kv* kv, const float* qref,
                   const zha_tree* tree, int64_t max_new_tokens,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * zha_route -- [ZHA] "전제와 한계": level-wise top-p routing of each query head.
 *
 * Level L candidates are all level-L nodes.  At each level every candidate n of
 * query head j is scored by its best tangent plane, max_r (scale q_j.k_hat_{r,n}
 * + b_hat_{r,n}) (fp32); candidates are ordered by (score desc, id asc); with
 * w_i = exp(s_i - max s) and W = sum w_i the head keeps the shortest prefix whose
 * mass reaches p W (p >= 1 keeps all).  The next level's candidates are the
 * children of the kept nodes plus the parentless nodes n >= C n_{l+1}.  The kept
 * leaves of all G heads of a group are written as one leaf list (ascending ids,
 * head masks).  The sink token and the open chunk are not in the list; zha_attend
 * adds them.  Requires a current tree (n_built == T / C^l, else ZHA_ESTALE in the
 * workspace status) and cfg.leaf_cap >= T_cap / C.  The cut sums masses exactly
 * as 64-bit fixed point (w 2^40, w <= 1), so every routing call (zha_route,
 * _sched, _topk, _quality, _level) returns ZHA_EUNSUPPORTED when a pool could
 * exceed 2^24 - 1 entries: T_cap / C (level 1, the largest), or cand_cap for
 * zha_route_level.
 */
int32_t zha_route(const zha_cfg* cfg, const float* q, const zha_tree* tree,
                  const int64_t* T, float p,
                  int32_t* leaf_ids, uint32_t* leaf_mask, int32_t* leaf_count,
                  void* ws, size_t ws_bytes, void* stream);

/*
 * zha_route_sched -- zha_route with one top-p per level (host array p_levels,
 * entry l-1 for level l, each in (0, 1]): a depth schedule of the per-level cut,
 * the open question of scaling p with depth raised in [ZHA] "전제와 한계".
 * zha_route(p) equals zha_route_sched with every entry p.
 */
int32_t zha_route_sched(const zha_cfg* cfg, const float* q, const zha_tree* tree,
                        const int64_t* T, const float* p_levels,
                        int32_t* leaf_ids, uint32_t* leaf_mask, int32_t* leaf_count,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * zha_p_schedule -- the per-level top-p of a depth schedule whose levels
 * together keep p ([ZHA] "전제와 한계" leaves open how p should scale with
 * depth; these are the plainest candidates).  Host function: no device work.
 *   ZHA_SCHED_UNIFORM: p at every level (the levels together keep p^L);
 *   ZHA_SCHED_ROOT:    p^(1/L) at every level;
 *   ZHA_SCHED_POWER:   p^(w_l) at level l, w_l = l^-gamma / sum_k k^-gamma, so the
 *                      leaf level (l = 1, the most candidates) cuts hardest when
 *                      gamma > 0.
 * Writes p_levels[l-1] for level l = 1..L (caller-owned host array of L floats),
 * each computed in double and rounded to float.  Returns ZHA_EINVAL for a null
 * p_levels, L outside [1, ZHA_MAX_L], p outside (0, 1], an unknown kind, or a
 * non-finite gamma (power only).
 */
int32_t zha_p_schedule(int32_t kind, float p, int32_t L, float gamma, float* p_levels);

/*
 * zha_route_topk -- zha_route with a fixed node budget per level instead of top-p
 * (host array k_levels, entry l-1 for level l, each >= 1): each query head keeps
 * its k_l best candidates of level l in (score desc, id asc) order, or all of
 * them when fewer.  With L = 1 this is the flat top-K chunk selection that the
 * tree is compared against ([ZHA] "어떻게 동작하나": a flat indexer scores every
 * chunk).
 */
int32_t zha_route_topk(const zha_cfg* cfg, const float* q, const zha_tree* tree,
                       const int64_t* T, const int32_t* k_levels,
                       int32_t* leaf_ids, uint32_t* leaf_mask, int32_t* leaf_count,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * zha_route_quality -- routing quality per level ([ZHA] "어떻게 쓰나": the
 * reference queries are fit so the estimated node distribution follows the true
 * one).  For each level l and query head j, over the level's complete nodes n:
 * kl[(l-1)][b][j] = KL(p || p_hat), p = softmax_n F_n(q_j), F_n the exact
 * log-mass LSE over the node's keys of scale q.k, and p_hat = softmax_n of the
 * routing score max_r (scale q.k_hat_{r,n} + b_hat_{r,n}).  kl is [L][B][Hq] fp32
 * (NaN for a level with no complete node).  Reads every key: a diagnostic, not
 * part of a decode step.  Uses the route workspace.
 */
int32_t zha_route_quality(const zha_cfg* cfg, const float* q, const zha_kv* kv,
                          const zha_tree* tree, float* kl,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * zha_route_level -- one level of zha_route on a given candidate list, for tests
 * and custom schedules.  cand_ids/cand_mask/cand_count use the leaf-list layout
 * with capacity cand_cap ([B][H_kv][cand_cap]; ids ascending, bit g = candidate of
 * head g).  Writes scores [B][Hq][cand_cap] fp32 (every listed entry, every head)
 * and sel [B][Hq][cand_cap] uint8 (1 = kept by that head's top-p cut, 0 otherwise,
 * including entries that are not that head's candidates).
 */
int32_t zha_route_level(const zha_cfg* cfg, int32_t level, const float* q,
                        const zha_tree* tree, float p,
                        const int32_t* cand_ids, const uint32_t* cand_mask,
                        const int32_t* cand_count, int32_t cand_cap,
                        float* scores, uint8_t* sel,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * zha_attend -- exact softmax attention of each query head over its routed key set
 * S_j = {0} U keys(leaves with bit j) U [C (T/C), T), [ZHA] "전제와 한계" (sink and
 * open chunk always included).  Split-K over the leaf list ([ATT] Flash-Decoding):
 * each split produces a partial (max, sum, unnormalised output) and the partials
 * are combined with the (a, Z) merge of [ASM] "방법론".  Writes out and lse.
 * leaf lists must have at most cfg.leaf_cap entries.
 */
int32_t zha_attend(const zha_cfg* cfg, const float* q, const zha_kv* kv,
                   const int32_t* leaf_ids, const uint32_t* leaf_mask,
                   const int32_t* leaf_count, float* out, float* lse,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * zha_attend_static -- zha_attend for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The same kernels and results as zha_attend, with no workspace
 * argument: their scratch (split partials and the chunk
 * prefix) lives in a buffer of 64 MiB that the library holds on every device it
 * runs on, from the first call there until the process ends (the call looks up
 * that device's address on its first use; the current device must be the
 * stream's).  Nothing is allocated or freed.  Returns ZHA_EWORKSPACE when the
 * geometry needs more than 64 MiB of scratch (B Hq 2 s (d + 2) 4 bytes
 * and a little more, s the split slots per query head, about T_cap / 512).
 * status: device int32, or NULL; device-detected errors (ZHA_ECAPACITY) are
 * recorded there with the sticky first-error rule of the workspace status word.
 * Every call on one device shares the buffer and its contents stay from the
 * previous call, so calls that overlap on one device (several streams, several
 * host threads) race: serialise them.
 */
int32_t zha_attend_static(const zha_cfg* cfg, const float* q, const zha_kv* kv,
                          const int32_t* leaf_ids, const uint32_t* leaf_mask,
                          const int32_t* leaf_count, float* out, float* lse,
                          int32_t* status, void* stream);

/*
 * dense_attend -- the same split-K attention over every key [0, T): the dense
 * decode baseline, [ATT] "토큰을 하나씩 생성할 때의 attention 과 KV cache".
 * Uses the same split plan as zha_attend given every leaf with every head bit.
 */
int32_t dense_attend(const zha_cfg* cfg, const float* q, const zha_kv* kv,
                     float* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * zha_route_counts -- diagnostics of the most recent zha_route that used ``ws``:
 * copies, on ``stream``, the per-level size of every group's candidate union
 * list into union_count [L][B][H_kv] and every query head's kept count into
 * kept_count [L][B][Hq] (int32, device; level l at index l-1).  Used to count the
 * summary bytes a step actually scored.
 */
int32_t zha_route_counts(const zha_cfg* cfg, const void* ws, int32_t* union_count,
                         int32_t* kept_count, void* stream);

/*
 * zha_ws_status -- synchronise ``stream``, copy the workspace status word into
 * *status (host; 0 or a ZHA_E* code of the first device-detected error since the
 * last clear) and clear it.  ws must be a workspace used with this library.
 */
int32_t zha_ws_status(void* ws, void* stream, int32_t* status);

#ifdef __cplusplus
}
#endif

#endif /* ZHA_H */
