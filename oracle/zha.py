"""Plain float64 oracle of tree-summarised (ZHA) decode attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Sources (the pages; sections named as they are titled there):
  [ZHA]  "ZHA는 KV 캐시를 트리로 요약해 어텐션 비용을 준(sub)이차로 낮춘다",
         onedev.kr/papers/1556.  Sections: "어떻게 동작하나" (how it works),
         "무엇과 다른가" (how it differs: chunk log-mass, tangent planes, parents,
         RoPE correction, GQA, append cadence), "전제와 한계" (premises and limits:
         level-wise top-p routing, sink, open chunk).
  [ATT]  "Attention", zzong2006.github.io/machine_learning/nlp/attention-function.
         Sections: "Scaled dot-product attention 의 식" (the SDPA equation),
         "토큰 세 개로 직접 계산하기" (three-token worked example), "Attention 은 순서를
         모르므로 위치 정보를 따로 넣는다" (RoPE), "토큰을 하나씩 생성할 때의 attention 과
         KV cache" (decode order), "같은 계산을 메모리 IO 를 줄여서 한다: FlashAttention
         계열" (online softmax worked table, Flash-Decoding).
  [ASM]  "효율적인 긴 컨텍스트 생성을 위한 컨텍스트 기억화", aitrends.kr/articles/59378.
         Sections "핵심 아이디어 이해하기" (decomposability / composability) and
         "방법론" (the (a, Z) merge formula).

Readings taken where the pages are silent or garbled (each is listed with its
reason in the design notes of the repository):
  * scale = 1/sqrt(d) everywhere; passed explicitly so a worked example can pad d.
  * A parent's plane r merges its children's planes r (same r), each evaluated at
    the parent's reference query; children's compressed keys act as keys.
  * Reference query of node n at level l is q_ref[r] (NoPE) or q_ref[r] rotated to
    the node's first key position n * C**l (RoPE, rotate-half pairs, base^(-2i/d)).
  * Top-p: candidates ordered by (fp32 score descending, node id ascending); the
    estimated mass of a candidate is exp(score - max score) over the current pool;
    keep the shortest prefix whose mass is >= p * total; p >= 1 keeps every one.
  * Roots at level l: every node when l = L, else nodes n >= C * n_{l+1}
    ("parentless chunks").  The final key set is {0} U keys of selected leaves U
    the open chunk [C * n_1, T).
  * Merge garbling: a = (Z_A a_A + Z_B a_B) / (Z_A + Z_B), Z = Z_A + Z_B with
    Z = exp(lse), evaluated in the log domain.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

__all__ = [
    "logsumexp", "softmax", "attention", "merge", "rope", "n_nodes",
    "node_ref_query", "leaf_summary", "parent_summary", "build_tree",
    "plane", "node_score", "topp_cut", "topk_cut", "route", "routed_keys", "attend_keys",
    "TopP", "LevelRoute", "Route", "fp32", "node_logmass", "level_kl", "p_schedule",
]


def fp32(x):
    """Round to the nearest float32 value (returned as float64)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# [ATT] "Scaled dot-product attention 의 식": softmax(z)_j = e^{z_j} / sum_l e^{z_l}
# --------------------------------------------------------------------------

def logsumexp(z) -> float:
    """log sum_j exp(z_j) of a 1-D array, shifted by the max for range safety."""
    z = np.asarray(z, dtype=np.float64)
    if z.size == 0:
        return -math.inf
    m = np.max(z)
    if not np.isfinite(m):
        return float(m)
    return float(m + np.log(np.sum(np.exp(z - m))))


def softmax(z) -> np.ndarray:
    """Row softmax of a 1-D array ([ATT] SDPA step 3)."""
    z = np.asarray(z, dtype=np.float64)
    return np.exp(z - logsumexp(z))


def attention(q, K, V, scale: float):
    """One query row of softmax(scale * q K^T) V ([ATT] SDPA steps 1-4).

    Returns (o, lse): the weighted mean of the value rows and the log partition
    log sum_j exp(scale * q.k_j).  An empty key set gives (zeros, -inf).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros(V.shape[1]), -math.inf
    z = scale * (K @ q)
    lse = logsumexp(z)
    w = np.exp(z - lse)
    return w @ V, lse


def merge(a_A, lse_A, a_B, lse_B):
    """[ASM] "방법론": merge two attention states of disjoint key blocks.

    a = (Z_A a_A + Z_B a_B) / (Z_A + Z_B) and Z = Z_A + Z_B, where Z = exp(lse);
    computed as lse = log(e^{lse_A} + e^{lse_B}) and a = sum e^{lse_X - lse} a_X.
    This is the rescaling of [ATT]'s online-softmax table.
    """
    if lse_A == -math.inf:
        return np.asarray(a_B, dtype=np.float64), lse_B
    if lse_B == -math.inf:
        return np.asarray(a_A, dtype=np.float64), lse_A
    lse = float(np.logaddexp(lse_A, lse_B))
    a = math.exp(lse_A - lse) * np.asarray(a_A, np.float64) + \
        math.exp(lse_B - lse) * np.asarray(a_B, np.float64)
    return a, lse


# --------------------------------------------------------------------------
# [ATT] RoPE section: pair i of a vector at position m is rotated by m * theta_i.
# Reading: pairs (i, i + d/2), theta_i = base^(-2i/d), angles in float64.
# --------------------------------------------------------------------------

def rope(x, pos: int, base: float) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    theta = base ** (-2.0 * np.arange(h) / d)
    ang = float(pos) * theta
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


# --------------------------------------------------------------------------
# Tree geometry ([ZHA] "무엇과 다른가": a level-1 summary every C decode steps,
# a level-2 summary every C^2 steps) -- node n at level l covers keys
# [n C^l, (n+1) C^l); only complete nodes exist.
# --------------------------------------------------------------------------

def n_nodes(T: int, C: int, level: int) -> int:
    return T // (C ** level)


def node_ref_query(qref, n: int, level: int, C: int, rope_base: Optional[float]):
    """Reference queries [R, d] of node n at ``level``: q_ref (NoPE) or q_ref rotated
    to the node's first key position n * C^level (RoPE)."""
    qref = np.asarray(qref, dtype=np.float64)
    if rope_base is None:
        return qref
    return rope(qref, n * C ** level, rope_base)


def leaf_summary(qhat, Kc, scale: float):
    """[ZHA] "무엇과 다른가": tangent plane of the chunk log-mass at q_hat.

    F_C(q) = LSE_j(scale * q.k_j); its first-order expansion at q_hat is
    t(q) = scale * q.k_hat + b_hat with k_hat = Attn(q_hat, K_C, K_C) (the
    softmax-weighted mean of the chunk's keys) and b_hat = F_C(q_hat) -
    scale * q_hat.k_hat.  Returns (k_hat [d], b_hat).
    """
    qhat = np.asarray(qhat, dtype=np.float64)
    Kc = np.asarray(Kc, dtype=np.float64)
    z = scale * (Kc @ qhat)
    F = logsumexp(z)
    w = np.exp(z - F)
    khat = w @ Kc
    bhat = F - scale * float(qhat @ khat)
    return khat, bhat


def parent_summary(qhat_P, qhat_c, khat_c, bhat_c, scale: float):
    """[ZHA] "무엇과 다른가": a parent merges its children's summaries the same way.

    Child c's plane r, evaluated at the parent's reference query, is the child's
    own tangent value at its reference query plus the RoPE correction
    scale * <k_hat_{r,c}, q_hat_{r,P} - q_hat_{r,c}>; these values play the
    logits and the children's compressed keys play the keys of the leaf formula.
      qhat_P [d], qhat_c [C, d], khat_c [C, d], bhat_c [C].
    Returns (k_hat_P [d], b_hat_P).
    """
    qhat_P = np.asarray(qhat_P, dtype=np.float64)
    qhat_c = np.asarray(qhat_c, dtype=np.float64)
    khat_c = np.asarray(khat_c, dtype=np.float64)
    bhat_c = np.asarray(bhat_c, dtype=np.float64)
    own = scale * np.sum(qhat_c * khat_c, axis=1) + bhat_c
    correction = scale * np.sum(khat_c * (qhat_P[None, :] - qhat_c), axis=1)
    s = own + correction
    F = logsumexp(s)
    w = np.exp(s - F)
    khat = w @ khat_c
    bhat = F - scale * float(qhat_P @ khat)
    return khat, bhat


def build_tree(K, qref, T: int, C: int, L: int, scale: float,
               rope_base: Optional[float] = None):
    """Summaries of one (sequence, KV head) tree over keys [0, T).

    K [>=T, d] (one KV head's cache), qref [R, d].  Returns a list indexed by
    level-1 of dicts {"khat": [n_l, R, d], "bhat": [n_l, R]}.
    """
    K = np.asarray(K, dtype=np.float64)
    qref = np.asarray(qref, dtype=np.float64)
    R, d = qref.shape
    levels = []
    for level in range(1, L + 1):
        n = n_nodes(T, C, level)
        kh = np.zeros((n, R, d))
        bh = np.zeros((n, R))
        for node in range(n):
            Q = node_ref_query(qref, node, level, C, rope_base)
            if level == 1:
                Kc = K[node * C:(node + 1) * C]
                for r in range(R):
                    kh[node, r], bh[node, r] = leaf_summary(Q[r], Kc, scale)
            else:
                prev = levels[level - 2]
                ch = np.arange(node * C, (node + 1) * C)
                Qc = np.stack([node_ref_query(qref, c, level - 1, C, rope_base) for c in ch])
                for r in range(R):
                    kh[node, r], bh[node, r] = parent_summary(
                        Q[r], Qc[:, r, :], prev["khat"][ch, r, :], prev["bhat"][ch, r], scale)
        levels.append({"khat": kh, "bhat": bh})
    return levels


def plane(q, khat_r, bhat_r, scale: float) -> float:
    """Tangent plane t_r(q) = scale * q.k_hat_r + b_hat_r ([ZHA] "무엇과 다른가")."""
    return scale * float(np.asarray(q, np.float64) @ np.asarray(khat_r, np.float64)) + float(bhat_r)


def node_score(q, khat_n, bhat_n, scale: float) -> float:
    """Estimated log-mass of a node: the maximum over its R tangent planes."""
    q = np.asarray(q, dtype=np.float64)
    return float(np.max(scale * (np.asarray(khat_n, np.float64) @ q) + np.asarray(bhat_n, np.float64)))


# --------------------------------------------------------------------------
# [ZHA] "전제와 한계": level-wise top-p routing.
# --------------------------------------------------------------------------

@dataclass
class TopP:
    ids: np.ndarray            # candidate ids in the pool order given
    scores: np.ndarray         # fp32-rounded scores (float64 array)
    order: np.ndarray          # positions into ids, by (score desc, id asc)
    w: np.ndarray              # exp(score - max) per candidate (pool order)
    W: float                   # total estimated mass
    target: float              # p * W
    m: int                     # selected prefix length
    selected: np.ndarray       # selected ids, ascending


def topp_cut(ids: Sequence[int], scores: Sequence[float], p: float) -> TopP:
    """Shortest prefix, in (score desc, id asc) order, holding fraction p of the mass.

    Scores are rounded to fp32 (the routing precision); the mass of candidate i
    is w_i = exp(s_i - max s) in float64, W = sum w_i; the prefix length m is the
    least m with sum_{i<=m} w_(i) >= p * W (p taken as the fp32 value passed);
    p >= 1 keeps every candidate.
    """
    ids = np.asarray(ids, dtype=np.int64)
    s = fp32(np.asarray(scores, dtype=np.float64))
    n = ids.size
    if n == 0:
        e = np.zeros(0)
        return TopP(ids, s, np.zeros(0, np.int64), e, 0.0, 0.0, 0, np.zeros(0, np.int64))
    order = np.array(sorted(range(n), key=lambda i: (-s[i], ids[i])), dtype=np.int64)
    smax = s[order[0]]
    w = np.exp(s - smax)
    W = float(np.sum(w))
    pf = float(np.float32(p))
    target = pf * W
    if pf >= 1.0:
        m = n
    else:
        m = n
        acc = 0.0
        for k, i in enumerate(order):
            acc += w[i]
            if acc >= target:
                m = k + 1
                break
    sel = np.sort(ids[order[:m]])
    return TopP(ids, s, order, w, W, target, m, sel)


@dataclass
class LevelRoute:
    level: int
    cand: np.ndarray           # candidate node ids (children of selected, then roots)
    cut: TopP


@dataclass
class Route:
    levels: List[LevelRoute] = field(default_factory=list)   # top level first
    leaves: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))
    T: int = 0
    C: int = 1

    def level(self, l: int) -> LevelRoute:
        for lr in self.levels:
            if lr.level == l:
                return lr
        raise KeyError(l)


def topk_cut(ids: Sequence[int], scores: Sequence[float], k: int) -> TopP:
    """The k best candidates in (fp32 score desc, id asc) order, or all of them:
    the fixed-budget selection of a flat chunk indexer ([ZHA] "어떻게 동작하나").
    ``target`` holds the budget used, min(k, n)."""
    ids = np.asarray(ids, dtype=np.int64)
    s = fp32(np.asarray(scores, dtype=np.float64))
    n = ids.size
    if n == 0:
        e = np.zeros(0)
        return TopP(ids, s, np.zeros(0, np.int64), e, 0.0, 0.0, 0, np.zeros(0, np.int64))
    order = np.array(sorted(range(n), key=lambda i: (-s[i], ids[i])), dtype=np.int64)
    w = np.exp(s - s[order[0]])
    m = min(int(k), n)
    return TopP(ids, s, order, w, float(np.sum(w)), float(m), m, np.sort(ids[order[:m]]))


def p_schedule(kind: str, p: float, L: int, gamma: float = 1.0):
    """Per-level top-p for levels 1..L (entry l-1 for level l), in float64.

    [ZHA] "전제와 한계" leaves open how the cut should scale with depth; a route
    keeps at most the product of its levels' p of the estimated mass.  The
    schedules are the plain candidates for that product:
      uniform  p at every level (product p**L);
      root     p**(1/L) at every level (product p);
      power    p**w_l with w_l = l**-gamma / sum_k k**-gamma (product p), so with
               gamma > 0 the leaf level, which holds the most candidates, keeps
               the smallest share.
    """
    p = float(p)
    if kind == "uniform":
        return [p] * L
    if kind == "root":
        return [p ** (1.0 / L)] * L
    if kind == "power":
        w = np.array([float(l) ** (-float(gamma)) for l in range(1, L + 1)])
        return [p ** float(x) for x in w / w.sum()]
    raise ValueError(f"unknown schedule {kind!r}")


def route(q, tree, T: int, C: int, L: int, p, scale: float,
          level_override=None, topk=None) -> Route:
    """Route one query down a tree ([ZHA] "전제와 한계").

    Level L candidates are all level-L nodes.  At each level the candidates are
    scored (max over planes), cut by top-p, and the next level's candidates are
    the children of the selected nodes plus that level's parentless nodes
    (n >= C * n_{l+1}).  An empty pool selects nothing.
    ``p`` is one top-p for every level, or a sequence of L values (entry l-1 for
    level l): a depth schedule, the open question of scaling p with depth that
    the same section raises.
    ``topk`` (one count, or L counts) replaces top-p by a fixed budget per level.
    ``level_override`` (optional dict level -> selected ids) replaces the cut of
    that level, so a comparison can continue from another implementation's
    allowed choice.
    """
    q = np.asarray(q, dtype=np.float64)
    out = Route(T=T, C=C)
    cand = np.arange(n_nodes(T, C, L), dtype=np.int64)
    sel = np.zeros(0, np.int64)
    for level in range(L, 0, -1):
        lv = tree[level - 1]
        scores = np.array([node_score(q, lv["khat"][n], lv["bhat"][n], scale) for n in cand])
        if topk is not None:
            cut = topk_cut(cand, scores, topk[level - 1] if np.ndim(topk) else topk)
        else:
            cut = topp_cut(cand, scores, p[level - 1] if np.ndim(p) else p)
        if level_override is not None and level in level_override:
            cut.selected = np.sort(np.asarray(level_override[level], np.int64))
            cut.m = cut.selected.size
        out.levels.append(LevelRoute(level, cand, cut))
        sel = cut.selected
        if level > 1:
            children = (sel[:, None] * C + np.arange(C)[None, :]).reshape(-1)
            roots = np.arange(C * n_nodes(T, C, level), n_nodes(T, C, level - 1), dtype=np.int64)
            cand = np.concatenate([children, roots]).astype(np.int64)
    out.leaves = sel
    return out


def routed_keys(leaves, T: int, C: int) -> np.ndarray:
    """Final key set: sink token 0, every key of a selected leaf, and the open
    chunk [C * n_1, T) ([ZHA] "전제와 한계"); sorted, each key once."""
    keys = {0} if T > 0 else set()
    for n in np.asarray(leaves, np.int64):
        keys.update(range(int(n) * C, int(n) * C + C))
    keys.update(range(C * n_nodes(T, C, 1), T))
    return np.array(sorted(keys), dtype=np.int64)


def attend_keys(q, K, V, keys, scale: float):
    """Exact softmax attention of q over the listed cache rows."""
    keys = np.asarray(keys, dtype=np.int64)
    return attention(q, np.asarray(K)[keys], np.asarray(V)[keys], scale)


def node_logmass(q, K, T: int, C: int, L: int, scale: float):
    """True log-mass of every complete node for one query, per level (list index
    level-1): F_n(q) = LSE over the node's keys of scale * q.k ([ZHA] "무엇과 다른가":
    the chunk log-mass the tangent planes estimate).  A node's keys are the union
    of its children's, so each level's F is the LSE of its children's F."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    out = []
    n1 = n_nodes(T, C, 1)
    z = scale * (K[: n1 * C] @ q)
    f = np.array([logsumexp(z[n * C:(n + 1) * C]) for n in range(n1)])
    out.append(f)
    for level in range(2, L + 1):
        n = n_nodes(T, C, level)
        f = np.array([logsumexp(out[-1][c * C:(c + 1) * C]) for c in range(n)])
        out.append(f)
    return out


def level_kl(q, K, tree, T: int, C: int, L: int, scale: float):
    """Routing quality per level ([ZHA] "어떻게 쓰나": the reference queries are fit
    so the estimated node distribution matches the true one): KL(p || p_hat) over
    the complete nodes of each level, p = softmax_n F_n(q), p_hat = softmax_n of
    the routing score max_r t_r(q).  Levels with no node give nan."""
    F = node_logmass(q, K, T, C, L, scale)
    out = []
    for level in range(1, L + 1):
        f = F[level - 1]
        if f.size == 0:
            out.append(float("nan"))
            continue
        lv = tree[level - 1]
        s = np.array([node_score(q, lv["khat"][n], lv["bhat"][n], scale) for n in range(f.size)])
        lp = f - logsumexp(f)
        lph = s - logsumexp(s)
        out.append(float(np.sum(np.exp(lp) * (lp - lph))))
    return out
