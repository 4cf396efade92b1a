"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test names the passage it pins.  Page abbreviations:
  [ATT] "Attention" tutorial page (zzong2006.github.io); [ZHA] the ZHA summary page
  (onedev.kr/papers/1556); [ASM] the Attention-State Memory page (aitrends.kr).
None of these tests runs on a GPU.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- [ATT] worked numbers

def test_pin1_three_token_example():
    """[ATT] 'three-token worked example': S/sqrt2, A and O to 3 dp."""
    g = gold("three_token_example.json")
    Q, K, V = (np.array(g[k], float) for k in ("Q", "K", "V"))
    scale = 1 / math.sqrt(2)
    tol = g["tolerance"]
    for i in range(3):
        # single-key log partition is the scaled score itself
        for j in range(3):
            _, s = O.attention(Q[i], K[j:j + 1], V[j:j + 1], scale)
            assert abs(s - g["S_scaled"][i][j]) < tol
        # with V = I the output row is the weight row A_i
        a, _ = O.attention(Q[i], K, np.eye(3), scale)
        np.testing.assert_allclose(a, g["A"][i], atol=tol)
        o, _ = O.attention(Q[i], K, V, scale)
        np.testing.assert_allclose(o, g["O"][i], atol=tol)
    # the page's row-1 arithmetic: 0.401*[1,0] + 0.198*[0,2] + 0.401*[3,3]
    o1, _ = O.attention(Q[0], K, V, scale)
    np.testing.assert_allclose(o1, [1.604, 1.599], atol=tol)


def test_pin1b_softmax_saturation():
    """[ATT] 'why divide by sqrt(d_k)': softmax of [1,0,-1] and [11.3,0,-11.3]."""
    for case in gold("softmax_saturation.json")["cases"]:
        s = O.softmax(case["z"])
        np.testing.assert_allclose(s[:2], case["softmax"][:2], atol=case["atol"])
        if "rtol_last" in case:
            assert abs(s[2] - case["softmax"][2]) <= case["rtol_last"] * case["softmax"][2]
        else:
            assert abs(s[2] - case["softmax"][2]) <= case["atol"]
        assert abs(s.sum() - 1) < 1e-15


def test_pin2_causal_is_decode_over_prefix():
    """[ATT] 'causal mask': row i of O_causal is a decode of query i over keys 1..i."""
    g3 = gold("three_token_example.json")
    g = gold("causal_example.json")
    Q, K, V = (np.array(g3[k], float) for k in ("Q", "K", "V"))
    scale = 1 / math.sqrt(2)
    for i in range(3):
        o, _ = O.attention(Q[i], K[:i + 1], V[:i + 1], scale)
        np.testing.assert_allclose(o, g["O_causal"][i], atol=g["tolerance"])
    a2, _ = O.attention(Q[1], K[:2], np.eye(2), scale)
    np.testing.assert_allclose(a2, g["A_row2"], atol=g["tolerance"])


def test_pin3_online_softmax_table():
    """[ATT] FlashAttention section: the two-block online-softmax table for token 3,
    reproduced from the (a, Z) merge of [ASM] '방법론'."""
    g3 = gold("three_token_example.json")
    g = gold("online_softmax_table.json")
    Q, K, V = (np.array(g3[k], float) for k in ("Q", "K", "V"))
    scale = 1 / math.sqrt(2)
    tol = g["tolerance"]
    q = Q[2]
    a1, lse1 = O.attention(q, K[:2], V[:2], scale)
    a2, lse2 = O.attention(q, K[2:], V[2:], scale)
    m1, m2 = g["block1"]["m"], g["block2"]["m"]
    # block 1: l = sum exp(z - m) and o = l * a
    l1 = math.exp(lse1 - scale * 1.0)
    assert abs(scale * 1.0 - m1) < tol
    assert abs(l1 - g["block1"]["l"]) < tol
    np.testing.assert_allclose(l1 * a1, g["block1"]["o"], atol=tol)
    assert abs(math.exp(m1 - m2) - g["factor"]) < tol
    a, lse = O.merge(a1, lse1, a2, lse2)
    l = math.exp(lse - scale * 2.0)
    assert abs(l - g["block2"]["l"]) < 2 * tol
    np.testing.assert_allclose(l * a, g["block2"]["o"], atol=2 * tol)
    np.testing.assert_allclose(a, g["final"], atol=tol)


# ---------------------------------------------------------------- [ASM] merge exactness

def test_pin4_merge_exact_any_partition():
    """[ASM] '핵심 아이디어' steps 1-3: merging block states reproduces full attention."""
    rng = np.random.default_rng(1)
    for trial in range(20):
        n, d = rng.integers(2, 200), 16
        K = rng.normal(size=(n, d)) * 2
        V = rng.normal(size=(n, d))
        q = rng.normal(size=d)
        full_o, full_lse = O.attention(q, K, V, 0.25)
        perm = rng.permutation(n)
        cuts = np.sort(rng.choice(np.arange(1, n), size=min(5, n - 1), replace=False))
        parts = np.split(perm, cuts)
        a, lse = np.zeros(d), -math.inf
        for part in parts:
            pa, pl = O.attention(q, K[part], V[part], 0.25)
            a, lse = O.merge(a, lse, pa, pl)
        np.testing.assert_allclose(a, full_o, rtol=1e-12, atol=1e-12)
        assert abs(lse - full_lse) < 1e-12 * max(1, abs(full_lse))
    # an empty block is the identity of the merge
    a, l = O.merge(np.ones(3), 0.5, np.zeros(3), -math.inf)
    assert l == 0.5 and np.all(a == 1)


# ---------------------------------------------------------------- trees

def _small_tree(rope_base=None, T=None, C=4, L=3, R=3, d=8, seed=0):
    rng = np.random.default_rng(seed)
    n_cl = 5
    mu = rng.normal(size=(n_cl, d))
    T = T if T is not None else C ** L * 2 + 3
    z = rng.integers(0, n_cl, size=T)
    K = mu[z] + 0.3 * rng.normal(size=(T, d))
    K[0] *= 4
    if rope_base is not None:
        K = np.stack([O.rope(K[t], t, rope_base) for t in range(T)])
    V = rng.normal(size=(T, d))
    qref = rng.normal(size=(R, d)) / math.sqrt(d)
    scale = 1 / math.sqrt(d)
    tree = O.build_tree(K, qref, T, C, L, scale, rope_base)
    return K, V, qref, tree, T, C, L, scale


def _subtree_lse(q, K, n, level, C, scale):
    keys = K[n * C ** level:(n + 1) * C ** level]
    return O.attention(q, keys, keys, scale)[1]


@pytest.mark.parametrize("rope_base", [None, 100.0])
def test_pin5_lower_bound_every_level(rope_base):
    """[ZHA] '무엇과 다른가': t_r is a tangent plane of the convex log-mass F, so
    t_r(q) <= F(q) everywhere, at every level; equality at the leaves' tangent point
    (and at every level without RoPE)."""
    K, V, qref, tree, T, C, L, scale = _small_tree(rope_base)
    rng = np.random.default_rng(7)
    qs = [rng.normal(size=K.shape[1]) * s for s in (0.3, 1, 3, 10)]
    for level in range(1, L + 1):
        lv = tree[level - 1]
        for n in range(lv["khat"].shape[0]):
            Qn = O.node_ref_query(qref, n, level, C, rope_base)
            for q in qs + list(Qn):
                F = _subtree_lse(q, K, n, level, C, scale)
                for r in range(qref.shape[0]):
                    t = O.plane(q, lv["khat"][n, r], lv["bhat"][n, r], scale)
                    assert t <= F + 1e-9 * max(1.0, abs(F))
            for r in range(qref.shape[0]):
                F = _subtree_lse(Qn[r], K, n, level, C, scale)
                t = O.plane(Qn[r], lv["khat"][n, r], lv["bhat"][n, r], scale)
                if level == 1 or rope_base is None:
                    assert abs(t - F) < 1e-11 * max(1.0, abs(F))
                else:
                    assert t <= F + 1e-9


def test_pin5_rope_parent_is_tangent_of_child_planes():
    """[ZHA] '무엇과 다른가': with RoPE a parent rescoring its children at its own rotated
    reference query adds 1/sqrt(d) <k_hat_c, q_hat_P - q_hat_c>; the result is the
    tangent at q_hat_P of LSE_c t_c(q) (value and gradient), t_c being child plane r."""
    rope_base = 50.0
    K, V, qref, tree, T, C, L, scale = _small_tree(rope_base)
    for level in range(2, L + 1):
        lv, ch = tree[level - 1], tree[level - 2]
        for n in range(lv["khat"].shape[0]):
            QP = O.node_ref_query(qref, n, level, C, rope_base)
            kids = range(n * C, (n + 1) * C)
            for r in range(qref.shape[0]):
                def G(q):
                    return O.logsumexp([O.plane(q, ch["khat"][c, r], ch["bhat"][c, r], scale) for c in kids])
                tP = O.plane(QP[r], lv["khat"][n, r], lv["bhat"][n, r], scale)
                assert abs(tP - G(QP[r])) < 1e-11 * max(1, abs(tP))
                h = 1e-5
                grad = np.array([(G(QP[r] + h * e) - G(QP[r] - h * e)) / (2 * h) for e in np.eye(len(QP[r]))])
                np.testing.assert_allclose(grad, scale * lv["khat"][n, r], atol=1e-7)
    # and the correction is not zero here (positions rotate the reference queries)
    Q0 = O.node_ref_query(qref, 1, 1, C, rope_base)
    assert np.max(np.abs(Q0 - qref)) > 1e-3


def test_pin6_gradient_is_scaled_khat():
    """[ZHA] '무엇과 다른가': the plane's slope is grad_q F at q_hat = k_hat / sqrt(d)."""
    K, V, qref, tree, T, C, L, scale = _small_tree(None)
    h = 1e-5
    for level in (1, 2, 3):
        lv = tree[level - 1]
        for n in range(min(3, lv["khat"].shape[0])):
            for r in range(qref.shape[0]):
                q0 = qref[r]
                grad = np.array([(_subtree_lse(q0 + h * e, K, n, level, C, scale)
                                  - _subtree_lse(q0 - h * e, K, n, level, C, scale)) / (2 * h)
                                 for e in np.eye(len(q0))])
                np.testing.assert_allclose(grad, scale * lv["khat"][n, r], atol=1e-7)


def test_pin7_nope_hierarchy_equals_flat_summary():
    """[ZHA] '무엇과 다른가' + [ASM] composability: without RoPE, a parent built from its
    children equals the leaf formula applied to all keys of its subtree."""
    K, V, qref, tree, T, C, L, scale = _small_tree(None)
    for level in (2, 3):
        lv = tree[level - 1]
        for n in range(lv["khat"].shape[0]):
            keys = K[n * C ** level:(n + 1) * C ** level]
            for r in range(qref.shape[0]):
                kh, bh = O.leaf_summary(qref[r], keys, scale)
                np.testing.assert_allclose(lv["khat"][n, r], kh, rtol=1e-12, atol=1e-12)
                assert abs(lv["bhat"][n, r] - bh) < 1e-12 * max(1, abs(bh))


def test_pin8_closed_forms():
    """q_hat = 0 gives the mean key and b_hat = log C; a one-key chunk gives k_hat = k,
    b_hat = 0 and a plane equal to F everywhere."""
    rng = np.random.default_rng(3)
    Kc = rng.normal(size=(16, 8))
    kh, bh = O.leaf_summary(np.zeros(8), Kc, 0.3)
    np.testing.assert_allclose(kh, Kc.mean(0), rtol=1e-14, atol=1e-14)
    assert abs(bh - math.log(16)) < 1e-14
    k = rng.normal(size=(1, 8))
    kh, bh = O.leaf_summary(rng.normal(size=8), k, 0.3)
    np.testing.assert_allclose(kh, k[0], rtol=1e-14)
    assert abs(bh) < 1e-14
    for _ in range(5):
        q = rng.normal(size=8) * 3
        assert abs(O.plane(q, kh, bh, 0.3) - O.attention(q, k, k, 0.3)[1]) < 1e-12


# ---------------------------------------------------------------- routing ([ZHA] '전제와 한계')

def test_pin9_p_one_selects_everything_and_equals_dense():
    K, V, qref, tree, T, C, L, scale = _small_tree(None, T=4 ** 3 * 2 + 3)
    rng = np.random.default_rng(5)
    for _ in range(4):
        q = rng.normal(size=K.shape[1]) * 2
        rt = O.route(q, tree, T, C, L, 1.0, scale)
        keys = O.routed_keys(rt.leaves, T, C)
        np.testing.assert_array_equal(keys, np.arange(T))
        o, l = O.attend_keys(q, K, V, keys, scale)
        od, ld = O.attention(q, K[:T], V[:T], scale)
        np.testing.assert_allclose(o, od, rtol=1e-13, atol=1e-13)


def _brute_min_subset(w, target):
    n = len(w)
    for size in range(1, n + 1):
        best = max(sum(w[i] for i in c) for c in itertools.combinations(range(n), size))
        if best >= target:
            return size
    return n


def test_pin10_topp_is_minimum_cardinality():
    """'the smallest prefix holding fraction p of the estimated mass' is the smallest
    subset of any kind reaching p*W (brute force over <= 10 candidates)."""
    rng = np.random.default_rng(11)
    for trial in range(60):
        n = int(rng.integers(1, 10))
        ids = rng.permutation(100)[:n]
        scores = rng.normal(size=n) * rng.choice([0.1, 1, 5])
        p = float(rng.choice([0.1, 0.5, 0.75, 0.9, 0.99]))
        cut = O.topp_cut(ids, scores, p)
        assert cut.m == _brute_min_subset(cut.w, cut.target)
        # the kept ones are the highest-scoring
        kept = set(cut.selected.tolist())
        for i in range(n):
            for j in range(n):
                if ids[i] in kept and ids[j] not in kept:
                    assert cut.scores[i] >= cut.scores[j]
    # uniform scores: ceil(p n) candidates, lowest ids
    for n, p in ((16, 0.9), (4, 0.75), (10, 0.5), (7, 0.3)):
        ids = np.arange(n)[::-1] + 5
        cut = O.topp_cut(ids, np.full(n, 2.5), p)
        m = math.ceil(float(np.float32(p)) * n - 1e-12)
        assert cut.m == m
        np.testing.assert_array_equal(cut.selected, np.arange(5, 5 + m))
    # a dominant node: s1 - LSE(rest) >= log(p/(1-p)) gives m = 1
    p = 0.9
    rest = np.array([0.0, -1.0, 0.5])
    s1 = O.logsumexp(rest) + math.log(p / (1 - p)) + 1e-3
    cut = O.topp_cut([4, 1, 2, 3], np.concatenate([[s1], rest]), p)
    assert cut.m == 1 and cut.selected.tolist() == [4]
    # p >= 1 keeps all, p just below 1 may drop underflowing tails only
    cut = O.topp_cut([0, 1, 2], [0.0, -200.0, -300.0], 1.0)
    assert cut.m == 3


def test_pin11_ties_go_to_lower_id():
    """Duplicated chunks (identical keys) give equal scores; the lower id wins."""
    rng = np.random.default_rng(2)
    C, d, T = 4, 8, 64
    K = rng.normal(size=(T, d))
    K[3 * C:4 * C] = K[9 * C:10 * C] = 5 * np.ones(d) + 0.01 * rng.normal(size=(C, d))
    K[9 * C:10 * C] = K[3 * C:4 * C]
    qref = rng.normal(size=(2, d)) / math.sqrt(d)
    scale = 1 / math.sqrt(d)
    tree = O.build_tree(K, qref, T, C, 1, scale)
    q = np.ones(d)
    rt = O.route(q, tree, T, C, 1, 0.3, scale)
    cut = rt.level(1).cut
    assert cut.scores[3] == cut.scores[9]
    assert cut.selected.tolist() == [3]
    rt = O.route(q, tree, T, C, 1, 0.6, scale)
    assert rt.leaves.tolist() == [3, 9]


def test_route_structure_orphans_open_chunk_and_sink():
    """Candidates at each level = children of the selected nodes + parentless nodes;
    final keys = {0} U selected leaves U [C n_1, T)."""
    K, V, qref, tree, T, C, L, scale = _small_tree(None, T=2 * 16 + 3 * 4 + 2, C=4, L=2)
    # n_2 = 2, n_1 = 11: leaves 8, 9, 10 have no parent; open chunk [44, 46)
    assert O.n_nodes(T, C, 2) == 2 and O.n_nodes(T, C, 1) == 11
    rng = np.random.default_rng(9)
    for _ in range(10):
        q = rng.normal(size=K.shape[1]) * 2
        p = float(rng.choice([0.3, 0.6, 0.9]))
        rt = O.route(q, tree, T, C, L, p, scale)
        top = rt.level(2)
        np.testing.assert_array_equal(top.cand, [0, 1])
        lev1 = rt.level(1)
        expect = sorted([c for s in top.cut.selected for c in range(s * C, s * C + C)] + [8, 9, 10])
        assert sorted(lev1.cand.tolist()) == expect
        keys = O.routed_keys(rt.leaves, T, C)
        assert keys[0] == 0 and 44 in keys and 45 in keys
        for leaf in rt.leaves:
            assert all(t in keys for t in range(leaf * C, leaf * C + C))
        assert len(keys) == len(set(keys.tolist()))
    # T < C: no leaves at all, every token is in the open chunk
    rt = O.route(np.ones(K.shape[1]), O.build_tree(K, qref, 3, C, L, scale), 3, C, L, 0.5, scale)
    assert rt.leaves.size == 0
    np.testing.assert_array_equal(O.routed_keys(rt.leaves, 3, C), [0, 1, 2])
    # n_L = 0: every level-(L-1) node is a root
    T2 = 3 * C + 1
    rt = O.route(np.ones(K.shape[1]), O.build_tree(K, qref, T2, C, L, scale), T2, C, L, 0.9, scale)
    assert rt.level(2).cand.size == 0
    np.testing.assert_array_equal(rt.level(1).cand, [0, 1, 2])


def test_routing_concentrated_mass_is_sparse():
    """Adaptivity ([ZHA] '전제와 한계'): a query aligned with one chunk's keys routes to
    few nodes; a query orthogonal to all keys routes to most of them."""
    rng = np.random.default_rng(4)
    C, L, d = 8, 2, 32
    T = C ** L * 4
    K = 0.1 * rng.normal(size=(T, d))
    hot = 17
    direction = rng.normal(size=d)
    K[hot * C:(hot + 1) * C] += 3 * direction
    qref = rng.normal(size=(4, d)) / math.sqrt(d)
    scale = 1 / math.sqrt(d)
    tree = O.build_tree(K, qref, T, C, L, scale)
    rt = O.route(3 * direction, tree, T, C, L, 0.9, scale)
    assert hot in rt.leaves.tolist() and rt.leaves.size <= 3
    rt2 = O.route(np.zeros(d), tree, T, C, L, 0.9, scale)
    assert rt2.leaves.size >= 0.5 * (T // C)


# ---------------------------------------------------------------- RoPE convention

def test_rope_relative_and_generator_agrees():
    """[ATT] RoPE section: rotated dot products depend only on the position
    difference, and values are not rotated; the workload generator's rotation is the
    same convention as the oracle's."""
    rng = np.random.default_rng(8)
    d, base = 16, 1e4
    q, k = rng.normal(size=d), rng.normal(size=d)
    for m, n in ((5, 3), (1000, 998), (0, 0), (7, 20)):
        lhs = O.rope(q, m, base) @ O.rope(k, n, base)
        rhs = O.rope(q, m - n, base) @ k
        assert abs(lhs - rhs) < 1e-10
    assert abs(np.linalg.norm(O.rope(q, 12345, base)) - np.linalg.norm(q)) < 1e-12
    x = torch.tensor(rng.normal(size=(3, d)), dtype=torch.float64)
    pos = torch.tensor([0, 17, 262143])
    got = synth.rope_rotate(x, pos, base).numpy()
    for i in range(3):
        np.testing.assert_allclose(got[i], O.rope(x[i].numpy(), int(pos[i]), base), atol=1e-12)


def test_depth_schedule_indexing_reduces_to_flat_route():
    """With p = 1 at every level above the leaves, the level-wise route keeps every
    upper node, so its leaves are the flat top-p over all leaves (L = 1) at the
    leaf level's p; a schedule entry applied to the wrong level breaks this."""
    rng = np.random.default_rng(5)
    C, d, R, T = 8, 16, 3, 8 ** 3 * 2 + 5
    K = rng.standard_normal((T, d))
    K[: T // 2] += 1.5 * rng.standard_normal(d)
    qref = rng.standard_normal((R, d)) / np.sqrt(d)
    scale = 1 / np.sqrt(d)
    t3 = O.build_tree(K, qref, T, C, 3, scale)
    t1 = O.build_tree(K, qref, T, C, 1, scale)
    for s in range(4):
        q = rng.standard_normal(d) * 2
        for p in (0.5, 0.8):
            deep = O.route(q, t3, T, C, 3, [p, 1.0, 1.0], scale)
            flat = O.route(q, t1, T, C, 1, p, scale)
            np.testing.assert_array_equal(deep.leaves, flat.leaves)
            wrong = O.route(q, t3, T, C, 3, [1.0, 1.0, p], scale)
            assert wrong.leaves.size >= deep.leaves.size
        # a uniform schedule is the scalar route
        a = O.route(q, t3, T, C, 3, [0.7, 0.7, 0.7], scale)
        b = O.route(q, t3, T, C, 3, 0.7, scale)
        np.testing.assert_array_equal(a.leaves, b.leaves)


def test_topk_cut_definition_and_ties():
    """Every kept candidate outranks every dropped one in (score desc, id asc);
    exactly min(k, n) are kept; equal scores keep the lower ids."""
    rng = np.random.default_rng(9)
    for n in (1, 5, 12, 40):
        ids = rng.permutation(100)[:n]
        sc = np.round(rng.standard_normal(n), 1)          # many ties
        for k in (1, 3, 12, 50):
            cut = O.topk_cut(ids, sc, k)
            assert cut.m == min(k, n) == cut.selected.size
            keep = set(cut.selected.tolist())
            s32 = O.fp32(sc)
            for i in range(n):
                for j in range(n):
                    if ids[i] in keep and ids[j] not in keep:
                        assert (s32[i] > s32[j]) or (s32[i] == s32[j] and ids[i] < ids[j])
    tie = O.topk_cut(np.array([7, 3, 9, 1]), np.zeros(4), 2)
    assert tie.selected.tolist() == [1, 3]


def test_flat_topk_route_is_the_leaf_topk():
    rng = np.random.default_rng(10)
    C, d, R, T = 8, 16, 3, 8 * 60 + 3
    K = rng.standard_normal((T, d))
    qref = rng.standard_normal((R, d)) / np.sqrt(d)
    scale = 1 / np.sqrt(d)
    t1 = O.build_tree(K, qref, T, C, 1, scale)
    q = rng.standard_normal(d)
    n1 = T // C
    scores = [O.node_score(q, t1[0]["khat"][n], t1[0]["bhat"][n], scale) for n in range(n1)]
    for k in (1, 7, 60, 100):
        r = O.route(q, t1, T, C, 1, 0.5, scale, topk=k)
        np.testing.assert_array_equal(r.leaves, O.topk_cut(np.arange(n1), scores, k).selected)


def test_level_kl_zero_for_constant_chunks_and_positive_otherwise():
    """Closed form: when every key of a leaf is the same vector k, F_n = scale q.k +
    log C and every tangent plane of the leaf is exactly that (k_hat = k, b_hat =
    log C), so the leaf-level KL is 0.  Distinct keys make the estimate a strict
    lower bound somewhere: KL > 0 at every level."""
    rng = np.random.default_rng(12)
    C, d, R, L = 4, 8, 2, 3
    n1 = 4 ** 2 * 3
    T = n1 * C
    base = rng.standard_normal((n1, d))
    K_const = np.repeat(base, C, axis=0)
    qref = rng.standard_normal((R, d)) / np.sqrt(d)
    scale = 1 / np.sqrt(d)
    tree = O.build_tree(K_const, qref, T, C, L, scale)
    q = rng.standard_normal(d)
    kl = O.level_kl(q, K_const, tree, T, C, 1, scale)
    assert abs(kl[0]) < 1e-12
    K = K_const + 0.5 * rng.standard_normal(K_const.shape)
    tree = O.build_tree(K, qref, T, C, L, scale)
    kl = O.level_kl(q, K, tree, T, C, L, scale)
    assert all(x > 1e-6 for x in kl)


def test_level_kl_matches_brute_force_definition():
    rng = np.random.default_rng(13)
    C, d, R, L = 4, 8, 3, 2
    T = 4 * 4 * 5 + 3
    K = rng.standard_normal((T, d))
    qref = rng.standard_normal((R, d)) / np.sqrt(d)
    scale = 1 / np.sqrt(d)
    tree = O.build_tree(K, qref, T, C, L, scale)
    q = rng.standard_normal(d)
    kl = O.level_kl(q, K, tree, T, C, L, scale)
    z = scale * (K @ q)
    for level in (1, 2):
        span = C ** level
        n = T // span
        # true mass of each node straight from the keys, estimated from the planes
        P = np.array([np.exp(z[i * span:(i + 1) * span]).sum() for i in range(n)])
        P /= P.sum()
        lv = tree[level - 1]
        S = np.array([max(scale * lv["khat"][i][r] @ q + lv["bhat"][i][r] for r in range(R)) for i in range(n)])
        Ph = np.exp(S) / np.exp(S).sum()
        assert abs(kl[level - 1] - float(np.sum(P * np.log(P / Ph)))) < 1e-10


# ---------------------------------------------------------------- node positions and scores

def _periodic_rope_keys(C, T, d, base, seed):
    """Keys whose unrotated content repeats every C tokens: k_t = RoPE(u_{t mod C}, t)."""
    rng = np.random.default_rng(seed)
    u = rng.normal(size=(C, d)) * 1.5
    return np.stack([O.rope(u[t % C], t, base) for t in range(T)])


def test_rope_node_reference_query_is_at_first_key():
    """[ZHA] '무엇과 다른가' (RoPE: a node rescores at its rotated reference query):
    the reference query of node n at level l sits at the node's first key, n C^l.

    (a) Equivariance.  When every leaf holds the same unrotated keys, the keys of
        node n are those of node 0 rotated by n C^l (rotations compose by adding
        angles), so node n's summary must be node 0's with k_hat rotated by n C^l and
        b_hat unchanged; a position of n C^(l-1), or one that ignores n, breaks it.
    (b) Anchor.  Position 0 is the identity rotation, so leaf 0 is the plain leaf
        formula at the unrotated reference queries; the last key as the position
        (an offset shared by every node, which (a) cannot see) breaks it.
    (c) Tangency at the stated point, computed here with rope() and not with the
        oracle's own position helper: every plane r of node n touches its target at
        q* = RoPE(q_ref[r], n C^l) -- the exact log-mass of the leaf's keys, or the
        LSE of the children's planes r for a parent -- and stays below it elsewhere.
    """
    base, C, L, R, d = 40.0, 4, 3, 3, 8
    rng = np.random.default_rng(21)
    qref = rng.normal(size=(R, d)) / math.sqrt(d)
    scale = 1 / math.sqrt(d)
    T = C ** L * 2 + C + 1
    K = _periodic_rope_keys(C, T, d, base, seed=22)
    tree = O.build_tree(K, qref, T, C, L, scale, base)
    for level in range(1, L + 1):
        lv = tree[level - 1]
        for n in range(1, lv["khat"].shape[0]):
            for r in range(R):
                np.testing.assert_allclose(lv["khat"][n, r], O.rope(lv["khat"][0, r], n * C ** level, base),
                                           rtol=0, atol=1e-10)
                assert abs(lv["bhat"][n, r] - lv["bhat"][0, r]) < 1e-10
    for r in range(R):
        kh, bh = O.leaf_summary(qref[r], K[0:C], scale)
        np.testing.assert_allclose(tree[0]["khat"][0, r], kh, rtol=0, atol=1e-13)
        assert abs(tree[0]["bhat"][0, r] - bh) < 1e-13

    # (c) on keys with no period
    K, V, qref, tree, T, C, L, scale = _small_tree(rope_base=base, seed=23)
    probes = [rng.normal(size=K.shape[1]) * s for s in (0.5, 2.0)]
    for level in range(1, L + 1):
        lv = tree[level - 1]
        for n in range(lv["khat"].shape[0]):
            for r in range(qref.shape[0]):
                qs = O.rope(qref[r], n * C ** level, base)
                if level == 1:
                    def target(q):
                        return _subtree_lse(q, K, n, 1, C, scale)
                else:
                    ch = tree[level - 2]
                    kids = range(n * C, (n + 1) * C)

                    def target(q):
                        return O.logsumexp([O.plane(q, ch["khat"][c, r], ch["bhat"][c, r], scale)
                                            for c in kids])
                t_at = O.plane(qs, lv["khat"][n, r], lv["bhat"][n, r], scale)
                assert abs(t_at - target(qs)) < 1e-11 * max(1.0, abs(t_at)), (level, n, r)
                for q in probes:
                    assert O.plane(q, lv["khat"][n, r], lv["bhat"][n, r], scale) <= target(q) + 1e-9


def test_node_score_is_the_best_plane():
    """[ZHA] '무엇과 다른가': a node's estimated log-mass is the maximum of its R
    tangent planes.  Every plane is below the convex log-mass F, so the score is too
    (a sum of planes is not); at a leaf's tangent point q_hat_r plane r equals F and
    the others are below it, so the score equals F there (a minimum or a mean of
    the planes does not)."""
    K, V, qref, tree, T, C, L, scale = _small_tree(None, R=4, seed=24)
    R = qref.shape[0]
    rng = np.random.default_rng(25)
    lv = tree[0]
    strict = 0
    for n in range(lv["khat"].shape[0]):
        for _ in range(3):
            q = rng.normal(size=K.shape[1]) * 2
            F = _subtree_lse(q, K, n, 1, C, scale)
            assert O.node_score(q, lv["khat"][n], lv["bhat"][n], scale) <= F + 1e-12 * max(1, abs(F))
        for r in range(R):
            F = _subtree_lse(qref[r], K, n, 1, C, scale)
            s = O.node_score(qref[r], lv["khat"][n], lv["bhat"][n], scale)
            assert abs(s - F) < 1e-11 * max(1.0, abs(F))
            others = [O.plane(qref[r], lv["khat"][n, x], lv["bhat"][n, x], scale) for x in range(R) if x != r]
            strict += int(max(others) < F - 1e-6)
    # the test has teeth: the other planes are strictly below F at most tangent points
    assert strict > lv["khat"].shape[0]


# ---------------------------------------------------------------- depth schedules

def test_p_schedule_closed_forms():
    """[ZHA] "전제와 한계": a route keeps at most the product of its levels' p.
    root and power keep p in all (their weights sum to one); power's level l
    takes the share l^-gamma of the first level's log p (a flipped exponent, an
    unnormalised weight or a level taken in reverse fails); gamma = 0 reduces
    power to root; a one-level tree is the flat cut at p."""
    for p in (0.5, 0.8, 0.9):
        for L in (1, 2, 3, 6, 8):
            assert O.p_schedule("uniform", p, L) == [p] * L
            root = O.p_schedule("root", p, L)
            assert abs(np.prod(root) - p) < 1e-14 and np.allclose(root, root[0], rtol=0, atol=0)
            for gamma in (0.5, 1.0, 1.5, 3.0):
                pw = O.p_schedule("power", p, L, gamma)
                assert abs(np.prod(pw) - p) < 1e-14
                ratio = np.log(pw) / np.log(pw[0])
                np.testing.assert_allclose(ratio, np.arange(1, L + 1) ** -gamma, rtol=1e-12)
                assert pw == sorted(pw)   # the leaf level (l = 1) keeps the least
            np.testing.assert_allclose(O.p_schedule("power", p, L, 0.0), root, rtol=1e-15)
            if L == 1:
                assert O.p_schedule("power", p, 1, 1.5) == [p] and root == [p]
    with pytest.raises(ValueError):
        O.p_schedule("cubic", 0.9, 3)
