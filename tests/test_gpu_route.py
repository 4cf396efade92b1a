"""GPU parity of the router (zha_route_level, zha_route) against the oracle.

The GPU and the oracle route over the same fp32 tree (built by the oracle and
rounded to fp32), so any difference is the router's own.  Levels are compared
one at a time; after an allowed mismatch (near-tie or near-threshold, see
route_check) the oracle continues from the GPU's selection.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.gpu_util import f64, lists_from_sets, sets_from_lists
from tests.route_check import classify

pytestmark = pytest.mark.gpu
zha = pytest.importorskip("hierarchical_kv_cache_amd.zha")
DEV = "cuda"
SCORE_TOL = 2e-5  # |s_gpu - s_ref| / max(1, |s_ref|): fp32 dot of d terms + fp32 plane


def t_of(T, b):
    """Cache length of sequence b: T is one length for the batch or one per sequence."""
    return int(T[b]) if isinstance(T, (list, tuple)) else int(T)


def oracle_tree32(wl, T, K):
    """Oracle trees of every (b, h), rounded to fp32: list[b][h] of levels."""
    qref = f64(synth.make_qref(wl, "cpu"))
    trees = []
    for b in range(wl.B):
        row = []
        Tb = t_of(T, b)
        for h in range(wl.H_kv):
            t = O.build_tree(f64(K[b, h, :Tb]), qref[h], Tb, wl.C, wl.L, wl.scale,
                             wl.rope_base if wl.rope else None)
            row.append([{"khat": O.fp32(lv["khat"]), "bhat": O.fp32(lv["bhat"])} for lv in t])
        trees.append(row)
    return trees


def upload(cfg, trees, T):
    tree = zha.Tree(cfg, DEV)
    for b in range(cfg.B):
        Tb = t_of(T, b)
        for h in range(cfg.H_kv):
            for level in range(1, cfg.L + 1):
                n = Tb // cfg.C ** level
                if n:
                    tree.khat[level - 1][b, h, :n] = torch.tensor(trees[b][h][level - 1]["khat"], dtype=torch.float32)
                    tree.bhat[level - 1][b, h, :n] = torch.tensor(trees[b][h][level - 1]["bhat"], dtype=torch.float32)
        for level in range(1, cfg.L + 1):
            tree.n_built[level - 1, b] = Tb // cfg.C ** level
    return tree


def level_sync_compare(cfg, tree_gpu, trees_host, q, T, p, ws, report):
    """Route level by level on the GPU (zha_route_level) and check each level
    against the oracle; returns GPU leaf sets per (b, query head)."""
    qh = f64(q)
    G, C, L = cfg.G, cfg.C, cfg.L
    over = [[{} for _ in range(cfg.Hq)] for _ in range(cfg.B)]
    leaves = [[None] * cfg.Hq for _ in range(cfg.B)]
    for level in range(L, 0, -1):
        cuts, cands = [], []
        for b in range(cfg.B):
            cb, kb = [], []
            for j in range(cfg.Hq):
                rt = O.route(qh[b, j], trees_host[b][j // G], t_of(T, b), C, L, p, cfg.scale,
                             level_override=over[b][j])
                lr = rt.level(level)
                cb.append(lr.cut)
                kb.append(lr.cand)
            cuts.append(cb)
            cands.append(kb)
        ids, mask, count = lists_from_sets(cands, cfg.B, cfg.H_kv, G)
        cap = ids.shape[-1]
        scores = torch.full((cfg.B, cfg.Hq, cap), float("nan"), device=DEV)
        sel = torch.zeros(cfg.B, cfg.Hq, cap, dtype=torch.uint8, device=DEV)
        p_here = p[level - 1] if isinstance(p, (list, tuple)) else p
        zha.route_level(cfg, level, q, tree_gpu, p_here, ids.to(DEV), mask.to(DEV), count.to(DEV),
                        scores, sel, ws)
        torch.cuda.synchronize()
        sc, sl = scores.cpu().numpy(), sel.cpu().numpy()
        idn, cnt = ids.numpy(), count.numpy()
        for b in range(cfg.B):
            for j in range(cfg.Hq):
                h = j // G
                n = int(cnt[b, h])
                cut = cuts[b][j]
                pos = {int(x): k for k, x in enumerate(idn[b, h, :n])}
                # scores of this head's candidates
                for k, cid in enumerate(cut.ids):
                    s_g = sc[b, j, pos[int(cid)]]
                    assert abs(s_g - cut.scores[k]) <= SCORE_TOL * max(1.0, abs(cut.scores[k])), \
                        (level, b, j, int(cid), s_g, cut.scores[k])
                # the GPU keeps only this head's candidates
                gsel = [int(idn[b, h, u]) for u in range(n) if sl[b, j, u]]
                cand_set = set(int(x) for x in cut.ids)
                assert set(gsel) <= cand_set
                ok, note = classify(cut, gsel)
                assert ok, (level, b, j, note)
                if note:
                    report.append((level, b, j, note))
                over[b][j][level] = np.array(sorted(gsel), dtype=np.int64)
                if level == 1:
                    leaves[b][j] = np.array(sorted(gsel), dtype=np.int64)
    return leaves


def _setup(wl, T, step=0):
    K, V = synth.make_cache(wl.with_(N=T, open_len=0, steps=0), "cpu", T)
    cfg = zha.Config(B=wl.B, H_kv=wl.H_kv, G=wl.G, d=wl.d, C=wl.C, L=wl.L, R=wl.R, T_cap=T,
                     kv_dtype=zha.F32 if wl.kv_dtype == "f32" else zha.BF16,
                     rope=wl.rope, rope_base=wl.rope_base)
    trees = oracle_tree32(wl, T, K)
    return cfg, K, V, trees


CASES = {
    "tiny": (synth.WORKLOADS["tiny"], 4096),
    "tiny_iid": (synth.WORKLOADS["tiny"].with_(placement="iid"), 4096),
    "gqa_c16": (synth.WORKLOADS["gqa128k"].with_(H_kv=2, C=16, L=3, n_clusters=256), 20000 + 7),
    "deep": (synth.WORKLOADS["deep"].with_(H_kv=1, C=4, L=5, N=4 ** 5 * 3 + 50), 4 ** 5 * 3 + 50),
    "rope": (synth.WORKLOADS["rope_batch"].with_(B=2, H_kv=1, G=4, C=16, L=3, n_clusters=64),
             16 ** 3 * 2 + 40),
    # sixteen query heads per KV head: the widest head masks (scoring, cut and
    # compaction with G = 16)
    "g16": (synth.WORKLOADS["gqa128k"].with_(H_kv=1, G=16, C=16, L=3, n_clusters=128), 12000 + 3),
    # group sizes that are not a power of two: kernels pad the group to 4, 8 or 16
    # heads, and the padding heads must neither score, cut nor set mask bits
    "g3": (synth.WORKLOADS["gqa128k"].with_(H_kv=2, G=3, C=16, L=3, n_clusters=128), 9000 + 5),
    "g6": (synth.WORKLOADS["gqa128k"].with_(H_kv=1, G=6, C=8, L=3, n_clusters=64), 4000 + 3),
    # the largest chunks: C = 64 and 32 with more than 256 leaves (the full cut path)
    "c64": (synth.WORKLOADS["gqa128k"].with_(H_kv=1, G=4, C=64, L=2, n_clusters=64), 64 * 64 * 5 + 33),
    "c32": (synth.WORKLOADS["gqa128k"].with_(H_kv=1, G=8, C=32, L=3, n_clusters=64), 32 ** 3 + 777),
    # the deepest tree (L = 8, C = 2): seven small levels in the walk, then the leaves
    "deep8": (synth.WORKLOADS["gqa128k"].with_(H_kv=1, G=4, C=2, L=8, n_clusters=32), 2 ** 8 * 3 + 37),
    # three levels below the walk (512, 2048 and 8193 nodes): the first two are
    # compacted by the next level's scoring, the leaves by their own launch
    "fused": (synth.WORKLOADS["gqa128k"].with_(H_kv=2, G=4, C=4, L=7, n_clusters=64), 4 ** 7 * 2 + 5),
    # one level of 20000 / 30000 leaves: candidate pools beyond 16384 entries (the
    # cut's LDS staging of the general path) and beyond 24576 (the staged path's
    # capacity), and final expansions longer than one register batch per wave
    "wide20k": (synth.WORKLOADS["tiny"].with_(G=2, C=2, L=1, R=2, n_clusters=64), 40000),
    "wide30k": (synth.WORKLOADS["tiny"].with_(G=2, C=2, L=1, R=2, n_clusters=64), 60000 + 1),
}


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("p", [0.05, 0.5, 0.9, 0.99])
def test_route_level_parity_and_zha_route_composition(case, p):
    wl, T = CASES[case]
    cfg, K, V, trees = _setup(wl, T)
    tree = upload(cfg, trees, T)
    ws = zha.new_workspace(cfg)
    Tt = torch.full((cfg.B,), T, dtype=torch.int64, device=DEV)
    report = []
    for step in range(3):
        q = synth.make_query(wl, step, T, "cpu").to(DEV)
        leaves = level_sync_compare(cfg, tree, trees, q, T, p, ws, report)
        lst = zha.LeafList(cfg, DEV)
        zha.route(cfg, q, tree, Tt, p, lst.ids, lst.mask, lst.count, ws)
        torch.cuda.synchronize()
        full = sets_from_lists(lst.ids, lst.mask, lst.count, cfg.G)
        for b in range(cfg.B):
            for j in range(cfg.Hq):
                np.testing.assert_array_equal(full[b][j], leaves[b][j])
        assert zha.ws_status(ws) == 0
    for r in report:
        print("allowed:", case, p, r)


def test_p_one_selects_every_leaf_and_matches_dense():
    wl, T = CASES["gqa_c16"]
    cfg, K, V, trees = _setup(wl, T)
    tree = upload(cfg, trees, T)
    ws = zha.new_workspace(cfg)
    Tt = torch.full((cfg.B,), T, dtype=torch.int64, device=DEV)
    q = synth.make_query(wl, 0, T, "cpu").to(DEV)
    lst = zha.LeafList(cfg, DEV)
    zha.route(cfg, q, tree, Tt, 1.0, lst.ids, lst.mask, lst.count, ws)
    torch.cuda.synchronize()
    n1 = T // cfg.C
    assert lst.count.cpu().tolist() == [[n1] * cfg.H_kv] * cfg.B
    assert torch.equal(lst.ids[0, 0, :n1].cpu(), torch.arange(n1, dtype=torch.int32))
    full = (1 << cfg.G) - 1
    assert bool(torch.all(lst.mask[:, :, :n1] == full))
    Kd, Vd = K.to(DEV), V.to(DEV)
    out, lse = torch.empty(cfg.B, cfg.Hq, cfg.d, device=DEV), torch.empty(cfg.B, cfg.Hq, device=DEV)
    out2, lse2 = torch.empty_like(out), torch.empty_like(lse)
    zha.attend(cfg, q, Kd, Vd, Tt, lst.ids, lst.mask, lst.count, out, lse, ws)
    zha.dense_attend(cfg, q, Kd, Vd, Tt, out2, lse2, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_ties_go_to_lower_id_on_gpu():
    """Leaves 3 and 9 hold identical keys: equal scores; with one kept, it is 3."""
    C, d, T = 16, 64, 16 * 16
    g = torch.Generator().manual_seed(0)
    K = torch.randn(1, 1, T, d, generator=g)
    K[0, 0, 3 * C:4 * C] = 4.0 + 0.01 * torch.randn(C, d, generator=g)
    K[0, 0, 9 * C:10 * C] = K[0, 0, 3 * C:4 * C]
    V = torch.randn(1, 1, T, d, generator=g)
    cfg = zha.Config(B=1, H_kv=1, G=1, d=d, C=C, L=1, R=4, T_cap=T, kv_dtype=zha.F32)
    qref = (torch.randn(1, 4, d, generator=g) / 8).to(DEV)
    tree = zha.Tree(cfg, DEV)
    ws = zha.new_workspace(cfg)
    Tt = torch.tensor([T], dtype=torch.int64, device=DEV)
    zha.build(cfg, K.to(DEV), V.to(DEV), Tt, qref, tree, ws)
    q = torch.ones(1, 1, d, device=DEV)
    lst = zha.LeafList(cfg, DEV)
    for p, expect in ((0.3, [3]), (0.6, [3, 9])):
        zha.route(cfg, q, tree, Tt, p, lst.ids, lst.mask, lst.count, ws)
        torch.cuda.synchronize()
        n = int(lst.count[0, 0])
        assert lst.ids[0, 0, :n].cpu().tolist() == expect
    assert torch.equal(tree.khat[0][0, 0, 3], tree.khat[0][0, 0, 9])


def test_stale_tree_is_reported():
    wl, T = CASES["tiny"]
    cfg, K, V, trees = _setup(wl, T)
    tree = upload(cfg, trees, T)
    ws = zha.new_workspace(cfg)
    Tt = torch.full((1,), T + cfg.C, dtype=torch.int64, device=DEV)  # grew without append
    cfg2 = zha.Config(**{**cfg.__dict__, "T_cap": T + cfg.C, "leaf_cap": None})
    tree2 = zha.Tree(cfg2, DEV)
    for level in range(cfg.L):
        n = tree.khat[level].shape[2]
        tree2.khat[level][:, :, :n] = tree.khat[level]
        tree2.bhat[level][:, :, :n] = tree.bhat[level]
        tree2.n_built[level] = tree.n_built[level]
    ws2 = zha.new_workspace(cfg2)
    lst = zha.LeafList(cfg2, DEV)
    q = synth.make_query(wl, 0, T, "cpu").to(DEV)
    zha.route(cfg2, q, tree2, Tt, 0.9, lst.ids, lst.mask, lst.count, ws2)
    assert zha.ws_status(ws2) == zha.ESTALE


@pytest.mark.parametrize("p", [0.5, 0.9, 0.3])
def test_all_equal_scores_take_lowest_ids(p):
    """2048 identical leaves: every score ties, so the cut keeps ceil(p n) leaves
    with the lowest ids (the same count the oracle's rule gives for uniform
    masses).  More than 1024 ties at the threshold exercises the radix path."""
    C, d, n = 16, 64, 2048
    T = C * n
    g = torch.Generator().manual_seed(1)
    chunk = torch.randn(C, d, generator=g)
    K = chunk.repeat(n, 1).reshape(1, 1, T, d)
    V = torch.randn(1, 1, T, d, generator=g)
    cfg = zha.Config(B=1, H_kv=1, G=1, d=d, C=C, L=1, R=2, T_cap=T, kv_dtype=zha.F32)
    qref = (torch.randn(1, 2, d, generator=g) / 8).to(DEV)
    tree = zha.Tree(cfg, DEV)
    ws = zha.new_workspace(cfg)
    Tt = torch.tensor([T], dtype=torch.int64, device=DEV)
    zha.build(cfg, K.to(DEV), V.to(DEV), Tt, qref, tree, ws)
    q = torch.randn(1, 1, d, generator=g).to(DEV)
    lst = zha.LeafList(cfg, DEV)
    zha.route(cfg, q, tree, Tt, p, lst.ids, lst.mask, lst.count, ws)
    torch.cuda.synchronize()
    m = math.ceil(float(np.float32(p)) * n - 1e-9)
    cut = O.topp_cut(np.arange(n), np.zeros(n), p)
    assert cut.m == m
    assert int(lst.count[0, 0]) == m
    assert lst.ids[0, 0, :m].cpu().tolist() == list(range(m))


@pytest.mark.parametrize("n_band", [40, 120, 200, 400, 600, 1000, 1500])
@pytest.mark.parametrize("p", [0.5, 0.9])
def test_cut_crossing_bucket_sizes(n_band, p):
    """Scores set exactly through the summaries (k_hat = 0, so a node's score is
    its best b_hat): n_band nodes sit inside one bucket of the cut's relative-score
    histogram (1/128 of a score unit below the maximum per bucket), around the
    mass cut, so the bucket the cut falls in holds exactly n_band entries.  One
    wave sorts up to 1024 of them in registers (64, 128, 256, 512 or 1024 at a
    time); 1500 take the radix select.  The rest sit far above (kept) or below
    (dropped)."""
    rng = np.random.default_rng(7 + n_band)
    n_hi, n_lo = 5, 3000
    n = n_hi + n_band + n_lo
    C, d, R = 16, 64, 2
    T = n * C
    s = np.empty(n)
    s[:n_hi] = np.float32(3.0 + rng.uniform(0, 1, n_hi))
    mx = float(np.max(s[:n_hi]))
    # the band holds three times the mass of the nodes above it, so the cut
    # (1/3 of the way in at p = 0.5, 87% at p = 0.9) falls inside it; its scores
    # are placed 0.25 .. 0.75 of the way through bucket k, clear of its edges
    b0 = math.log(3.0 * np.exp(s[:n_hi]).sum() / n_band)
    k = math.floor((mx - b0) * 128.0)
    s[n_hi:n_hi + n_band] = mx - (k + 0.25 + 0.5 * rng.uniform(0, 1, n_band)) / 128.0
    s[n_hi + n_band:] = b0 - 14.0 + rng.uniform(0, 1, n_lo)
    s = np.float32(s)
    perm = rng.permutation(n)
    s = s[perm]
    cfg = zha.Config(B=1, H_kv=1, G=1, d=d, C=C, L=1, R=R, T_cap=T, kv_dtype=zha.F32)
    khat = np.zeros((n, R, d), np.float32)
    bhat = np.stack([s, s - np.float32(1.0)], axis=1).astype(np.float32)
    trees = [[[{"khat": khat, "bhat": bhat}]]]
    tree = upload(cfg, trees, T)
    ws = zha.new_workspace(cfg)
    q = torch.zeros(1, 1, d, device=DEV)
    ids = torch.arange(n, dtype=torch.int32).reshape(1, 1, n)
    mask = torch.ones(1, 1, n, dtype=torch.int32)
    count = torch.tensor([[n]], dtype=torch.int32)
    scores = torch.empty(1, 1, n, device=DEV)
    sel = torch.zeros(1, 1, n, dtype=torch.uint8, device=DEV)
    zha.route_level(cfg, 1, q, tree, p, ids.to(DEV), mask.to(DEV), count.to(DEV), scores, sel, ws)
    torch.cuda.synchronize()
    assert torch.equal(scores[0, 0].cpu(), torch.tensor(s)), "scores are the b_hat values"
    cut = O.topp_cut(np.arange(n), s.astype(np.float64), p)
    gsel = np.nonzero(sel[0, 0].cpu().numpy())[0]
    np.testing.assert_array_equal(np.sort(gsel), np.sort(cut.selected))
    # and the whole route (fused paths) keeps the same leaves
    lst = zha.LeafList(cfg, DEV)
    Tt = torch.tensor([T], dtype=torch.int64, device=DEV)
    zha.route(cfg, q, tree, Tt, p, lst.ids, lst.mask, lst.count, ws)
    torch.cuda.synchronize()
    m = int(lst.count[0, 0])
    np.testing.assert_array_equal(lst.ids[0, 0, :m].cpu().numpy(), np.sort(cut.selected))
    assert zha.ws_status(ws) == 0


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("case", ["gqa_c16", "deep", "tiny"])
@pytest.mark.parametrize("kind", ["root", "power", "mixed"])
def test_depth_scheduled_p(case, kind, bf16):
    """zha_route_sched: one top-p per level, level by level against the oracle,
    and end to end equal to the level-by-level composition; also scoring from
    the bf16 copy of k_hat, against the oracle on the rounded summaries."""
    wl, T = CASES[case]
    cfg, K, V, trees = _setup(wl, T)
    tree = upload(cfg, trees, T)
    if bf16:
        trees = bf16_trees(trees)
        tree = upload_bf16(cfg, trees, T)
        for k in tree.khat:
            k.fill_(float("nan"))
    ws = zha.new_workspace(cfg)
    Tt = torch.full((cfg.B,), T, dtype=torch.int64, device=DEV)
    if kind == "mixed":
        pl = [0.6 if l % 2 else 0.97 for l in range(1, cfg.L + 1)]
    else:
        pl = zha.p_schedule(kind, 0.8, cfg.L, gamma=1.5)
    report = []
    for step in range(2):
        q = synth.make_query(wl, step, T, "cpu").to(DEV)
        leaves = level_sync_compare(cfg, tree, trees, q, T, pl, ws, report)
        lst = zha.LeafList(cfg, DEV)
        zha.route(cfg, q, tree, Tt, pl, lst.ids, lst.mask, lst.count, ws)
        torch.cuda.synchronize()
        full = sets_from_lists(lst.ids, lst.mask, lst.count, cfg.G)
        for b in range(cfg.B):
            for j in range(cfg.Hq):
                np.testing.assert_array_equal(full[b][j], leaves[b][j])
        assert zha.ws_status(ws) == 0
    for r in report:
        print("allowed:", case, kind, r)


def _check_topk_selection(cut_ids, cut_scores, k, gsel):
    """The GPU's flat top-k set: min(k, n) entries; every kept entry outranks every
    dropped one in (score desc, id asc) except near-ties (oracle scores within TIE)."""
    from tests.route_check import TIE
    ids = np.asarray(cut_ids, np.int64)
    s = np.asarray(cut_scores, np.float64)
    keep = set(int(x) for x in gsel)
    assert len(keep) == min(k, ids.size)
    kept = [(s[i], ids[i]) for i in range(ids.size) if ids[i] in keep]
    dropped = [(s[i], ids[i]) for i in range(ids.size) if ids[i] not in keep]
    if kept and dropped:
        worst_kept = min(kept, key=lambda t: (t[0], -t[1]))
        best_dropped = max(dropped, key=lambda t: (t[0], -t[1]))
        ok = (worst_kept[0] > best_dropped[0]) or (worst_kept[0] == best_dropped[0] and worst_kept[1] < best_dropped[1])
        assert ok or abs(worst_kept[0] - best_dropped[0]) < TIE, (worst_kept, best_dropped)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("case", ["wide20k", "tiny", "gqa_c16", "deep"])
@pytest.mark.parametrize("frac", [0.1, 0.5])
def test_fixed_budget_topk(case, frac, bf16):
    """zha_route_topk against the oracle's fixed-budget route: a budget of
    frac * n_l nodes per level (at least one); also scoring from the bf16 copy
    of k_hat, against the oracle on the rounded summaries."""
    wl, T = CASES[case]
    cfg, K, V, trees = _setup(wl, T)
    tree = upload(cfg, trees, T)
    if bf16:
        trees = bf16_trees(trees)
        tree = upload_bf16(cfg, trees, T)
        for k in tree.khat:
            k.fill_(float("nan"))
    ws = zha.new_workspace(cfg)
    Tt = torch.full((cfg.B,), T, dtype=torch.int64, device=DEV)
    ks = [max(1, int(frac * (T // cfg.C ** l))) for l in range(1, cfg.L + 1)]
    for step in range(2):
        q = synth.make_query(wl, step, T, "cpu").to(DEV)
        lst = zha.LeafList(cfg, DEV)
        zha.route_topk(cfg, q, tree, Tt, ks, lst.ids, lst.mask, lst.count, ws)
        torch.cuda.synchronize()
        assert zha.ws_status(ws) == 0
        full = sets_from_lists(lst.ids, lst.mask, lst.count, cfg.G)
        qh = f64(q)
        for b in range(cfg.B):
            for j in range(cfg.Hq):
                rt = O.route(qh[b, j], trees[b][j // cfg.G], T, cfg.C, cfg.L, 1.0, cfg.scale,
                             topk=ks)
                if cfg.L == 1:
                    lv = rt.level(1)
                    _check_topk_selection(lv.cut.ids, lv.cut.scores, ks[0], full[b][j])
                else:
                    np.testing.assert_array_equal(full[b][j], rt.leaves)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("case", ["tiny", "gqa_c16", "deep", "rope"])
def test_route_quality_kl_per_level(case, bf16):
    """zha_route_quality against the oracle's per-level KL on the oracle's tree
    (its estimate scored from the bf16 copy of k_hat too, against the oracle on
    the rounded summaries)."""
    wl, T = CASES[case]
    cfg, K, V, trees = _setup(wl, T)
    tree = upload(cfg, trees, T)
    if bf16:
        trees = bf16_trees(trees)
        tree = upload_bf16(cfg, trees, T)
        for k in tree.khat:
            k.fill_(float("nan"))
    ws = zha.new_workspace(cfg)
    Tt = torch.full((cfg.B,), T, dtype=torch.int64, device=DEV)
    Kd, Vd = K.to(DEV), V.to(DEV)
    q = synth.make_query(wl, 0, T, "cpu").to(DEV)
    kl = torch.full((cfg.L, cfg.B, cfg.Hq), -1.0, device=DEV)
    zha.route_quality(cfg, q, Kd, Vd, Tt, tree, kl, ws)
    torch.cuda.synchronize()
    assert zha.ws_status(ws) == 0
    klh = kl.cpu().numpy()
    qh = f64(q)
    for b in range(cfg.B):
        for j in range(cfg.Hq):
            ref = O.level_kl(qh[b, j], f64(K[b, j // cfg.G, :T]), trees[b][j // cfg.G], T, cfg.C,
                             cfg.L, cfg.scale)
            for l in range(cfg.L):
                if np.isnan(ref[l]):
                    assert np.isnan(klh[l, b, j])
                else:
                    assert abs(klh[l, b, j] - ref[l]) <= 5e-4 + 2e-3 * abs(ref[l]), (l, b, j, klh[l, b, j], ref[l])


# ---------------------------------------------------------------- bf16 copy of k_hat

def bf16_trees(trees):
    """The oracle trees with every k_hat rounded to bf16 (nearest even) and
    upcast exactly: the values a zha_tree.khat16 copy holds; b_hat stays fp32."""
    out = []
    for row in trees:
        out.append([[{"khat": f64(torch.tensor(lv["khat"], dtype=torch.float32).to(torch.bfloat16)),
                       "bhat": lv["bhat"]} for lv in levels] for levels in row])
    return out


def upload_bf16(cfg, trees16, T):
    """A tree whose khat16 copies hold the rounded k_hat (khat holds it too)."""
    tree = upload(cfg, trees16, T)
    tree.khat16 = [k.to(torch.bfloat16) for k in tree.khat]
    return tree


@pytest.mark.parametrize("case", ["tiny", "gqa_c16", "deep", "rope", "g16", "g3", "c64", "fused", "wide20k"])
@pytest.mark.parametrize("p", [0.5, 0.9])
def test_route_scores_from_the_bf16_copy(case, p):
    """With zha_tree.khat16 set, every routing call scores from the bf16 copy:
    level by level the same as the oracle routing on the rounded summaries, and
    zha_route's sets equal to that composition.  The fp32 khat of the uploaded
    tree is poisoned, so a level scored from it would fail."""
    wl, T = CASES[case]
    cfg, K, V, trees = _setup(wl, T)
    trees16 = bf16_trees(trees)
    tree = upload_bf16(cfg, trees16, T)
    for k in tree.khat:
        k.fill_(float("nan"))
    ws = zha.new_workspace(cfg)
    Tt = torch.full((cfg.B,), T, dtype=torch.int64, device=DEV)
    report = []
    for step in range(2):
        q = synth.make_query(wl, step, T, "cpu").to(DEV)
        leaves = level_sync_compare(cfg, tree, trees16, q, T, p, ws, report)
        lst = zha.LeafList(cfg, DEV)
        zha.route(cfg, q, tree, Tt, p, lst.ids, lst.mask, lst.count, ws)
        torch.cuda.synchronize()
        full = sets_from_lists(lst.ids, lst.mask, lst.count, cfg.G)
        for b in range(cfg.B):
            for j in range(cfg.Hq):
                np.testing.assert_array_equal(full[b][j], leaves[b][j])
        assert zha.ws_status(ws) == 0
    for r in report:
        print("allowed:", case, p, r)
