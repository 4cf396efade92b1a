"""End-to-end parity of the decode step on three workloads, run the way a decode
loop runs them (Decoder: prefill build, append when a chunk completes, route,
attend), each step checked against the oracle.

  * tiny: 1 KV head x 1 query head, d = 64, fp32 K/V, 4096 keys from 32 clusters,
    C = 16, L = 2, R = 4.  Eight decode queries against the fixed cache, at
    p = 0.9 and at p = 1.  fp32 outputs within 1e-5 of the oracle; at p = 1 the
    route keeps every leaf and the output equals dense_attend bit for bit.
  * gqa128k: 8 KV heads x 4 query heads, d = 128, bf16 K/V, 131,072 summarised
    tokens + an open chunk of 32, C = 64, L = 3, R = 16, p = 0.9.  All 64 decode
    steps, all 8 KV heads; the chunk that completes at step 32 is appended.
  * long1m: the same heads at 1,048,576 + 32 tokens, 8192 Zipf(1.1) clusters.
    Four spot steps of the 32, on four KV heads.

Routing is compared level by level on the step's own GPU tree (its fp32
summaries), with only the near-tie / near-threshold allowances; the route's final
leaf sets must equal the level-synchronised ones; outputs are compared with the
oracle's exact attention over the keys the GPU routed.  The GPU trees themselves
are checked against the oracle's trees by the builder tests (tests/test_gpu_build.py,
tests/test_gpu_fullsize.py) and, for the appended leaf here, directly.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.gpu_util import TOL, f64, rel_err, sets_from_lists
from tests.test_gpu_build import BHAT_TOL, KHAT_TOL
from tests.test_gpu_route import level_sync_compare, upload

pytestmark = pytest.mark.gpu
zha = pytest.importorskip("hierarchical_kv_cache_amd.zha")
DEV = "cuda"


def host_trees(tree, cfg, T, heads, b=0):
    """The GPU tree of the listed KV heads of sequence b, as float64 levels."""
    out = {}
    for h in heads:
        lv = []
        for level in range(1, cfg.L + 1):
            n = T // cfg.C ** level
            lv.append({"khat": f64(tree.khat[level - 1][b, h, :n]),
                       "bhat": f64(tree.bhat[level - 1][b, h, :n])})
        out[h] = lv
    return out


def check_routing(cfg, trees_h, heads, q, T, p, gpu_sets, tag):
    """Level-synchronised routing of the listed KV heads on their GPU trees
    against the oracle; the decode step's sets must equal the synchronised ones."""
    for h in heads:
        cfg1 = zha.Config(B=1, H_kv=1, G=cfg.G, d=cfg.d, C=cfg.C, L=cfg.L, R=cfg.R, T_cap=T,
                          kv_dtype=cfg.kv_dtype)
        trees = [[trees_h[h]]]
        tree1 = upload(cfg1, trees, T)
        ws1 = zha.new_workspace(cfg1)
        q1 = q[:, h * cfg.G:(h + 1) * cfg.G].contiguous()
        report = []
        leaves = level_sync_compare(cfg1, tree1, trees, q1, T, p, ws1, report)
        for g in range(cfg.G):
            np.testing.assert_array_equal(gpu_sets[0][h * cfg.G + g], leaves[0][g], err_msg=str((tag, h, g)))
        for r in report:
            print("allowed:", tag, h, r)
        del tree1, ws1


def check_outputs(cfg, Kh, Vh, q, out, lse, gpu_sets, heads, T, tol, tag):
    qh = f64(q[0])
    for h in heads:
        for g in range(cfg.G):
            j = h * cfg.G + g
            keys = O.routed_keys(gpu_sets[0][j], T, cfg.C)
            o_ref, lse_ref = O.attend_keys(qh[j], Kh[h], Vh[h], keys, cfg.scale)
            e = rel_err(f64(out[0, j]), o_ref)
            assert e <= tol, (tag, h, g, e)
            assert abs(float(lse[0, j]) - lse_ref) <= tol * max(1.0, abs(lse_ref)), (tag, h, g)


# ---------------------------------------------------------------- tiny, fp32

def test_tiny_fp32_eight_queries_end_to_end():
    wl = synth.WORKLOADS["tiny"]
    T = wl.N
    K, V = synth.make_cache(wl.with_(steps=0), DEV, T)
    qref = synth.make_qref(wl, DEV)
    cfg = zha.Config(B=1, H_kv=1, G=1, d=wl.d, C=wl.C, L=wl.L, R=wl.R, T_cap=T, kv_dtype=zha.F32)
    dec = zha.Decoder(cfg, qref, DEV)
    Tt = torch.tensor([T], dtype=torch.int64, device=DEV)
    dec.prefill(K, V, Tt)
    torch.cuda.synchronize()
    Kh, Vh = {0: f64(K[0, 0, :T])}, {0: f64(V[0, 0, :T])}
    # the GPU tree against the oracle's, every node
    ref = O.build_tree(Kh[0], f64(qref[0]), T, cfg.C, cfg.L, cfg.scale)
    trees_h = host_trees(dec.tree, cfg, T, [0])
    for level in range(1, cfg.L + 1):
        kr, br = ref[level - 1]["khat"], ref[level - 1]["bhat"]
        kg, bg = trees_h[0][level - 1]["khat"], trees_h[0][level - 1]["bhat"]
        assert np.max(np.abs(kg - kr)) / np.max(np.abs(kr)) <= KHAT_TOL[level]
        assert np.max(np.abs(bg - br) / np.maximum(1.0, np.abs(br))) <= BHAT_TOL[level]
    recall = []
    for s in range(wl.steps):
        q = synth.make_query(wl, s, T, DEV)
        out, lse = dec.step(q, K, V, Tt, wl.p)
        out, lse = out.clone(), lse.clone()
        torch.cuda.synchronize()
        assert zha.ws_status(dec.ws) == 0
        sets = sets_from_lists(dec.leaves.ids, dec.leaves.mask, dec.leaves.count, cfg.G)
        check_routing(cfg, trees_h, [0], q, T, wl.p, sets, ("tiny", s))
        check_outputs(cfg, Kh, Vh, q, out, lse, sets, [0], T, TOL["f32"], ("tiny", s))
        # p = 1: every leaf, and the same numbers as the dense kernel
        out1, lse1 = dec.step(q, K, V, Tt, 1.0)
        out1, lse1 = out1.clone(), lse1.clone()
        n1 = T // cfg.C
        assert int(dec.leaves.count[0, 0]) == n1
        assert torch.equal(dec.leaves.ids[0, 0, :n1].cpu(), torch.arange(n1, dtype=torch.int32))
        outd, lsed = dec.dense(q, K, V, Tt)
        torch.cuda.synchronize()
        assert torch.equal(out1, outd) and torch.equal(lse1, lsed), s
        od, ld = O.attention(f64(q[0, 0]), Kh[0], Vh[0], cfg.scale)
        assert rel_err(f64(outd[0, 0]), od) <= TOL["f32"], s
        assert abs(float(lsed[0, 0]) - ld) <= 1e-5 * max(1.0, abs(ld))
        recall.append(float(np.exp(float(lse[0, 0]) - ld)))
    print("tiny p=0.9 dense-mass recall per query:", [round(x, 4) for x in recall])


# ---------------------------------------------------------------- gqa128k, every step

GQA_STEPS = 64
GQA_BLOCKS = 8


@pytest.fixture(scope="module")
def gqa_run():
    """Runs the 64-step decode once; keeps each step's queries, outputs and leaf
    sets, and the GPU tree before and after the step-32 append."""
    wl = synth.WORKLOADS["gqa128k"]
    T0, C = wl.T0, wl.C
    T_cap = T0 + GQA_STEPS + C
    K, V = synth.make_cache(wl.with_(steps=GQA_STEPS), DEV, T_cap)
    qref = synth.make_qref(wl, DEV)
    cfg = zha.Config(B=1, H_kv=wl.H_kv, G=wl.G, d=wl.d, C=C, L=wl.L, R=wl.R, T_cap=T_cap)
    dec = zha.Decoder(cfg, qref, DEV)
    Tt = torch.tensor([T0], dtype=torch.int64, device=DEV)
    dec.prefill(K, V, Tt)
    heads = list(range(cfg.H_kv))
    steps, trees, append_steps = [], {}, []
    for s in range(GQA_STEPS):
        T = T0 + s
        Tt.fill_(T)
        if T % C == 0:
            dec.append(K, V, Tt, 1)
            append_steps.append(s)
        q = synth.make_query(wl, s, T, DEV)
        out, lse = dec.step(q, K, V, Tt, wl.p)
        torch.cuda.synchronize()
        assert zha.ws_status(dec.ws) == 0, s
        assert dec.tree.n_built[:, 0].tolist() == [T // C ** l for l in range(1, cfg.L + 1)]
        sets = sets_from_lists(dec.leaves.ids, dec.leaves.mask, dec.leaves.count, cfg.G)
        steps.append(dict(T=T, q=q.clone(), out=out.clone(), lse=lse.clone(), sets=sets))
        n1 = T // C
        if n1 not in trees:
            trees[n1] = host_trees(dec.tree, cfg, T, heads)
    T_end = T0 + GQA_STEPS
    Kh = {h: f64(K[0, h, :T_end]) for h in heads}
    Vh = {h: f64(V[0, h, :T_end]) for h in heads}
    return dict(wl=wl, cfg=cfg, steps=steps, trees=trees, Kh=Kh, Vh=Vh, qref=f64(qref),
                append_steps=append_steps)


def test_gqa128k_append_fires_once_and_matches_the_oracle_leaf(gqa_run):
    r = gqa_run
    cfg, wl = r["cfg"], r["wl"]
    assert r["append_steps"] == [32]
    new_leaf = (wl.T0 + 32) // cfg.C - 1
    assert new_leaf == 2048
    T = wl.T0 + 32
    tr = r["trees"][T // cfg.C]
    for h in range(cfg.H_kv):
        Kc = r["Kh"][h][new_leaf * cfg.C:(new_leaf + 1) * cfg.C]
        for pl in range(cfg.R):
            kh, bh = O.leaf_summary(r["qref"][h, pl], Kc, cfg.scale)
            kg = tr[h][0]["khat"][new_leaf, pl]
            assert np.max(np.abs(kg - kh)) / np.max(np.abs(kh)) <= KHAT_TOL[1], (h, pl)
            assert abs(tr[h][0]["bhat"][new_leaf, pl] - bh) / max(1.0, abs(bh)) <= BHAT_TOL[1], (h, pl)
    # no level-3 node exists (n_3 = 0): the level-2 nodes are the roots and the
    # new leaf 2048 is a parentless level-1 node
    assert T // cfg.C ** 3 == 0 and (T // cfg.C) // cfg.C == 32


@pytest.mark.parametrize("block", range(GQA_BLOCKS))
def test_gqa128k_every_step_every_head(gqa_run, block):
    r = gqa_run
    cfg, wl = r["cfg"], r["wl"]
    heads = list(range(cfg.H_kv))
    per = GQA_STEPS // GQA_BLOCKS
    for s in range(block * per, (block + 1) * per):
        st = r["steps"][s]
        T = st["T"]
        trees_h = r["trees"][T // cfg.C]
        check_routing(cfg, trees_h, heads, st["q"], T, wl.p, st["sets"], ("gqa128k", s))
        check_outputs(cfg, r["Kh"], r["Vh"], st["q"], st["out"], st["lse"], st["sets"], heads, T,
                      TOL["bf16"], ("gqa128k", s))


# ---------------------------------------------------------------- long1m, spot steps

LONG_SPOT_STEPS = (0, 10, 21, 31)
LONG_HEADS = (0, 2, 5, 7)


@pytest.fixture(scope="module")
def long_run():
    wl = synth.WORKLOADS["long1m"]
    T0, C = wl.T0, wl.C
    T_cap = T0 + wl.steps + C
    K, V = synth.make_cache(wl, DEV, T_cap)
    qref = synth.make_qref(wl, DEV)
    cfg = zha.Config(B=1, H_kv=wl.H_kv, G=wl.G, d=wl.d, C=C, L=wl.L, R=wl.R, T_cap=T_cap)
    dec = zha.Decoder(cfg, qref, DEV)
    Tt = torch.tensor([T0], dtype=torch.int64, device=DEV)
    dec.prefill(K, V, Tt)
    steps = {}
    for s in range(wl.steps):
        T = T0 + s
        Tt.fill_(T)
        if T % C == 0:
            dec.append(K, V, Tt, 1)
        q = synth.make_query(wl, s, T, DEV)
        out, lse = dec.step(q, K, V, Tt, wl.p)
        if s in LONG_SPOT_STEPS:
            torch.cuda.synchronize()
            assert zha.ws_status(dec.ws) == 0, s
            sets = sets_from_lists(dec.leaves.ids, dec.leaves.mask, dec.leaves.count, cfg.G)
            steps[s] = dict(T=T, q=q.clone(), out=out.clone(), lse=lse.clone(), sets=sets)
    torch.cuda.synchronize()
    T_last = T0 + wl.steps - 1
    assert all(T0 // C == st["T"] // C for st in steps.values()), "the tree is fixed over the steps"
    return dict(wl=wl, cfg=cfg, steps=steps, dec=dec, K=K, V=V, T_last=T_last)


@pytest.mark.parametrize("step", LONG_SPOT_STEPS)
def test_long1m_spot_steps_on_four_kv_heads(long_run, step):
    r = long_run
    cfg, wl = r["cfg"], r["wl"]
    st = r["steps"][step]
    T = st["T"]
    for h in LONG_HEADS:
        trees_h = host_trees(r["dec"].tree, cfg, T, [h])
        check_routing(cfg, trees_h, [h], st["q"], T, wl.p, st["sets"], ("long1m", step))
        Kh = {h: f64(r["K"][0, h, :T])}
        Vh = {h: f64(r["V"][0, h, :T])}
        check_outputs(cfg, Kh, Vh, st["q"], st["out"], st["lse"], st["sets"], [h], T, TOL["bf16"],
                      ("long1m", step))
        del Kh, Vh, trees_h
