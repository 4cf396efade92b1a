"""Parity at the workloads' full sizes, in the configuration the bench times.

long1m: 8 KV heads x 4 query heads, d = 128, bf16 K/V, 1,048,608 cached tokens,
C = 64, L = 3, R = 16.  gqa128k: the same heads at 131,104 tokens.  deep: 4 KV
heads x 8 query heads, 262,146 tokens, C = 4, L = 6.  rope_batch: 16 sequences x
262,160 tokens, 4 KV heads x 8 query heads, RoPE base 1e6, C = 32, L = 3.  p = 0.9,
and long1m also at p = 0.75, the other top-p the bench times.

The oracle cannot afford every head, so a few (sequence, KV head) pairs are
sampled:
  * the GPU-built tree against the oracle's tree, at sampled nodes of every level;
  * the router on the oracle's own (fp32-rounded) tree of that head, level by
    level and end to end, against the oracle's routing;
  * the GPU's attention outputs of the sampled heads against the oracle's exact
    attention over the key sets the GPU routed.
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
NODES_PER_LEVEL = 512
# sampled (sequence, KV head) pairs per workload
SAMPLED = {
    "long1m": [(0, 0), (0, 5)],
    "gqa128k": [(0, 3)],
    "deep": [(0, 1)],
    "rope_batch": [(3, 2), (11, 0)],
}


@pytest.mark.parametrize("name,p", [("long1m", None), ("long1m", 0.75), ("gqa128k", None),
                                    ("deep", None), ("rope_batch", None)])
def test_full_size_build_route_attend_on_sampled_heads(name, p):
    wl = synth.WORKLOADS[name]
    T = wl.T0
    p = wl.p if p is None else p
    K, V = synth.make_cache(wl.with_(steps=0), DEV, T)
    qref = synth.make_qref(wl, DEV)
    cfg = zha.Config(B=wl.B, H_kv=wl.H_kv, G=wl.G, d=wl.d, C=wl.C, L=wl.L, R=wl.R, T_cap=T,
                     rope=wl.rope, rope_base=wl.rope_base)
    dec = zha.Decoder(cfg, qref, DEV)
    Tt = torch.full((wl.B,), T, dtype=torch.int64, device=DEV)
    dec.prefill(K, V, Tt)
    q = synth.make_query(wl, 0, T, DEV)
    out, lse = dec.step(q, K, V, Tt, p)
    torch.cuda.synchronize()
    assert zha.ws_status(dec.ws) == 0
    gpu_sets = sets_from_lists(dec.leaves.ids, dec.leaves.mask, dec.leaves.count, cfg.G)
    rope_base = wl.rope_base if wl.rope else None
    rng = np.random.default_rng(11)
    for b, h in SAMPLED[name]:
        Kh = f64(K[b, h, :T])
        Vh = f64(V[b, h, :T])
        qh = f64(q[b])
        ref = O.build_tree(Kh, f64(qref[h]), T, cfg.C, cfg.L, cfg.scale, rope_base)

        # build: sampled nodes of every level
        for level in range(1, cfg.L + 1):
            n = T // cfg.C ** level
            if n == 0:
                continue
            nodes = np.unique(rng.integers(0, n, size=min(n, NODES_PER_LEVEL)))
            idx = torch.tensor(nodes, device=DEV)
            kg = f64(tree_slice(dec.tree.khat[level - 1], b, h, idx))
            bg = f64(tree_slice(dec.tree.bhat[level - 1], b, h, idx))
            kr, br = ref[level - 1]["khat"][nodes], ref[level - 1]["bhat"][nodes]
            ek = np.max(np.abs(kg - kr)) / np.max(np.abs(ref[level - 1]["khat"]))
            eb = np.max(np.abs(bg - br) / np.maximum(1.0, np.abs(br)))
            assert ek <= KHAT_TOL[level], (name, b, h, level, ek)
            assert eb <= BHAT_TOL[level], (name, b, h, level, eb)

        # route: the oracle's tree of this head on the GPU, one KV head
        cfg1 = zha.Config(B=1, H_kv=1, G=cfg.G, d=cfg.d, C=cfg.C, L=cfg.L, R=cfg.R, T_cap=T)
        trees = [[[{"khat": O.fp32(lv["khat"]), "bhat": O.fp32(lv["bhat"])} for lv in ref]]]
        tree1 = upload(cfg1, trees, T)
        ws1 = zha.new_workspace(cfg1)
        q1 = q[b:b + 1, h * cfg.G:(h + 1) * cfg.G].contiguous()
        T1 = torch.tensor([T], dtype=torch.int64, device=DEV)
        report = []
        leaves = level_sync_compare(cfg1, tree1, trees, q1, T, p, ws1, report)
        lst = zha.LeafList(cfg1, DEV)
        zha.route(cfg1, q1, tree1, T1, p, lst.ids, lst.mask, lst.count, ws1)
        torch.cuda.synchronize()
        full = sets_from_lists(lst.ids, lst.mask, lst.count, cfg1.G)
        for g in range(cfg.G):
            np.testing.assert_array_equal(full[0][g], leaves[0][g])
        assert zha.ws_status(ws1) == 0
        for r in report:
            print("allowed:", name, b, h, r)
        del tree1, ws1, lst

        # attend: the GPU outputs over the sets the GPU routed
        for g in range(cfg.G):
            j = h * cfg.G + g
            keys = O.routed_keys(gpu_sets[b][j], T, cfg.C)
            o_ref, lse_ref = O.attend_keys(qh[j], Kh, Vh, keys, cfg.scale)
            e = rel_err(f64(out[b, j]), o_ref)
            assert e <= TOL["bf16"], (name, b, h, g, e)
            assert abs(float(lse[b, j]) - lse_ref) <= 1e-3 * max(1.0, abs(lse_ref)), (name, b, h, g)
        del Kh, Vh, ref


def tree_slice(level_tensor, b, h, idx):
    """Rows idx of KV head h of sequence b of one tree level."""
    return level_tensor[b, h].index_select(0, idx)


@pytest.mark.parametrize("name", ["long1m", "rope_batch"])
def test_full_size_bf16_copy(name):
    """The tree's bf16 copy of k_hat at full size: after the prefill every level's
    copy is the fp32 tree rounded to bf16 (nearest even) bit for bit; the router
    scoring from a copy of the oracle's tree matches the oracle routing on the
    same rounded values, level by level and end to end, on sampled heads; and the
    decode step routed from the GPU's own copy attends within tolerance of the
    oracle over the sets it routed."""
    from tests.test_gpu_route import bf16_trees, upload_bf16
    wl = synth.WORKLOADS[name]
    T, p = wl.T0, wl.p
    K, V = synth.make_cache(wl.with_(steps=0), DEV, T)
    qref = synth.make_qref(wl, DEV)
    cfg = zha.Config(B=wl.B, H_kv=wl.H_kv, G=wl.G, d=wl.d, C=wl.C, L=wl.L, R=wl.R, T_cap=T,
                     rope=wl.rope, rope_base=wl.rope_base)
    dec = zha.Decoder(cfg, qref, DEV, bf16_copy=True)
    Tt = torch.full((wl.B,), T, dtype=torch.int64, device=DEV)
    dec.prefill(K, V, Tt)
    torch.cuda.synchronize()
    for level in range(cfg.L):
        assert torch.equal(dec.tree.khat16[level].view(torch.int16),
                           dec.tree.khat[level].to(torch.bfloat16).view(torch.int16)), level
    q = synth.make_query(wl, 1, T, DEV)
    out, lse = dec.step(q, K, V, Tt, p)
    torch.cuda.synchronize()
    assert zha.ws_status(dec.ws) == 0
    gpu_sets = sets_from_lists(dec.leaves.ids, dec.leaves.mask, dec.leaves.count, cfg.G)
    rope_base = wl.rope_base if wl.rope else None
    b, h = SAMPLED[name][0]
    Kh, Vh, qh = f64(K[b, h, :T]), f64(V[b, h, :T]), f64(q[b])
    ref = O.build_tree(Kh, f64(qref[h]), T, cfg.C, cfg.L, cfg.scale, rope_base)
    cfg1 = zha.Config(B=1, H_kv=1, G=cfg.G, d=cfg.d, C=cfg.C, L=cfg.L, R=cfg.R, T_cap=T)
    trees16 = bf16_trees([[[{"khat": O.fp32(lv["khat"]), "bhat": O.fp32(lv["bhat"])} for lv in ref]]])
    tree1 = upload_bf16(cfg1, trees16, T)
    for k in tree1.khat:
        k.fill_(float("nan"))          # only the copy may be read
    ws1 = zha.new_workspace(cfg1)
    q1 = q[b:b + 1, h * cfg.G:(h + 1) * cfg.G].contiguous()
    report = []
    leaves = level_sync_compare(cfg1, tree1, trees16, q1, T, p, ws1, report)
    lst = zha.LeafList(cfg1, DEV)
    zha.route(cfg1, q1, tree1, torch.tensor([T], dtype=torch.int64, device=DEV), p,
              lst.ids, lst.mask, lst.count, ws1)
    torch.cuda.synchronize()
    full = sets_from_lists(lst.ids, lst.mask, lst.count, cfg1.G)
    for g in range(cfg.G):
        np.testing.assert_array_equal(full[0][g], leaves[0][g])
    assert zha.ws_status(ws1) == 0
    for r in report:
        print("allowed:", name, b, h, r)
    for g in range(cfg.G):
        j = h * cfg.G + g
        keys = O.routed_keys(gpu_sets[b][j], T, cfg.C)
        o_ref, lse_ref = O.attend_keys(qh[j], Kh, Vh, keys, cfg.scale)
        assert rel_err(f64(out[b, j]), o_ref) <= TOL["bf16"], (name, g)
        assert abs(float(lse[b, j]) - lse_ref) <= 1e-3 * max(1.0, abs(lse_ref)), (name, g)
