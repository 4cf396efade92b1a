"""A batch whose sequences hold different numbers of tokens, through the whole path.

Four sequences of 20,007, 9,000, 15 and 0 tokens share one cache of capacity
20,007: 2 KV heads x 4 query heads, d = 128, bf16 K/V, C = 16, L = 3, R = 16.
The third is shorter than one chunk, so it has no nodes at any level and its key
set is the sink plus the open chunk, all of its keys.  The fourth is empty: no
keys, a zero output and lse = -inf.  Every level's node count follows each
sequence's own length ([ZHA] "무엇과 다른가": one tree per KV head, its nodes
completed as the cache grows).

Checked against the oracle: the tree the GPU builds for every (sequence, KV
head); the router level by level and end to end on the oracle's fp32 trees,
each sequence at its own length; and attention over the sets the GPU routes on
its own tree.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.gpu_util import TOL, f64, rel_err, sets_from_lists
from tests.test_gpu_build import _compare_tree
from tests.test_gpu_route import level_sync_compare, oracle_tree32, upload

pytestmark = pytest.mark.gpu
zha = pytest.importorskip("hierarchical_kv_cache_amd.zha")
DEV = "cuda"
TLIST = [20007, 9000, 15, 0]


@pytest.mark.parametrize("p", [0.5, 0.9])
def test_ragged_batch_build_route_attend(p):
    wl = synth.WORKLOADS["gqa128k"].with_(B=len(TLIST), H_kv=2, G=4, C=16, L=3, n_clusters=128)
    T_cap = max(TLIST)
    K, V = synth.make_cache(wl.with_(N=T_cap, open_len=0, steps=0), "cpu", T_cap)
    qref = synth.make_qref(wl, "cpu")
    cfg = zha.Config(B=wl.B, H_kv=wl.H_kv, G=wl.G, d=wl.d, C=wl.C, L=wl.L, R=wl.R, T_cap=T_cap,
                     kv_dtype=zha.BF16)
    Kd, Vd = K.to(DEV), V.to(DEV)
    Tt = torch.tensor(TLIST, dtype=torch.int64, device=DEV)

    # the GPU's own tree, every sequence at its own length
    dec = zha.Decoder(cfg, qref.to(DEV), DEV)
    dec.prefill(Kd, Vd, Tt)
    torch.cuda.synchronize()
    for b, Tb in enumerate(TLIST):
        for h in range(cfg.H_kv):
            _compare_tree(cfg, K, qref, dec.tree, Tb, None, b=b, h=h)

    # the router on the oracle's trees
    trees = oracle_tree32(wl, TLIST, K)
    tree = upload(cfg, trees, TLIST)
    ws = zha.new_workspace(cfg)
    report = []
    for step in range(2):
        q = synth.make_query(wl, step, T_cap, "cpu").to(DEV)
        leaves = level_sync_compare(cfg, tree, trees, q, TLIST, p, ws, report)
        lst = zha.LeafList(cfg, DEV)
        zha.route(cfg, q, tree, Tt, p, lst.ids, lst.mask, lst.count, ws)
        torch.cuda.synchronize()
        full = sets_from_lists(lst.ids, lst.mask, lst.count, cfg.G)
        for b in range(cfg.B):
            for j in range(cfg.Hq):
                np.testing.assert_array_equal(full[b][j], leaves[b][j])
        for b in (2, 3):   # no leaves below one chunk
            assert all(len(full[b][j]) == 0 for j in range(cfg.Hq))
        assert zha.ws_status(ws) == 0
    for r in report:
        print("allowed:", p, r)

    # attention over the sets the GPU routes on its own tree
    q = synth.make_query(wl, 5, T_cap, "cpu").to(DEV)
    out, lse = dec.step(q, Kd, Vd, Tt, p)
    torch.cuda.synchronize()
    assert zha.ws_status(dec.ws) == 0
    sets = sets_from_lists(dec.leaves.ids, dec.leaves.mask, dec.leaves.count, cfg.G)
    qh = f64(q)
    for b, Tb in enumerate(TLIST):
        for h in range(cfg.H_kv):
            Kh, Vh = f64(K[b, h, :Tb]), f64(V[b, h, :Tb])
            for g in range(cfg.G):
                j = h * cfg.G + g
                if Tb == 0:
                    assert torch.all(out[b, j] == 0) and float(lse[b, j]) == -math.inf, (p, b, j)
                    continue
                keys = O.routed_keys(sets[b][j], Tb, cfg.C)
                if Tb < cfg.C:
                    assert list(keys) == list(range(Tb))
                o_ref, lse_ref = O.attend_keys(qh[b, j], Kh, Vh, keys, cfg.scale)
                assert rel_err(f64(out[b, j]), o_ref) <= TOL["bf16"], (p, b, j)
                assert abs(float(lse[b, j]) - lse_ref) <= 1e-3 * max(1.0, abs(lse_ref)), (p, b, j)
