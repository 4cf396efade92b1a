"""GPU parity of dense_attend and zha_attend (split-K partials + (a, Z) merge)
against the oracle, through the C ABI."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from tests.gpu_util import TOL, f64, lists_from_sets, rel_err

pytestmark = pytest.mark.gpu

zha = pytest.importorskip("hierarchical_kv_cache_amd.zha")

DEV = "cuda"
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _cache(B, H_kv, T_cap, d, dtype, seed, T_fill):
    g = torch.Generator().manual_seed(seed)
    K = torch.randn(B, H_kv, T_cap, d, generator=g) * 1.5
    V = torch.randn(B, H_kv, T_cap, d, generator=g)
    K[:, :, T_fill:] = float("nan")  # never read: beyond every T
    V[:, :, T_fill:] = float("nan")
    return K.to(dtype).to(DEV), V.to(dtype).to(DEV)


def _dense_check(cfg, q, K, V, Tlist, out, lse, tol):
    Kh, Vh, qh = f64(K), f64(V), f64(q)
    worst = 0.0
    for b in range(cfg.B):
        T = Tlist[b]
        for j in range(cfg.Hq):
            h = j // cfg.G
            o_ref, l_ref = O.attention(qh[b, j], Kh[b, h, :T], Vh[b, h, :T], cfg.scale)
            if T == 0:
                assert np.all(out[b, j].cpu().numpy() == 0) and lse[b, j].item() == -math.inf
                continue
            e = rel_err(out[b, j].cpu().numpy(), o_ref)
            worst = max(worst, e)
            assert e <= tol, (b, j, T, e)
            assert abs(lse[b, j].item() - l_ref) <= max(tol, 1e-5) * max(1.0, abs(l_ref)), (b, j)
    return worst


def test_pin1_worked_example_through_dense_attend():
    """The attention page's three-token example (d_k = 2, zero-padded to 64, scale
    1/sqrt 2): decode of query i over keys 1..3 gives O row i; over keys 1..i the
    causal rows."""
    ex = json.load(open(os.path.join(GOLD, "three_token_example.json")))
    causal = json.load(open(os.path.join(GOLD, "causal_example.json")))
    for kvd, dt in ((zha.F32, torch.float32), (zha.BF16, torch.bfloat16)):
        cfg = zha.Config(B=1, H_kv=1, G=1, d=64, C=2, L=1, R=1, T_cap=4, kv_dtype=kvd,
                         scale=1 / math.sqrt(2))
        K = torch.zeros(1, 1, 4, 64)
        V = torch.zeros(1, 1, 4, 64)
        K[0, 0, :3, :2] = torch.tensor(ex["K"], dtype=torch.float32)
        V[0, 0, :3, :2] = torch.tensor(ex["V"], dtype=torch.float32)
        K, V = K.to(dt).to(DEV), V.to(dt).to(DEV)
        ws = zha.new_workspace(cfg)
        for i in range(3):
            q = torch.zeros(1, 1, 64, device=DEV)
            q[0, 0, :2] = torch.tensor(ex["Q"][i], dtype=torch.float32)
            out = torch.empty(1, 1, 64, device=DEV)
            lse = torch.empty(1, 1, device=DEV)
            for T, ref in ((3, ex["O"][i]), (i + 1, causal["O_causal"][i])):
                Tt = torch.tensor([T], dtype=torch.int64, device=DEV)
                zha.dense_attend(cfg, q, K, V, Tt, out, lse, ws)
                torch.cuda.synchronize()
                np.testing.assert_allclose(out[0, 0, :2].cpu().numpy(), ref, atol=5e-4)
                assert torch.all(out[0, 0, 2:] == 0)


@pytest.mark.parametrize("kvd,d,G,H_kv,B,C", [
    ("f32", 64, 1, 1, 1, 16),
    ("f32", 128, 4, 2, 2, 64),
    ("bf16", 128, 4, 2, 1, 64),
    ("bf16", 128, 8, 2, 2, 32),
    ("bf16", 64, 4, 3, 1, 4),
    ("bf16", 128, 16, 1, 1, 64),
    ("bf16", 64, 3, 2, 2, 16),
    ("f32", 128, 8, 1, 2, 4),
    ("f32", 64, 12, 2, 1, 64),
])
def test_dense_attend_matches_oracle(kvd, d, G, H_kv, B, C):
    dt = torch.float32 if kvd == "f32" else torch.bfloat16
    T_cap = 6000
    Tlist = [5003, 1][:B] if B == 2 else [4096 + 37]
    K, V = _cache(B, H_kv, T_cap, d, dt, seed=d + G + C, T_fill=max(Tlist))
    cfg = zha.Config(B=B, H_kv=H_kv, G=G, d=d, C=C, L=2, R=4, T_cap=T_cap,
                     kv_dtype=zha.F32 if kvd == "f32" else zha.BF16)
    q = torch.randn(B, cfg.Hq, d, generator=torch.Generator().manual_seed(7)).to(DEV)
    T = torch.tensor(Tlist, dtype=torch.int64, device=DEV)
    ws = zha.new_workspace(cfg)
    out = torch.empty(B, cfg.Hq, d, device=DEV)
    lse = torch.empty(B, cfg.Hq, device=DEV)
    zha.dense_attend(cfg, q, K, V, T, out, lse, ws)
    torch.cuda.synchronize()
    _dense_check(cfg, q, K, V, Tlist, out, lse, TOL[kvd])
    assert zha.ws_status(ws) == 0


def test_dense_edge_lengths():
    """T = 0 (no keys), T < C (only the open chunk), T multiple of 64 and of C."""
    d, C = 128, 64
    for Tv in (0, 1, 5, 63, 64, 65, 1024, 1024 + 63):
        cfg = zha.Config(B=1, H_kv=1, G=4, d=d, C=C, L=2, R=4, T_cap=2048)
        K, V = _cache(1, 1, 2048, d, torch.bfloat16, seed=Tv, T_fill=max(Tv, 1))
        q = torch.randn(1, 4, d).to(DEV)
        T = torch.tensor([Tv], dtype=torch.int64, device=DEV)
        ws = zha.new_workspace(cfg)
        out = torch.empty(1, 4, d, device=DEV)
        lse = torch.empty(1, 4, device=DEV)
        zha.dense_attend(cfg, q, K, V, T, out, lse, ws)
        torch.cuda.synchronize()
        _dense_check(cfg, q, K, V, [Tv], out, lse, TOL["bf16"])


def _random_sets(rng, n1, Hq, frac):
    sets = []
    for j in range(Hq):
        k = int(rng.integers(0, max(1, int(frac * n1)) + 1))
        sets.append(np.sort(rng.choice(n1, size=min(k, n1), replace=False)))
    return sets


@pytest.mark.parametrize("kvd,d,G,H_kv,B,C,frac", [
    ("f32", 64, 1, 1, 1, 16, 0.3),
    ("bf16", 128, 4, 2, 2, 64, 0.2),
    ("bf16", 128, 8, 1, 1, 32, 0.5),
    ("bf16", 64, 4, 2, 1, 4, 0.1),
    ("bf16", 128, 4, 1, 1, 64, 1.0),
    # group sizes that are not a power of two (padded heads must stay silent)
    ("bf16", 128, 3, 2, 1, 64, 0.4),
    ("bf16", 128, 6, 1, 2, 32, 0.4),
    ("bf16", 64, 12, 1, 1, 16, 0.3),
    # fp32 keys with eight and twelve query heads (the 8- and 16-head kernels),
    # at the smallest and largest chunks
    ("f32", 128, 8, 1, 1, 4, 0.2),
    ("f32", 128, 8, 2, 1, 64, 0.4),
    ("f32", 64, 12, 1, 2, 4, 0.3),
    ("f32", 128, 12, 1, 1, 64, 1.0),
])
def test_zha_attend_matches_oracle_on_key_set(kvd, d, G, H_kv, B, C, frac):
    """out_j = attention over {0} U keys(leaves with bit j) U [C n_1, T)."""
    dt = torch.float32 if kvd == "f32" else torch.bfloat16
    T_cap = 9000
    Tlist = [8000 + 13, 3 * C + 1][:B]
    K, V = _cache(B, H_kv, T_cap, d, dt, seed=11 + d + G, T_fill=max(Tlist))
    cfg = zha.Config(B=B, H_kv=H_kv, G=G, d=d, C=C, L=2, R=4, T_cap=T_cap,
                     kv_dtype=zha.F32 if kvd == "f32" else zha.BF16)
    rng = np.random.default_rng(5)
    sets = [_random_sets(rng, Tlist[b] // C, cfg.Hq, frac) for b in range(B)]
    if frac == 1.0:
        sets = [[np.arange(Tlist[b] // C)] * cfg.Hq for b in range(B)]
    ids, mask, count = lists_from_sets(sets, B, H_kv, G, cfg.leaf_cap)
    q = torch.randn(B, cfg.Hq, d, generator=torch.Generator().manual_seed(3)).to(DEV)
    T = torch.tensor(Tlist, dtype=torch.int64, device=DEV)
    ws = zha.new_workspace(cfg)
    out = torch.empty(B, cfg.Hq, d, device=DEV)
    lse = torch.empty(B, cfg.Hq, device=DEV)
    zha.attend(cfg, q, K, V, T, ids.to(DEV), mask.to(DEV), count.to(DEV), out, lse, ws)
    torch.cuda.synchronize()
    Kh, Vh, qh = f64(K), f64(V), f64(q)
    for b in range(B):
        for j in range(cfg.Hq):
            keys = O.routed_keys(sets[b][j], Tlist[b], C)
            o_ref, l_ref = O.attend_keys(qh[b, j], Kh[b, j // G], Vh[b, j // G], keys, cfg.scale)
            e = rel_err(out[b, j].cpu().numpy(), o_ref)
            assert e <= TOL[kvd], (b, j, e)
            assert abs(lse[b, j].item() - l_ref) <= 1e-4 * max(1.0, abs(l_ref))
    if frac == 1.0:
        # full list, every head: same split plan as dense -> bitwise equal
        out2 = torch.empty_like(out)
        lse2 = torch.empty_like(lse)
        zha.dense_attend(cfg, q, K, V, T, out2, lse2, ws)
        torch.cuda.synchronize()
        assert torch.equal(out, out2) and torch.equal(lse, lse2)
    # deterministic: a second run is bitwise identical
    out3 = torch.empty_like(out)
    lse3 = torch.empty_like(lse)
    zha.attend(cfg, q, K, V, T, ids.to(DEV), mask.to(DEV), count.to(DEV), out3, lse3, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out3) and torch.equal(lse, lse3)


def test_attend_folded_runs_across_groups():
    """More work items than workgroups: each workgroup folds a contiguous run of
    items into one state, and runs cross group boundaries.  Dense and routed
    attention at ~1000 items over 6 groups of different lengths, then a short
    call on the same workspace (the merge must read only this call's runs)."""
    B, H_kv, G, d, C = 2, 3, 4, 128, 64
    T_cap = 200_000
    Tlist = [196_613, 150_001]
    K, V = _cache(B, H_kv, T_cap, d, torch.bfloat16, seed=41, T_fill=max(Tlist))
    cfg = zha.Config(B=B, H_kv=H_kv, G=G, d=d, C=C, L=2, R=4, T_cap=T_cap, kv_dtype=zha.BF16)
    q = torch.randn(B, cfg.Hq, d, generator=torch.Generator().manual_seed(9)).to(DEV)
    T = torch.tensor(Tlist, dtype=torch.int64, device=DEV)
    ws = zha.new_workspace(cfg)
    out = torch.empty(B, cfg.Hq, d, device=DEV)
    lse = torch.empty(B, cfg.Hq, device=DEV)
    zha.dense_attend(cfg, q, K, V, T, out, lse, ws)
    torch.cuda.synchronize()
    _dense_check(cfg, q, K, V, Tlist, out, lse, TOL["bf16"])

    rng = np.random.default_rng(17)
    sets = [_random_sets(rng, Tlist[b] // C, cfg.Hq, 0.7) for b in range(B)]
    ids, mask, count = lists_from_sets(sets, B, H_kv, G, cfg.leaf_cap)
    zha.attend(cfg, q, K, V, T, ids.to(DEV), mask.to(DEV), count.to(DEV), out, lse, ws)
    torch.cuda.synchronize()
    Kh, Vh, qh = f64(K), f64(V), f64(q)
    for b in range(B):
        for j in range(cfg.Hq):
            keys = O.routed_keys(sets[b][j], Tlist[b], C)
            o_ref, l_ref = O.attend_keys(qh[b, j], Kh[b, j // G], Vh[b, j // G], keys, cfg.scale)
            assert rel_err(out[b, j].cpu().numpy(), o_ref) <= TOL["bf16"], (b, j)
            assert abs(lse[b, j].item() - l_ref) <= 1e-4 * max(1.0, abs(l_ref))

    short = [5000, 3]
    T.copy_(torch.tensor(short, dtype=torch.int64))
    zha.dense_attend(cfg, q, K, V, T, out, lse, ws)
    torch.cuda.synchronize()
    _dense_check(cfg, q, K, V, short, out, lse, TOL["bf16"])
    assert zha.ws_status(ws) == 0


@pytest.mark.parametrize("kvd,C,T,routed,B", [
    ("bf16", 64, 300_000, False, 1),   # dense: 512 workgroup runs in one group
    ("bf16", 4, 40_000, True, 1),      # gathered 4-key leaves: 157 items of 256 keys
    ("f32", 16, 140_000, True, 1),     # fp32 per-item kernel: 137 items of 1024 keys
    ("bf16", 4, 9_000, True, 64),      # 256 heads (the four-wave merge): 36 items each
])
def test_merge_of_many_partials_per_head(kvd, C, T, routed, B):
    """Heads holding more partials than the merge loads in one round (16 waves x
    8, or 4 waves x 8 when there are 256 heads or more): the merge first finds
    their maximum, then weights them.  Checked against the oracle's attention over
    every key (the full leaf list when routed)."""
    dt = torch.float32 if kvd == "f32" else torch.bfloat16
    d, G = 128, 4
    K, V = _cache(B, 1, T, d, dt, seed=C + 3, T_fill=T)
    cfg = zha.Config(B=B, H_kv=1, G=G, d=d, C=C, L=2, R=4, T_cap=T,
                     kv_dtype=zha.F32 if kvd == "f32" else zha.BF16)
    q = torch.randn(B, G, d, generator=torch.Generator().manual_seed(13)).to(DEV)
    Tt = torch.full((B,), T, dtype=torch.int64, device=DEV)
    ws = zha.new_workspace(cfg)
    out = torch.empty(B, G, d, device=DEV)
    lse = torch.empty(B, G, device=DEV)
    if routed:
        sets = [[np.arange(T // C)] * G for _ in range(B)]
        ids, mask, count = lists_from_sets(sets, B, 1, G, cfg.leaf_cap)
        zha.attend(cfg, q, K, V, Tt, ids.to(DEV), mask.to(DEV), count.to(DEV), out, lse, ws)
    else:
        zha.dense_attend(cfg, q, K, V, Tt, out, lse, ws)
    torch.cuda.synchronize()
    _dense_check(cfg, q, K, V, [T] * B, out, lse, TOL[kvd])
    assert zha.ws_status(ws) == 0


@pytest.mark.parametrize("Tlist", [[37, 0, 65, 1, 129, 64, 3, 200], [700, 5, 1300, 64, 2, 999, 64, 31]])
def test_attend_many_small_groups(Tlist):
    """8 sequences x 8 KV heads of short, unequal lengths (0, 1, exactly C, ...):
    workgroup ranges span many groups' tails, the range floor leaves few
    workgroups busy, and every group's partials are merged.  Dense and routed."""
    B, H_kv, G, d, C = 8, 8, 4, 128, 64
    T_cap = 1408
    K, V = _cache(B, H_kv, T_cap, d, torch.bfloat16, seed=5, T_fill=max(Tlist))
    cfg = zha.Config(B=B, H_kv=H_kv, G=G, d=d, C=C, L=2, R=4, T_cap=T_cap, kv_dtype=zha.BF16)
    q = torch.randn(B, cfg.Hq, d, generator=torch.Generator().manual_seed(21)).to(DEV)
    T = torch.tensor(Tlist, dtype=torch.int64, device=DEV)
    ws = zha.new_workspace(cfg)
    out = torch.empty(B, cfg.Hq, d, device=DEV)
    lse = torch.empty(B, cfg.Hq, device=DEV)
    zha.dense_attend(cfg, q, K, V, T, out, lse, ws)
    torch.cuda.synchronize()
    _dense_check(cfg, q, K, V, Tlist, out, lse, TOL["bf16"])
    rng = np.random.default_rng(3)
    sets = [_random_sets(rng, Tlist[b] // C, cfg.Hq, 0.6) for b in range(B)]
    ids, mask, count = lists_from_sets(sets, B, H_kv, G, cfg.leaf_cap)
    zha.attend(cfg, q, K, V, T, ids.to(DEV), mask.to(DEV), count.to(DEV), out, lse, ws)
    torch.cuda.synchronize()
    Kh, Vh, qh = f64(K), f64(V), f64(q)
    for b in range(B):
        for j in range(cfg.Hq):
            keys = O.routed_keys(sets[b][j], Tlist[b], C)
            if len(keys) == 0:
                assert np.all(out[b, j].cpu().numpy() == 0) and lse[b, j].item() == -math.inf
                continue
            o_ref, l_ref = O.attend_keys(qh[b, j], Kh[b, j // G], Vh[b, j // G], keys, cfg.scale)
            assert rel_err(out[b, j].cpu().numpy(), o_ref) <= TOL["bf16"], (b, j)
            assert abs(lse[b, j].item() - l_ref) <= 1e-4 * max(1.0, abs(l_ref))
    assert zha.ws_status(ws) == 0
