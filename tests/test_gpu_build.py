"""GPU parity of the tree builders (zha_build_level, zha_append) against the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.gpu_util import f64

pytestmark = pytest.mark.gpu
zha = pytest.importorskip("hierarchical_kv_cache_amd.zha")
DEV = "cuda"

# Bounds of the builder's fp32 rounding: |k_hat - ref| / max |ref| over a level,
# and |b_hat - ref| / max(1, |ref|).  A node's k_hat is a softmax-weighted mean
# (a convex combination) of its keys or of its children's k_hat, so the error it
# inherits from the level below does not grow, and each level adds one more
# rounding of a C-term weighted sum (about sqrt(C) 2^-24 typically, C 2^-24 at
# worst) plus the weights' rounding.  Measured worst errors over C = 2..64,
# L up to 8, fp32 and bf16 keys, with and without RoPE: k_hat 4.3e-7, b_hat
# 2.6e-7, with no growth from level 1 to level 8.  The bounds allow about five
# times that, and a slow linear growth with the level.
KHAT_TOL = {l: 2e-6 + 2e-7 * (l - 1) for l in range(1, 9)}
BHAT_TOL = {l: 1e-6 + 2e-7 * (l - 1) for l in range(1, 9)}


def _workload(name, **kw):
    return synth.WORKLOADS[name].with_(**kw)


def _build_gpu(wl, T, T_cap=None):
    T_cap = T_cap or T
    K, V = synth.make_cache(wl.with_(N=T, open_len=0, steps=0), DEV, T_cap)
    qref = synth.make_qref(wl, DEV)
    cfg = zha.Config(B=wl.B, H_kv=wl.H_kv, G=wl.G, d=wl.d, C=wl.C, L=wl.L, R=wl.R,
                     T_cap=T_cap, kv_dtype=zha.F32 if wl.kv_dtype == "f32" else zha.BF16,
                     rope=wl.rope, rope_base=wl.rope_base)
    tree = zha.Tree(cfg, DEV)
    ws = zha.new_workspace(cfg)
    Tt = torch.full((wl.B,), T, dtype=torch.int64, device=DEV)
    zha.build(cfg, K, V, Tt, qref, tree, ws)
    torch.cuda.synchronize()
    return cfg, K, V, qref, tree, ws, Tt


def _compare_tree(cfg, K, qref, tree, T, rope_base, b=0, h=0):
    ref = O.build_tree(f64(K[b, h, :T]), f64(qref[h]), T, cfg.C, cfg.L, cfg.scale, rope_base)
    assert tree.n_built[:, b].tolist() == [T // cfg.C ** l for l in range(1, cfg.L + 1)]
    worst = {}
    for level in range(1, cfg.L + 1):
        n = T // cfg.C ** level
        if n == 0:
            continue
        kg = f64(tree.khat[level - 1][b, h, :n])
        bg = f64(tree.bhat[level - 1][b, h, :n])
        kr, br = ref[level - 1]["khat"], ref[level - 1]["bhat"]
        scale_k = np.max(np.abs(kr))
        ek = np.max(np.abs(kg - kr)) / scale_k
        eb = np.max(np.abs(bg - br) / np.maximum(1.0, np.abs(br)))
        worst[level] = (ek, eb)
        assert ek <= KHAT_TOL[level], (level, ek)
        assert eb <= BHAT_TOL[level], (level, eb)
    return worst


def test_build_tiny_fp32_nope():
    wl = _workload("tiny")
    cfg, K, V, qref, tree, ws, Tt = _build_gpu(wl, 4096)
    _compare_tree(cfg, K, qref, tree, 4096, None)


@pytest.mark.parametrize("C,L,T,G", [(16, 3, 10000, 4), (64, 2, 9000 + 17, 4), (4, 4, 1500, 8),
                                     (2, 8, 2 ** 8 * 3 + 37, 4)])
def test_build_bf16_nope_levels(C, L, T, G):
    wl = _workload("gqa128k", H_kv=2, G=G, C=C, L=L, n_clusters=64)
    cfg, K, V, qref, tree, ws, Tt = _build_gpu(wl, T)
    for h in range(2):
        _compare_tree(cfg, K, qref, tree, T, None, h=h)


@pytest.mark.parametrize("C,rope", [(32, False), (16, True), (64, False)])
def test_build_bf16_d64(C, rope):
    """Head dimension 64 on the matrix-core leaf builder, with and without RoPE."""
    wl = _workload("rope_batch" if rope else "gqa128k", B=1, H_kv=2, G=4, d=64, C=C, L=2,
                   n_clusters=64)
    T = C * C * 3 + C * 5 + 7
    cfg, K, V, qref, tree, ws, Tt = _build_gpu(wl, T)
    for h in range(2):
        _compare_tree(cfg, K, qref, tree, T, wl.rope_base if rope else None, h=h)


@pytest.mark.parametrize("C,d,rope,R", [(2, 128, False, 16), (4, 128, True, 16), (8, 128, False, 12),
                                         (8, 64, True, 16), (4, 64, False, 12)])
def test_build_bf16_small_chunks(C, d, rope, R):
    """C in {2, 4, 8}: the one-wave-per-leaf builder (lanes over dimensions) and
    parents of one or two child rounds, with and without RoPE, d = 64 and 128,
    and R < 16 (padded planes)."""
    wl = _workload("rope_batch" if rope else "gqa128k", B=1, H_kv=2, G=4, d=d, C=C, L=3, R=R,
                   n_clusters=64)
    T = C ** 3 * 5 + C * 3 + 1
    cfg, K, V, qref, tree, ws, Tt = _build_gpu(wl, T)
    for h in range(2):
        _compare_tree(cfg, K, qref, tree, T, wl.rope_base if rope else None, h=h)


def test_build_rope_parent_correction():
    """RoPE: reference queries rotated to each node's first key position; parents
    rescore children at their own rotated query (the correction term)."""
    wl = _workload("rope_batch", B=2, H_kv=1, G=2, C=32, L=3, n_clusters=64)
    T = 32 ** 3 * 2 + 100
    cfg, K, V, qref, tree, ws, Tt = _build_gpu(wl, T)
    for b in range(2):
        _compare_tree(cfg, K, qref, tree, T, wl.rope_base, b=b)


@pytest.mark.parametrize("C,L,kv,rope,R", [(8, 3, "bf16", False, 16), (16, 2, "bf16", False, 16),
                                           (4, 4, "bf16", False, 16), (64, 2, "bf16", False, 16),
                                           (16, 2, "f32", False, 16), (4, 3, "f32", False, 16),
                                           (4, 3, "bf16", True, 16), (32, 2, "bf16", True, 16),
                                           (2, 5, "bf16", False, 16), (8, 2, "bf16", False, 12),
                                           (2, 3, "bf16", True, 5)])
def test_append_cascade_equals_prefill_build(C, L, kv, rope, R):
    """Growing T one token at a time with zha_append yields exactly the tree a
    prefill build of the final length gives (the append cadence).  One token at a
    time takes the one-launch cascade (one workgroup per sequence); a jump of more
    than C tokens takes the per-level launches.  C = 16..64 bf16 leaves use the
    matrix-core builder; at C <= 8 the prefill builds a leaf per wave and the
    one-launch append a plane per wave (R < 16 included), which must agree bit
    for bit; fp32 keys use the workgroup-per-leaf builder.  Under RoPE the matrix-core prefill advances each
    wave's rotation angle from leaf to leaf while an append rotates from the
    leaf's own position, so there the two agree to the builder's accuracy, not
    bit for bit."""
    wl = _workload("rope_batch" if rope else "gqa128k", B=1, H_kv=2, G=4, C=C, L=L, R=R,
                   n_clusters=16, kv_dtype=kv)
    T0, T1 = C ** L - 37 if C ** L > 40 else C ** L - 3, C ** L * 2 + 70
    T_cap = T1 + C
    K, V = synth.make_cache(wl.with_(N=T1, open_len=0, steps=0), DEV, T_cap)
    qref = synth.make_qref(wl, DEV)
    cfg = zha.Config(B=1, H_kv=2, G=4, d=128, C=C, L=L, R=R, T_cap=T_cap,
                     kv_dtype=zha.F32 if kv == "f32" else zha.BF16, rope=rope, rope_base=wl.rope_base)
    tree = zha.Tree(cfg, DEV)
    ws = zha.new_workspace(cfg)
    T = torch.tensor([T0], dtype=torch.int64, device=DEV)
    zha.build(cfg, K, V, T, qref, tree, ws)
    for t in range(T0 + 1, T1 + 1):
        T.fill_(t)
        zha.append(cfg, K, V, T, qref, tree, ws, max_new_tokens=1)
    # one multi-token append on each path: any growth is built
    trees = []
    for m in (C, C + 1):
        t2 = zha.Tree(cfg, DEV)
        T.fill_(T0)
        zha.build(cfg, K, V, T, qref, t2, ws)
        T.fill_(T1)
        zha.append(cfg, K, V, T, qref, t2, ws, max_new_tokens=m)
        trees.append(t2)
    ref = zha.Tree(cfg, DEV)
    zha.build(cfg, K, V, T, qref, ref, ws)
    torch.cuda.synchronize()
    exact = not (rope and C >= 16)
    for level in range(1, L + 1):
        n = T1 // C ** level
        for t in [tree] + trees:
            kg, bg = t.khat[level - 1][:, :, :n], t.bhat[level - 1][:, :, :n]
            kr, br = ref.khat[level - 1][:, :, :n], ref.bhat[level - 1][:, :, :n]
            if exact:
                assert torch.equal(kg, kr), level
                assert torch.equal(bg, br), level
            else:
                ek = float((kg - kr).abs().max() / kr.abs().max())
                eb = float(((bg - br).abs() / br.abs().clamp_min(1.0)).max())
                assert ek <= KHAT_TOL[level] and eb <= BHAT_TOL[level], (level, ek, eb)
    for t in [tree] + trees:
        assert t.n_built[:, 0].tolist() == [T1 // C ** l for l in range(1, L + 1)]
    assert zha.ws_status(ws) == 0


@pytest.mark.parametrize("C,L", [(8, 3), (16, 2)])
def test_append_ragged_batch_equals_prefill_build(C, L):
    """Batched decode over sequences of different lengths: every sequence grows by
    one token per step, so each completes its chunks (and parents) at its own
    steps; one append per step must leave the tree a prefill build of the final
    lengths gives.  One sequence starts with two tokens (no nodes yet)."""
    wl = _workload("gqa128k", B=3, H_kv=2, G=4, C=C, L=L, n_clusters=16)
    T0 = [C ** L - 5, 5 * C - 1, 2]
    steps = 2 * C + 3
    T_cap = max(T0) + steps
    K, V = synth.make_cache(wl.with_(N=T_cap, open_len=0, steps=0), DEV, T_cap)
    qref = synth.make_qref(wl, DEV)
    cfg = zha.Config(B=3, H_kv=2, G=4, d=128, C=C, L=L, R=16, T_cap=T_cap)
    tree = zha.Tree(cfg, DEV)
    ws = zha.new_workspace(cfg)
    T = torch.tensor(T0, dtype=torch.int64, device=DEV)
    zha.build(cfg, K, V, T, qref, tree, ws)
    for _ in range(steps):
        T += 1
        zha.append(cfg, K, V, T, qref, tree, ws, max_new_tokens=1)
    ref = zha.Tree(cfg, DEV)
    zha.build(cfg, K, V, T, qref, ref, ws)
    torch.cuda.synchronize()
    T1 = [t + steps for t in T0]
    for b in range(3):
        assert tree.n_built[:, b].tolist() == [T1[b] // C ** l for l in range(1, L + 1)]
        for level in range(1, L + 1):
            n = T1[b] // C ** level
            assert torch.equal(tree.khat[level - 1][b, :, :n], ref.khat[level - 1][b, :, :n]), (b, level)
            assert torch.equal(tree.bhat[level - 1][b, :, :n], ref.bhat[level - 1][b, :, :n]), (b, level)
    for b in range(3):
        _compare_tree(cfg, K, qref, tree, T1[b], None, b=b, h=1)
    assert zha.ws_status(ws) == 0


def test_build_is_deterministic():
    wl = _workload("gqa128k", H_kv=1, G=4, C=64, L=2, n_clusters=8)
    cfg, K, V, qref, tree, ws, Tt = _build_gpu(wl, 8192)
    tree2 = zha.Tree(cfg, DEV)
    zha.build(cfg, K, V, Tt, qref, tree2, ws)
    torch.cuda.synchronize()
    for a, b in zip(tree.khat + tree.bhat, tree2.khat + tree2.bhat):
        assert torch.equal(a, b)


@pytest.mark.parametrize("C,L,kv,rope", [(64, 2, "bf16", False), (32, 2, "bf16", True), (16, 3, "bf16", False),
                                         (8, 3, "bf16", False), (4, 3, "bf16", True), (2, 4, "bf16", False),
                                         (16, 2, "f32", False), (4, 3, "f32", False)])
def test_bf16_copy_is_the_rounded_khat(C, L, kv, rope):
    """zha_tree.khat16: every builder kernel (matrix-core, small-C and generic
    leaves, parents), the one-launch append cascade and the per-level append
    write, beside each k_hat value, that value rounded to bf16 (nearest even):
    the copy equals torch's rounding of the fp32 tree bit for bit."""
    wl = _workload("rope_batch" if rope else "gqa128k", B=2, H_kv=2, G=4, C=C, L=L, R=16,
                   n_clusters=16, kv_dtype=kv)
    T0 = C ** L + 3
    T1 = T0 + 2 * C + 5
    T_cap = T1 + 2 * C
    K, V = synth.make_cache(wl.with_(N=T_cap, open_len=0, steps=0), DEV, T_cap)
    qref = synth.make_qref(wl, DEV)
    cfg = zha.Config(B=2, H_kv=2, G=4, d=128, C=C, L=L, R=16, T_cap=T_cap,
                     kv_dtype=zha.F32 if kv == "f32" else zha.BF16, rope=rope, rope_base=wl.rope_base)
    ws = zha.new_workspace(cfg)

    def same(tree, where):
        torch.cuda.synchronize()
        for level in range(1, L + 1):
            assert torch.equal(tree.khat16[level - 1].view(torch.int16),
                               tree.khat[level - 1].to(torch.bfloat16).view(torch.int16)), (where, level)
        assert bool(torch.isfinite(tree.khat[0][:, :, :T1 // C]).all())

    tree = zha.Tree(cfg, DEV, bf16_copy=True)
    T = torch.tensor([T0, T0 - C + 1], dtype=torch.int64, device=DEV)
    zha.build(cfg, K, V, T, qref, tree, ws)
    same(tree, "prefill")
    for _ in range(T1 - T0):                     # one token per step: one-launch cascade
        T += 1
        zha.append(cfg, K, V, T, qref, tree, ws, max_new_tokens=1)
    same(tree, "append")
    T += C + 1                                   # more than C at once: per-level launches
    zha.append(cfg, K, V, T, qref, tree, ws, max_new_tokens=C + 1)
    same(tree, "append per level")
    assert zha.ws_status(ws) == 0
