"""A decode step (zha_route + zha_attend) captured once in a HIP graph and replayed.

Both calls are asynchronous on the caller's stream, with no host
synchronisation and no memory-set or copy nodes, so a caller can capture a
step.  The graph is replayed for several queries, with eager work and
synchronisations between the replays, and every replay must give the eager
step's outputs bit for bit: the same kernels on the same inputs, with fixed
reduction orders.  The same holds with the route scoring from the tree's bf16
copy of k_hat.
"""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
zha = pytest.importorskip("hierarchical_kv_cache_amd.zha")
DEV = "cuda"


@pytest.mark.parametrize("bf16_copy", [False, True])
def test_decode_step_in_a_graph_matches_eager(bf16_copy):
    wl = synth.WORKLOADS["gqa128k"].with_(H_kv=2, G=4, C=16, L=3, n_clusters=128)
    T = 20000 + 7
    K, V = synth.make_cache(wl.with_(N=T, open_len=0, steps=0), DEV, T)
    qref = synth.make_qref(wl, DEV)
    cfg = zha.Config(B=1, H_kv=2, G=4, d=128, C=16, L=3, R=16, T_cap=T)
    dec = zha.Decoder(cfg, qref, DEV, bf16_copy=bf16_copy)
    Tt = torch.tensor([T], dtype=torch.int64, device=DEV)
    dec.prefill(K, V, Tt)
    q_static = synth.make_query(wl, 0, T, DEV).clone()

    # one eager step on a side stream before capture, then capture one step
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dec.step(q_static, K, V, Tt, 0.9)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out_g, lse_g = dec.step(q_static, K, V, Tt, 0.9)
    torch.cuda.synchronize()

    for step in range(1, 5):
        q = synth.make_query(wl, step, T, DEV)
        q_static.copy_(q)
        graph.replay()
        torch.cuda.synchronize()
        o_rep, l_rep = out_g.clone(), lse_g.clone()
        out_e, lse_e = dec.step(q, K, V, Tt, 0.9)   # eager, into the same buffers
        torch.cuda.synchronize()
        assert torch.equal(o_rep, out_e), step
        assert torch.equal(l_rep, lse_e), step
        assert torch.isfinite(o_rep).all()
    assert zha.ws_status(dec.ws) == 0
