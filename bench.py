#!/usr/bin/env python3
"""Decode-step benchmark of tree-summarised (ZHA) attention on one MI355X.

A step is one pass of the hot path for every query head of the batch: the
caller advances T (the new token's key/value are already in the cache), the tree
grows when a chunk completes (zha_append, every C steps), the queries are routed
down the tree (zha_route) and attend over the routed keys (zha_attend).  Inputs
are synthetic and resident in HBM before timing starts.  The same steps are then
timed with the dense split-K baseline (dense_attend) over every key.

Prints one JSON line.  ``--gpus`` above 1 is refused: the path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBPS = 8000.0
METRIC = "routed decode-attn µs/step at 1M ctx; effective KV GB/s vs HBM peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="long1m", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--p", type=float, default=None, help="top-p (default: the workload's)")
    ap.add_argument("--p-sweep", default="0.75", help="extra p values timed (comma list, '' for none)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense baseline")
    ap.add_argument("--no-stats", action="store_true", help="skip the byte-accounting replay")
    ap.add_argument("--schedules", default="",
                    help="depth schedules of p also measured (comma list of uniform,root,power)")
    ap.add_argument("--gamma", type=float, default=1.5, help="exponent of the power schedule")
    ap.add_argument("--flat", action="store_true",
                    help="also measure flat (one-level) top-p and top-K routing over all leaves")
    ap.add_argument("--n-sweep", default="17,18,19",
                    help="log2 context lengths also timed routed vs dense (comma list, '' for none)")
    ap.add_argument("--no-append-cadence", action="store_true",
                    help="skip the in-loop append measurement (profiler runs: its extra route and "
                         "attend calls would dilute the per-dispatch figures); the window's own "
                         "appends then stay in value as they fell")
    ap.add_argument("--no-bf16-copy", action="store_true",
                    help="skip the measurement of routing from bf16 copies of the summaries")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (known bytes) for counter calibration")
    return ap.parse_args()


def copy_calibration():
    """A plain copy of known size: 1 GiB read + 1 GiB written per launch, 8 launches.
    Its FETCH_SIZE / WRITE_SIZE readings calibrate the counters for other kernels."""
    n = 1 << 30
    src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(8):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": n, "copy_bytes_written_per_launch": n,
                      "launches": 8}))


ATTEND_SOURCES = ["hierarchical_kv_cache_amd/csrc/attend.hip", "hierarchical_kv_cache_amd/csrc/zha_internal.hpp"]


def attend_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in ATTEND_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic_ratio(workload, p):
    """HBM bytes over algorithmic bytes of zha_attend, from committed counter runs
    (FETCH_SIZE + WRITE_SIZE, calibrated on a plain copy), if they were taken on
    the current attend kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"attend_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != attend_source_hash() or abs(rec.get("p", -1) - p) > 1e-9:
        return None
    return rec["hbm_bytes_per_call"] / rec["algorithmic_bytes_per_call"]


class Run:
    """Device state of one workload: cache, queries, per-step lengths, tree, buffers."""

    def __init__(self, wl, steps_total, dev="cuda"):
        from hierarchical_kv_cache_amd import zha
        self.zha = zha
        self.wl = wl
        self.T_cap = wl.T0 + steps_total + wl.C
        t0 = time.time()
        self.K, self.V = synth.make_cache(wl.with_(steps=steps_total + wl.C), dev, self.T_cap)
        self.qref = synth.make_qref(wl, dev)
        self.Q = torch.stack([synth.make_query(wl, s, wl.T0 + s, dev) for s in range(steps_total)])
        # length of every sequence at step s (the token of step s is already cached)
        self.Ts = (wl.T0 + torch.arange(steps_total, dtype=torch.int64, device=dev)).unsqueeze(1) \
            .repeat(1, wl.B).contiguous()
        torch.cuda.synchronize()
        log(f"[bench] synthetic cache {wl.name}: {time.time() - t0:.1f}s")
        self.cfg = zha.Config(B=wl.B, H_kv=wl.H_kv, G=wl.G, d=wl.d, C=wl.C, L=wl.L, R=wl.R,
                              T_cap=self.T_cap,
                              kv_dtype=zha.F32 if wl.kv_dtype == "f32" else zha.BF16,
                              rope=wl.rope, rope_base=wl.rope_base)
        self.dec = zha.Decoder(self.cfg, self.qref, dev)

    def prefill(self):
        self.dec.tree.n_built.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        self.dec.prefill(self.K, self.V, self.Ts[0])
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def routed_steps(self, s0, s1, p, ev=None, counts=None, keep=None, router=None):
        """Steps s0..s1-1.  ev: dict collecting (route, attend, append) event pairs;
        keep: one LeafList per step, to hold each step's
        routed list; router: replaces the tree route (called with q, T and the
        step's leaf list)."""
        zha, dec, C = self.zha, self.dec, self.wl.C
        for s in range(s0, s1):
            T = self.Ts[s]
            q = self.Q[s]
            lst = keep[s - s0] if keep is not None else dec.leaves
            if (self.wl.T0 + s) % C == 0:
                marks = ev["append"] if ev is not None else None
                if marks is not None:
                    a0 = torch.cuda.Event(enable_timing=True)
                    a0.record()
                dec.append(self.K, self.V, T, 1)
                if marks is not None:
                    a1 = torch.cuda.Event(enable_timing=True)
                    a1.record()
                    marks.append((a0, a1))
            if ev is not None:
                r0 = torch.cuda.Event(enable_timing=True)
                r0.record()
            if router is not None:
                router(q, T, lst)
            else:
                zha.route(self.cfg, q, dec.tree, T, p, lst.ids, lst.mask, lst.count, dec.ws)
            if ev is not None:
                r1 = torch.cuda.Event(enable_timing=True)
                r1.record()
            zha.attend(self.cfg, q, self.K, self.V, T, lst.ids, lst.mask, lst.count,
                       dec.out, dec.lse, dec.ws)
            if ev is not None:
                r2 = torch.cuda.Event(enable_timing=True)
                r2.record()
                ev["route"].append((r0, r1))
                ev["attend"].append((r1, r2))
            if counts is not None:
                L = self.wl.L
                uc = torch.empty(L, self.wl.B, self.wl.H_kv, dtype=torch.int32, device="cuda")
                kc = torch.empty(L, self.wl.B, self.wl.Hq, dtype=torch.int32, device="cuda")
                zha.route_counts(self.cfg, dec.ws, uc, kc)
                first = lst.ids[:, :, 0].clone()
                counts.append((self.wl.T0 + s, uc, kc, lst.count.clone(), first))

    def attend_replay(self, s0, keep):
        """zha_attend of steps s0.. over their kept leaf lists, back to back."""
        zha, dec = self.zha, self.dec
        for i, lst in enumerate(keep):
            s = s0 + i
            zha.attend(self.cfg, self.Q[s], self.K, self.V, self.Ts[s], lst.ids, lst.mask,
                       lst.count, dec.out, dec.lse, dec.ws)

    def dense_steps(self, s0, s1, ev=None):
        for s in range(s0, s1):
            if ev is not None:
                d0 = torch.cuda.Event(enable_timing=True)
                d0.record()
            self.zha.dense_attend(self.cfg, self.Q[s], self.K, self.V, self.Ts[s], self.dec.out,
                                  self.dec.lse, self.dec.ws)
            if ev is not None:
                d1 = torch.cuda.Event(enable_timing=True)
                d1.record()
                ev.append((d0, d1))


def append_kind(wl, T):
    """The levels an append at length T completes (0: no chunk completes)."""
    if T <= 0 or T % wl.C:
        return 0
    k = 1
    while k < wl.L and T % wl.C ** (k + 1) == 0:
        k += 1
    return k


def append_cadence(run, p, reps=5, iters=32):
    """zha_append as a decode loop meets it: one call when a chunk completes, every
    C steps ([ZHA] page, append cadence).  An append that completes exactly the
    levels 1..k (the token count is a multiple of C^k and, below the top level,
    not of C^(k+1)) happens for a fraction 1/C^(k-1) - 1/C^k of the chunks
    (1/C^(L-1) for k = L).

    Each kind is measured inside the loop, by difference: at a length T_b of
    that kind, with the tree built, ``iters`` back-to-back iterations of (reset
    the built counts to those of T_b - 1, append, route, attend) against the
    same iterations with the counts reset to their own values and no append.
    The reset is the same small copy in both, and the append rebuilds the same
    nodes with the same values each time, so the difference is what the append
    adds to a step where it falls: its kernel queued between the attend and the
    next route, nothing bracketed by events.  Median over ``reps`` pairs.  The
    same append alone between two events, queued behind a prefill, is reported
    as ``isolated_us`` (the events' own overhead included).  The amortised cost per step is sum_k freq_k t_k / C."""
    zha, wl, dec = run.zha, run.wl, run.dec
    C, L = wl.C, wl.L
    Tt = torch.empty(wl.B, dtype=torch.int64, device="cuda")
    q = run.Q[0]
    lst = dec.leaves
    kinds = {}
    amort = 0.0
    for k in range(1, L + 1):
        span = C ** k
        Tb = (wl.T0 // span) * span
        if k < L and Tb % (span * C) == 0:
            Tb -= span
        freq = (1.0 / C ** (k - 1) - 1.0 / C ** k) if k < L else 1.0 / C ** (L - 1)
        if Tb < span:
            kinds[str(k)] = {"us": None, "isolated_us": None, "freq": freq, "T": None}
            continue
        assert append_kind(wl, Tb) == k
        Tt.fill_(Tb)
        dec.tree.n_built.zero_()
        dec.prefill(run.K, run.V, Tt)
        after = dec.tree.n_built.clone()
        before = torch.tensor([[(Tb - 1) // C ** l] * wl.B for l in range(1, L + 1)],
                              dtype=after.dtype, device="cuda")

        def loop(with_append):
            for _ in range(iters):
                dec.tree.n_built.copy_(before if with_append else after)
                if with_append:
                    dec.append(run.K, run.V, Tt, 1)
                zha.route(run.cfg, q, dec.tree, Tt, p, lst.ids, lst.mask, lst.count, dec.ws)
                zha.attend(run.cfg, q, run.K, run.V, Tt, lst.ids, lst.mask, lst.count,
                           dec.out, dec.lse, dec.ws)

        loop(True)
        loop(False)
        diffs = []
        for _ in range(reps):
            a = timed(lambda: loop(True))
            b = timed(lambda: loop(False))
            diffs.append(1000.0 * (a - b) / iters)
        if zha.ws_status(dec.ws) != 0:
            raise RuntimeError("append reported a device error")
        iso = []
        for _ in range(4):
            # queued behind a prefill to T_b - 1, so the GPU is busy when the first event is set
            Tt.fill_(Tb - 1)
            dec.tree.n_built.zero_()
            dec.prefill(run.K, run.V, Tt)
            Tt.fill_(Tb)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            dec.append(run.K, run.V, Tt, 1)
            e1.record()
            torch.cuda.synchronize()
            iso.append(1000.0 * e0.elapsed_time(e1))
        us = max(percentile(diffs, 0.5), 0.0)
        kinds[str(k)] = {"us": us, "isolated_us": percentile(iso[1:], 0.5), "freq": freq, "T": Tb}
        amort += freq * us
    return {"by_levels_completed": kinds,
            "us_per_append": amort,
            "us_per_step": amort / C}


def window_append_us(run, cad, s0, s1):
    """The in-loop cost of the appends that fall in steps s0..s1-1, by kind (none
    taken out when the measurement was skipped)."""
    if cad.get("skipped"):
        return 0.0, 0
    tot, n = 0.0, 0
    for s in range(s0, s1):
        k = append_kind(run.wl, run.wl.T0 + s)
        if k:
            us = cad["by_levels_completed"][str(k)]["us"]
            tot += us if us is not None else 0.0
            n += 1
    return tot, n


def graph_window(run, p, W, K, cad):
    """The same K steps with route + attend captured once in a HIP graph and
    replayed: each step copies its query and length into the captured buffers,
    runs zha_append eagerly when a chunk completes, then replays.  Returns the
    route + attend time per step (the window's appends taken out at their in-loop
    cost)."""
    zha, dec, wl = run.zha, run.dec, run.wl
    q_st, T_st = run.Q[W].clone(), run.Ts[W].clone()
    lst = dec.leaves
    run.prefill()
    run.routed_steps(0, W, p)

    def step():
        zha.route(run.cfg, q_st, dec.tree, T_st, p, lst.ids, lst.mask, lst.count, dec.ws)
        zha.attend(run.cfg, q_st, run.K, run.V, T_st, lst.ids, lst.mask, lst.count, dec.out,
                   dec.lse, dec.ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    def steps():
        for s in range(W, W + K):
            if (wl.T0 + s) % wl.C == 0:
                dec.append(run.K, run.V, run.Ts[s], 1)
            q_st.copy_(run.Q[s])
            T_st.copy_(run.Ts[s])
            g.replay()

    ms = timed(steps)
    if zha.ws_status(dec.ws) != 0:
        raise RuntimeError("graph replay reported a device error")
    del g
    return (ms * 1000.0 - window_append_us(run, cad, W, W + K)[0]) / K


def timed(fn):
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def finite_or_none(x):
    """x, or None where it is not finite (a level with no nodes): the line stays JSON."""
    return x if math.isfinite(x) else None


def percentile(v, q):
    """The q-quantile of a non-empty list (nearest rank)."""
    v = sorted(v)
    return v[min(len(v) - 1, int(round(q * (len(v) - 1))))]


def step_latency(ev, append_us_per_step):
    """Median and p90 over steps of route + attend (per-call events), plus the
    append cost amortised at its cadence."""
    per = [a.elapsed_time(b) + c.elapsed_time(d) for (a, b), (c, d) in zip(ev["route"], ev["attend"])]
    return {"median_us": 1000 * percentile(per, 0.5) + append_us_per_step,
            "p90_us": 1000 * percentile(per, 0.9) + append_us_per_step}


def copy_bandwidth():
    """Device-to-device copy rate of a 1 GiB buffer, read + written bytes per second."""
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    reps = 5
    ms = timed(lambda: [dst.copy_(src) for _ in range(reps)])
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n * reps / (ms * 1e-3) / 1e9


def bytes_of_step(wl, rec):
    """Algorithmic bytes of one routed step from its route counts: unique summary
    bytes scored per level, unique K/V bytes of the attended key set, q and out."""
    t, uc, kc, lc, first = rec
    uc, lc, first = uc.cpu(), lc.cpu(), first.cpu()
    node_bytes = wl.R * (wl.d + 1) * 4
    kv_row = 2 * wl.d * (2 if wl.kv_dtype == "bf16" else 4)
    n1 = t // wl.C
    route_b = int(uc.sum()) * node_bytes
    keys = 0
    for b in range(wl.B):
        for h in range(wl.H_kv):
            u = int(lc[b, h])
            sink = 1 if (n1 > 0 and (u == 0 or int(first[b, h]) != 0)) else 0
            keys += u * wl.C + (t - n1 * wl.C) + sink
    qo = wl.B * wl.Hq * (wl.d * 4 + (wl.d + 1) * 4)
    return route_b, keys * kv_row + qo, keys


def schedule_report(run, W, K, pl):
    """One depth schedule on the run's workload: step time, summary nodes scored
    and nodes kept per level, K/V bytes attended, dense-mass recall."""
    zha, wl = run.zha, run.wl
    run.prefill()
    run.routed_steps(0, W, pl)
    ms = timed(lambda: run.routed_steps(W, W + K, pl))
    run.prefill()
    run.routed_steps(0, W, pl)
    recs, keep = [], [zha.LeafList(run.cfg) for _ in range(K)]
    run.routed_steps(W, W + K, pl, counts=recs, keep=keep)
    torch.cuda.synchronize()
    scored = torch.zeros(wl.L, dtype=torch.float64)
    kept = torch.zeros(wl.L, dtype=torch.float64)
    rb = ab = 0
    for rec in recs:
        r, a, _ = bytes_of_step(wl, rec)
        rb += r
        ab += a
        scored += rec[1].cpu().to(torch.float64).sum(dim=(1, 2))
        kept += rec[2].cpu().to(torch.float64).sum(dim=(1, 2))
    recall = []
    o_r, l_r = torch.empty_like(run.dec.out), torch.empty_like(run.dec.lse)
    for i, lst in enumerate(keep):
        s = W + i
        zha.attend(run.cfg, run.Q[s], run.K, run.V, run.Ts[s], lst.ids, lst.mask, lst.count,
                   o_r, l_r, run.dec.ws)
        zha.dense_attend(run.cfg, run.Q[s], run.K, run.V, run.Ts[s], run.dec.out, run.dec.lse,
                         run.dec.ws)
        recall.append(torch.exp(l_r - run.dec.lse).flatten())
    recall = torch.cat(recall).double().cpu()
    return {
        "p_levels": [float(x) for x in (pl if isinstance(pl, (list, tuple)) else [pl] * wl.L)],
        "us_per_step": ms * 1000.0 / K,
        "nodes_scored_per_group_per_level": [float(x) / (K * wl.B * wl.H_kv) for x in scored],
        "nodes_kept_per_head_per_level": [float(x) / (K * wl.B * wl.Hq) for x in kept],
        "summary_MB_per_step": rb / K / 1e6, "kv_MB_per_step": ab / K / 1e6,
        "mass_recall_mean": float(recall.mean()), "mass_recall_min": float(recall.min()),
        "note": "levels listed from 1 (leaves) to L",
    }


def bf16_copy_report(run, W, K, p):
    """The same steps with the route scoring from a bf16 copy of every level's
    k_hat (zha_tree.khat16, written by the builder beside the fp32 tree): step
    time (raw window, its appends included), route time, summary bytes the route
    reads, and the dense-mass recall of the routed sets.  The tree goes back to
    fp32 routing afterwards."""
    zha, wl, tree = run.zha, run.wl, run.dec.tree
    tree.khat16 = [torch.zeros(k.shape, dtype=torch.bfloat16, device=k.device) for k in tree.khat]
    try:
        run.prefill()
        run.routed_steps(0, W, p)
        ms = timed(lambda: run.routed_steps(W, W + K, p))
        run.prefill()
        run.routed_steps(0, W, p)
        ev = {"route": [], "attend": [], "append": []}
        recs, keep = [], [zha.LeafList(run.cfg) for _ in range(K)]
        run.routed_steps(W, W + K, p, ev, counts=recs, keep=keep)
        torch.cuda.synchronize()
        route_us = 1000.0 * sum(a.elapsed_time(b) for a, b in ev["route"]) / K
        node_bytes = wl.R * wl.d * 2 + wl.R * 4          # bf16 k_hat rows + fp32 b_hat
        scored = sum(float(rec[1].to(torch.float64).sum()) for rec in recs) / K
        recall = []
        o_r, l_r = torch.empty_like(run.dec.out), torch.empty_like(run.dec.lse)
        for i, lst in enumerate(keep):
            s = W + i
            zha.attend(run.cfg, run.Q[s], run.K, run.V, run.Ts[s], lst.ids, lst.mask, lst.count,
                       o_r, l_r, run.dec.ws)
            zha.dense_attend(run.cfg, run.Q[s], run.K, run.V, run.Ts[s], run.dec.out, run.dec.lse,
                             run.dec.ws)
            recall.append(torch.exp(l_r - run.dec.lse).flatten())
        recall = torch.cat(recall).double().cpu()
    finally:
        tree.khat16 = [None] * wl.L
        torch.cuda.empty_cache()
    return {
        "us_per_step": ms * 1000.0 / K, "route_us": route_us,
        "route_summary_GB_per_step": scored * node_bytes / 1e9,
        "route_GBps": scored * node_bytes / (route_us * 1e-6) / 1e9,
        "mass_recall_mean": float(recall.mean()), "mass_recall_min": float(recall.min()),
        "note": "route scoring from bf16 copies of k_hat (b_hat and all arithmetic fp32); raw "
                "window over the same steps, its appends included; the headline value uses the "
                "fp32 summaries",
    }


def flat_report(run, W, K, mode, p, budget):
    """Flat routing over every leaf (a one-level view of the same leaf summaries):
    top-p at p, or a fixed budget of leaves per head.  Step time, route time,
    leaves kept and dense-mass recall over the same steps."""
    zha, wl = run.zha, run.wl
    cfg1 = zha.Config(B=wl.B, H_kv=wl.H_kv, G=wl.G, d=wl.d, C=wl.C, L=1, R=wl.R,
                      T_cap=run.T_cap, kv_dtype=run.cfg.kv_dtype, rope=wl.rope,
                      rope_base=wl.rope_base)
    tree1 = zha.Tree.lower_levels(run.dec.tree, cfg1)
    ws1 = zha.new_workspace(cfg1)

    def router(q, T, lst):
        if mode == "topk":
            zha.route_topk(cfg1, q, tree1, T, budget, lst.ids, lst.mask, lst.count, ws1)
        else:
            zha.route(cfg1, q, tree1, T, p, lst.ids, lst.mask, lst.count, ws1)

    run.prefill()
    run.routed_steps(0, W, p, router=router)
    ms = timed(lambda: run.routed_steps(W, W + K, p, router=router))
    run.prefill()
    run.routed_steps(0, W, p, router=router)
    ev = {"route": [], "attend": [], "append": []}
    keep = [zha.LeafList(run.cfg) for _ in range(K)]
    run.routed_steps(W, W + K, p, ev, keep=keep, router=router)
    torch.cuda.synchronize()
    if zha.ws_status(ws1) != 0:
        raise RuntimeError("flat route reported a device error")
    route_us = 1000 * sum(a.elapsed_time(b) for a, b in ev["route"]) / K
    leaves = sum(float(lst.count.sum()) for lst in keep) / (K * wl.B * wl.H_kv)
    recall = []
    o_r, l_r = torch.empty_like(run.dec.out), torch.empty_like(run.dec.lse)
    for i, lst in enumerate(keep):
        s = W + i
        zha.attend(run.cfg, run.Q[s], run.K, run.V, run.Ts[s], lst.ids, lst.mask, lst.count,
                   o_r, l_r, run.dec.ws)
        zha.dense_attend(run.cfg, run.Q[s], run.K, run.V, run.Ts[s], run.dec.out, run.dec.lse,
                         run.dec.ws)
        recall.append(torch.exp(l_r - run.dec.lse).flatten())
    recall = torch.cat(recall).double().cpu()
    return {"us_per_step": ms * 1000.0 / K, "route_us": route_us,
            "summary_MB_per_step": wl.B * wl.H_kv * (wl.T0 + W + K // 2) // wl.C * wl.R * (wl.d + 1) * 4 / 1e6,
            "leaves_per_group": leaves,
            "mass_recall_mean": float(recall.mean()), "mass_recall_min": float(recall.min()),
            "budget_leaves_per_head": budget if mode == "topk" else None}


def cpu_baseline(run, p, s):
    """The oracle timed on a bounded sample: one KV head of sequence 0 (its G query
    heads) for one decode step, with the oracle's own tree; scaled to a full step."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    import oracle as O
    wl = run.wl
    t = wl.T0 + s
    K = run.K[0, 0, :t].to("cpu").to(torch.float64).numpy()
    V = run.V[0, 0, :t].to("cpu").to(torch.float64).numpy()
    qref = run.qref[0].to("cpu").to(torch.float64).numpy()
    q = run.Q[s, 0, :wl.G].to("cpu").to(torch.float64).numpy()
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        t0 = time.perf_counter()
        tree = O.build_tree(K, qref, t, wl.C, wl.L, wl.scale, wl.rope_base if wl.rope else None)
        build_s = time.perf_counter() - t0
        t0 = time.perf_counter()
        for g in range(wl.G):
            rt = O.route(q[g], tree, t, wl.C, wl.L, p, wl.scale)
            keys = O.routed_keys(rt.leaves, t, wl.C)
            O.attend_keys(q[g], K, V, keys, wl.scale)
        step_s = time.perf_counter() - t0
        t0 = time.perf_counter()
        for g in range(wl.G):
            O.attention(q[g], K, V, wl.scale)
        dense_s = time.perf_counter() - t0
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    # the same routed step with numpy's thread pools at every core of this process
    ncores = len(os.sched_getaffinity(0))
    ctx = threadpool_limits(limits=ncores) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        t0 = time.perf_counter()
        for g in range(wl.G):
            rt = O.route(q[g], tree, t, wl.C, wl.L, p, wl.scale)
            keys = O.routed_keys(rt.leaves, t, wl.C)
            O.attend_keys(q[g], K, V, keys, wl.scale)
        step_all_s = time.perf_counter() - t0
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    groups = wl.B * wl.H_kv
    return {
        "value": step_s * groups * 1e6, "unit": "us/step", "cores": 1, "kind": "oracle",
        "sample": f"KV head 0 of sequence 0 ({wl.G} query heads), one decode step at T={t}, "
                  f"numpy float64 single-threaded; x{groups} KV-head groups for a full step",
        "dense_us_per_step": dense_s * groups * 1e6,
        "tree_build_s_one_head": build_s,
        "all_cores": {"value": step_all_s * groups * 1e6, "cores": ncores,
                      "note": "the same sample with numpy's BLAS/OpenMP pools at every core"},
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the path is not "
              "sharded over several GPUs", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    wl = synth.WORKLOADS[args.workload]
    p = args.p if args.p is not None else wl.p
    W, K = args.warmup, args.steps
    run = Run(wl, W + K)
    zha = run.zha

    run.prefill()                 # first call: the library's kernels load
    build_ms = run.prefill()
    log(f"[bench] prefill tree build: {build_ms:.2f} ms")

    # ---- routed: warmup, then exactly K timed steps back to back, nothing else in
    # the queue (the appends that fall in the window included, no events inside)
    run.routed_steps(0, W, p)
    total_ms = timed(lambda: run.routed_steps(W, W + K, p))
    st = zha.ws_status(run.dec.ws)
    if st != 0:
        raise RuntimeError(f"device status {zha.status_str(st)}")
    # the append at its cadence (one per C steps, with the parents it completes),
    # measured in the loop kind by kind: a K-step window holds too few chunks to
    # sample the mixture, so the window's own appends are replaced by it
    if args.no_append_cadence:
        cad = {"by_levels_completed": {}, "us_per_append": 0.0, "us_per_step": 0.0,
               "skipped": True}
        win_app_us, n_app = 0.0, sum(1 for s_ in range(W, W + K) if append_kind(wl, wl.T0 + s_))
    else:
        cad = append_cadence(run, p)
        win_app_us, n_app = window_append_us(run, cad, W, W + K)
    ra_us = (total_ms * 1000.0 - win_app_us) / K
    us_step = ra_us + cad["us_per_step"]
    log(f"[bench] routed p={p}: {us_step:.1f} us/step (route + attend {ra_us:.1f}, append "
        f"{cad['us_per_append']:.1f} us per chunk = {cad['us_per_step']:.2f} us/step; "
        f"raw window {total_ms * 1000.0 / K:.1f} with {n_app} appends)")

    # ---- the same steps again, for the breakdown: events around each call (each
    # event is a queue marker, so route_us + attend_us slightly exceed a step),
    # every step's leaf list kept, and the route diagnostics for byte accounting
    run.prefill()
    run.routed_steps(0, W, p)
    ev = {"route": [], "attend": [], "append": []}
    keep = [zha.LeafList(run.cfg) for _ in range(K)]
    recs = [] if not args.no_stats else None
    run.routed_steps(W, W + K, p, ev, counts=recs, keep=keep)
    torch.cuda.synchronize()
    route_ms = [a.elapsed_time(b) for a, b in ev["route"]]
    append_ms = [a.elapsed_time(b) for a, b in ev["append"]]
    # the K attends replayed back to back over their own lists: the attend time
    run.attend_replay(W, keep)
    attend_ms_total = timed(lambda: run.attend_replay(W, keep))
    attend_us = attend_ms_total * 1000.0 / K
    route_us = 1000 * sum(route_ms) / K
    log(f"[bench]   route {route_us:.1f} us (per-call events), attend {attend_us:.1f} us "
        f"(replayed), appends {len(append_ms)}")
    warm = step_latency(ev, cad["us_per_step"])

    # ---- cold steps: a 512 MB buffer is written before each step (untimed), so a
    # step starts with nothing of its data in the 256 MB last-level cache
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    run.prefill()
    run.routed_steps(0, W, p)
    evc = {"route": [], "attend": [], "append": []}
    for s in range(W, W + K):
        flush.fill_(s & 0x7f)
        run.routed_steps(s, s + 1, p, evc)
    torch.cuda.synchronize()
    cold = step_latency(evc, cad["us_per_step"])
    del flush
    torch.cuda.empty_cache()
    log(f"[bench]   per step (events): warm median {warm['median_us']:.1f} p90 {warm['p90_us']:.1f} us; "
        f"cold median {cold['median_us']:.1f} p90 {cold['p90_us']:.1f} us")
    graph_ra_us = graph_window(run, p, W, K, cad)
    log(f"[bench]   graph-replayed route + attend: {graph_ra_us:.1f} us/step "
        f"(eager {ra_us:.1f})")
    copy_gbps = copy_bandwidth()
    log(f"[bench]   device copy {copy_gbps:.0f} GB/s")

    extra = {}
    # ---- p sweep (same steps, warm)
    for ps in [float(x) for x in args.p_sweep.split(",") if x.strip()]:
        if ps == p:
            continue
        run.prefill()
        run.routed_steps(0, W, ps)
        ms = timed(lambda: run.routed_steps(W, W + K, ps))
        extra[f"p{ps}"] = {"us_per_step": (ms * 1000.0 - win_app_us) / K + cad["us_per_step"]}
        log(f"[bench] routed p={ps}: {extra[f'p{ps}']['us_per_step']:.1f} us/step")

    # ---- dense baseline over the same steps
    dense = None
    if not args.no_dense:
        run.dense_steps(0, W)
        ms = timed(lambda: run.dense_steps(W, W + K))
        dense_bytes = 0
        for s in range(W, W + K):
            dense_bytes += wl.B * wl.H_kv * (wl.T0 + s) * 2 * wl.d * (2 if wl.kv_dtype == "bf16" else 4)
        dense = {"us_per_step": ms * 1000.0 / K,
                 "effective_GBps": dense_bytes / K / (ms / K * 1e-3) / 1e9}
        dense["hbm_frac"] = dense["effective_GBps"] / HBM_PEAK_GBPS
        log(f"[bench] dense: {dense['us_per_step']:.1f} us/step, {dense['effective_GBps']:.0f} GB/s")

    # ---- quality of the routed steps against dense attention (untimed): the
    # dense softmax mass the routed key set holds is exp(lse_routed - lse_dense)
    if not args.no_dense:
        recall, oerr = [], []
        o_r = torch.empty_like(run.dec.out)
        l_r = torch.empty_like(run.dec.lse)
        for i, lst in enumerate(keep):
            s = W + i
            zha.attend(run.cfg, run.Q[s], run.K, run.V, run.Ts[s], lst.ids, lst.mask, lst.count,
                       o_r, l_r, run.dec.ws)
            zha.dense_attend(run.cfg, run.Q[s], run.K, run.V, run.Ts[s], run.dec.out,
                             run.dec.lse, run.dec.ws)
            recall.append(torch.exp(l_r - run.dec.lse).flatten())
            num = (o_r - run.dec.out).abs().amax(dim=-1)
            oerr.append((num / run.dec.out.abs().amax(dim=-1).clamp_min(1e-30)).flatten())
        recall = torch.cat(recall).double().cpu()
        oerr = torch.cat(oerr).double().cpu()
        # per-level KL(p || p_hat) of the routing estimate, on the final tree state
        # (every step's query against the tree at the last step's length)
        kl = torch.empty(wl.L, wl.B, wl.Hq, device="cuda")
        kls = []
        s_last = W + K - 1
        for s in range(W, W + K, max(1, K // 8)):
            zha.route_quality(run.cfg, run.Q[s], run.K, run.V, run.Ts[s_last], run.dec.tree, kl,
                              run.dec.ws)
            kls.append(kl.clone())
        kls = torch.stack(kls).double().cpu()
        extra["quality_vs_dense"] = {
            "mass_recall_mean": float(recall.mean()), "mass_recall_min": float(recall.min()),
            "out_rel_err_mean": float(oerr.mean()), "out_rel_err_max": float(oerr.max()),
            "kl_per_level_mean": [finite_or_none(float(kls[:, l].mean())) for l in range(wl.L)],
            "note": "per query head and step: recall = dense softmax mass of the routed key set; "
                    "kl = KL(true || estimated) node distribution per level (1 .. L)"}
        log(f"[bench] dense-mass recall of the routed sets: mean {float(recall.mean()):.4f}, "
            f"min {float(recall.min()):.4f}")

    # ---- byte accounting from the breakdown pass's route diagnostics
    route_bytes = attend_bytes = keys_total = 0
    sel_frac = None
    if recs is not None:
        kept = torch.zeros(wl.L)
        for rec in recs:
            rb, ab, keys = bytes_of_step(wl, rec)
            route_bytes += rb
            attend_bytes += ab
            keys_total += keys
            kept += rec[2].cpu().to(torch.float64).sum(dim=(1, 2))
        sel_frac = keys_total / sum(wl.B * wl.H_kv * (wl.T0 + s) for s in range(W, W + K))
        extra["kept_per_head_per_level"] = [float(x) / (K * wl.B * wl.Hq) for x in kept]

    att_s = attend_ms_total * 1e-3
    rte_s = sum(route_ms) * 1e-3
    att_gbps = attend_bytes / att_s / 1e9 if att_s > 0 and attend_bytes else None
    rte_gbps = route_bytes / rte_s / 1e9 if rte_s > 0 and route_bytes else None
    step_gbps = (attend_bytes + route_bytes) / (total_ms * 1e-3) / 1e9 if attend_bytes else None
    dominant = "attend" if attend_us >= route_us else "route"
    ach = att_gbps if dominant == "attend" else rte_gbps
    alg = (attend_bytes if dominant == "attend" else route_bytes) / K
    ratio = stored_traffic_ratio(wl.name, p) if dominant == "attend" else None
    roofline = {
        "bound": "hbm",
        "kernel": "zha_attend (split-K partial + merge)" if dominant == "attend" else "zha_route (all levels)",
        "achieved": ach, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
        "frac": (ach / HBM_PEAK_GBPS) if ach else None,
        "traffic": (ratio * alg) if (ratio is not None and alg) else None,
        "traffic_source": (f"counter HBM bytes / algorithmic bytes = {ratio:.4f} from "
                           f"profiles/attend_{wl.name}_traffic.json (same attend source), times "
                           f"this run's algorithmic bytes") if ratio is not None else None,
        "avg_launch_us": attend_us if dominant == "attend" else route_us,
        "algorithmic_bytes_per_launch": alg,
    }

    # ---- the route scoring from bf16 copies of k_hat (same steps, same p)
    if not args.no_bf16_copy:
        r16 = bf16_copy_report(run, W, K, p)
        extra["route_bf16_copy"] = r16
        log(f"[bench] route from bf16 k_hat copies: {r16['us_per_step']:.1f} us/step "
            f"(route {r16['route_us']:.1f} us, {r16['route_summary_GB_per_step']:.3f} GB), "
            f"recall {r16['mass_recall_mean']:.4f}")

    # ---- depth schedules of p (same product p = the headline p for root/power)
    kinds = [x.strip() for x in args.schedules.split(",") if x.strip()]
    if kinds:
        sched = {}
        for kind in kinds:
            pl = zha.p_schedule(kind, p, wl.L, gamma=args.gamma)
            sched[kind] = schedule_report(run, W, K, pl)
            r = sched[kind]
            log(f"[bench] schedule {kind}: {r['us_per_step']:.1f} us/step, summaries "
                f"{r['summary_MB_per_step']:.1f} MB, K/V {r['kv_MB_per_step']:.1f} MB, "
                f"recall {r['mass_recall_mean']:.3f}")
        extra["depth_schedules"] = sched

    # ---- flat routing over every leaf: top-p, and top-K at the tree's leaf budget
    if args.flat:
        budget = max(1, int(round(extra.get("kept_per_head_per_level", [64])[0])))
        flat = {}
        for mode in ("topp", "topk"):
            flat[mode] = flat_report(run, W, K, mode, p, budget)
            r = flat[mode]
            log(f"[bench] flat {mode}: {r['us_per_step']:.1f} us/step (route {r['route_us']:.1f}), "
                f"recall {r['mass_recall_mean']:.3f}, leaves/group {r['leaves_per_group']:.0f}")
        extra["flat_comparator"] = flat

    # ---- context-length sweep at the same geometry: routed vs dense
    sweep = {}
    for e in [int(x) for x in args.n_sweep.split(",") if x.strip()]:
        if (1 << e) == wl.N:
            continue
        del keep
        keep = None
        torch.cuda.empty_cache()
        wls = wl.with_(N=1 << e)
        Ws, Ks = 4, 16
        rs = Run(wls, Ws + Ks)
        rs.prefill()
        rs.routed_steps(0, Ws, p)
        ms_r = timed(lambda: rs.routed_steps(Ws, Ws + Ks, p))
        rs.dense_steps(0, Ws)
        ms_d = timed(lambda: rs.dense_steps(Ws, Ws + Ks))
        sweep[str(wls.T0)] = {"routed_us_per_step": ms_r * 1000.0 / Ks,
                              "dense_us_per_step": ms_d * 1000.0 / Ks,
                              "speedup_vs_dense": ms_d / ms_r}
        if not args.no_bf16_copy:
            r16 = bf16_copy_report(rs, Ws, Ks, p)
            sweep[str(wls.T0)]["routed_bf16_copy_us_per_step"] = r16["us_per_step"]
        if args.flat:
            rs.prefill()
            rs.routed_steps(0, Ws, p)
            recs_s = []
            rs.routed_steps(Ws, Ws + Ks, p, counts=recs_s)
            kept1 = sum(float(r[2][0].sum()) for r in recs_s) / (Ks * wls.B * wls.Hq)
            budget_s = max(1, int(round(kept1)))
            sweep[str(wls.T0)]["flat_topp"] = flat_report(rs, Ws, Ks, "topp", p, budget_s)
            sweep[str(wls.T0)]["flat_topk"] = flat_report(rs, Ws, Ks, "topk", p, budget_s)
            rs.prefill()
            rs.routed_steps(0, Ws, 0.75)
            ms_75 = timed(lambda: rs.routed_steps(Ws, Ws + Ks, 0.75))
            sweep[str(wls.T0)]["routed_p0.75_us_per_step"] = ms_75 * 1000.0 / Ks
        log(f"[bench] T={wls.T0}: routed {ms_r * 1000 / Ks:.1f} us/step, dense {ms_d * 1000 / Ks:.1f}"
            + (f", routed from the bf16 copy {sweep[str(wls.T0)]['routed_bf16_copy_us_per_step']:.1f}"
               if "routed_bf16_copy_us_per_step" in sweep[str(wls.T0)] else ""))
        del rs
        torch.cuda.empty_cache()
    if sweep:
        sweep[str(wl.T0)] = {"routed_us_per_step": us_step,
                             "dense_us_per_step": dense["us_per_step"] if dense else None,
                             "speedup_vs_dense": (dense["us_per_step"] / us_step) if dense else None}
        if "route_bf16_copy" in extra:
            sweep[str(wl.T0)]["routed_bf16_copy_us_per_step"] = extra["route_bf16_copy"]["us_per_step"]
        if args.flat:
            sweep[str(wl.T0)]["flat_topp"] = extra["flat_comparator"]["topp"]
            sweep[str(wl.T0)]["flat_topk"] = extra["flat_comparator"]["topk"]
            if "p0.75" in extra:
                sweep[str(wl.T0)]["routed_p0.75_us_per_step"] = extra["p0.75"]["us_per_step"]
        extra["context_sweep"] = sweep

    cpu = None
    if not args.no_cpu:
        log("[bench] oracle CPU baseline (bounded sample) ...")
        cpu = cpu_baseline(run, p, W)
        log(f"[bench] oracle: {cpu['value']:.0f} us/step (sample)")

    out = {
        "metric": METRIC, "value": us_step, "unit": "us/step", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": total_ms / K, "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.kv_dtype, "data": "synthetic",
        "precision": ("K/V bf16; q.k and p.v on bf16 MFMA with q and p each split into a hi + lo "
                      "bf16 pair (~2^-17 relative), fp32 accumulation; scores, softmax, summaries, "
                      "routing, out and lse in fp32") if wl.kv_dtype == "bf16" else
                     "fp32 throughout (K/V, scores, softmax, summaries, out, lse)",
        "config": {"workload": wl.name, "B": wl.B, "H_kv": wl.H_kv, "G": wl.G, "d": wl.d,
                   "T0": wl.T0, "C": wl.C, "L": wl.L, "R": wl.R, "p": p, "kv_dtype": wl.kv_dtype,
                   "clusters": wl.n_clusters, "cluster_law": wl.freq},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "route_us": route_us,
        "attend_us": attend_us,
        "route_attend_us": ra_us,
        "graph": {"route_attend_us": graph_ra_us, "us_per_step": graph_ra_us + cad["us_per_step"],
                  "note": "route + attend captured once in a HIP graph and replayed per step "
                          "(query and length copied into the captured buffers each step, appends "
                          "eager); value is the eager loop"},
        "append": {**cad, "frac_of_step": None if cad.get("skipped") else cad["us_per_step"] / us_step,
                   "within_1pct": None if cad.get("skipped") else cad["us_per_step"] <= 0.01 * us_step,
                   "note": "zha_append per completed chunk (one call every C steps), by the levels "
                           "it completes, measured inside the decode loop (difference of back-to-back "
                           "iterations with and without the append; isolated_us: the call alone "
                           "between two events), weighted by their cadence; us_per_step = "
                           "us_per_append / C, included in value in place of the window's own "
                           "appends"},
        "append_us_each": cad["us_per_append"],
        "window_us_per_step_raw": total_ms * 1000.0 / K,
        "appends_in_timed_steps": n_app,
        "prefill_build_ms": build_ms,
        "step_latency": {"warm": warm, "cold": cold,
                         "note": "per-step route + attend from per-call events (queue markers add "
                                 "a little), appends spread over the steps; cold: a 512 MB buffer "
                                 "written before each step"},
        "copy_GBps": copy_gbps,
        "effective_frac_of_copy": (step_gbps / copy_gbps) if step_gbps else None,
        "attend_frac_of_copy": (att_gbps / copy_gbps) if att_gbps else None,
        "effective_GBps_step": step_gbps,
        "route_GBps": rte_gbps,
        "attend_GBps": att_gbps,
        "selected_key_frac": sel_frac,
        "dense": dense,
        "speedup_vs_dense": (dense["us_per_step"] / us_step) if dense else None,
        **extra,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
