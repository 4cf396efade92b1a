"""Helpers for the GPU parity tests (host-side conversions and comparisons)."""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle as O

TOL = {"f32": 1e-5, "bf16": 2e-3}  # max |o - o_ref| / max |o_ref| per query head


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a device tensor (fp32 or bf16) to float64 numpy."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def rel_err(o, ref) -> float:
    o = np.asarray(o, np.float64)
    ref = np.asarray(ref, np.float64)
    den = max(np.max(np.abs(ref)), 1e-30)
    return float(np.max(np.abs(o - ref)) / den)


def union_cap(sets_per_head, B, H_kv, G):
    """Largest per-group union size of per-head sets (at least 1)."""
    m = 1
    for b in range(B):
        for h in range(H_kv):
            u = set()
            for g in range(G):
                u.update(int(x) for x in sets_per_head[b][h * G + g])
            m = max(m, len(u))
    return m


def lists_from_sets(sets_per_head, B, H_kv, G, cap=None):
    """Per-head leaf sets -> (ids, mask, count) union lists [B][H_kv][cap]."""
    if cap is None:
        cap = union_cap(sets_per_head, B, H_kv, G)
    ids = torch.zeros(B, H_kv, cap, dtype=torch.int32)
    mask = torch.zeros(B, H_kv, cap, dtype=torch.int32)
    count = torch.zeros(B, H_kv, dtype=torch.int32)
    for b in range(B):
        for h in range(H_kv):
            m = {}
            for g in range(G):
                for leaf in sets_per_head[b][h * G + g]:
                    m[int(leaf)] = m.get(int(leaf), 0) | (1 << g)
            keys = sorted(m)
            assert len(keys) <= cap
            count[b, h] = len(keys)
            if keys:
                ids[b, h, :len(keys)] = torch.tensor(keys, dtype=torch.int32)
                mask[b, h, :len(keys)] = torch.tensor([m[k] for k in keys], dtype=torch.int64).to(torch.int32)
    return ids, mask, count


def sets_from_lists(ids, mask, count, G):
    """(ids, mask, count) -> per (b, query head) sorted leaf arrays."""
    ids, mask, count = ids.cpu().numpy(), mask.cpu().numpy().astype(np.int64) & 0xffffffff, count.cpu().numpy()
    B, H_kv = count.shape
    out = [[None] * (H_kv * G) for _ in range(B)]
    for b in range(B):
        for h in range(H_kv):
            n = int(count[b, h])
            for g in range(G):
                sel = ids[b, h, :n][(mask[b, h, :n] >> g) & 1 == 1]
                out[b][h * G + g] = np.sort(sel.astype(np.int64))
    return out
