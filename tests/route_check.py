"""Comparison of a routed selection with the oracle's, with the allowed cases.

A GPU selection of one (level, query head) equals the oracle's, or differs only
in one of two ways that fp32 arithmetic cannot avoid:
  * near-tie: the GPU keeps x and drops y although the oracle ranks y above x,
    with |s(x) - s(y)| < TIE (oracle scores);
  * near-threshold: the kept count differs and every oracle prefix sum between
    the two counts lies within THR * W of the cut value p * W.
Every allowed case is returned so the caller can report it.
"""
from __future__ import annotations

import numpy as np

TIE = 1e-5
THR = 1e-5


def classify(cut, gpu_sel):
    """cut: oracle TopP of the level (its own scores); gpu_sel: GPU-kept ids.
    Returns (ok, note) where note describes an allowed mismatch or is None."""
    o_sel = set(int(x) for x in cut.selected)
    g_sel = set(int(x) for x in gpu_sel)
    if o_sel == g_sel:
        return True, None
    ids = [int(x) for x in cut.ids]
    if not g_sel.issubset(set(ids)):
        return False, f"GPU kept non-candidates {sorted(g_sel - set(ids))[:5]}"
    pos = {i: k for k, i in enumerate(ids)}
    s = cut.scores
    kept = [s[pos[i]] for i in g_sel]
    dropped = [s[pos[i]] for i in ids if i not in g_sel]
    if kept and dropped and min(kept) < max(dropped) - TIE:
        return False, f"order violated: min kept {min(kept)} < max dropped {max(dropped)}"
    m_o, m_g = len(o_sel), len(g_sel)
    cums = np.cumsum(cut.w[cut.order])
    tol = THR * cut.W
    if m_g != m_o:
        lo, hi = min(m_o, m_g), max(m_o, m_g)
        for m in range(lo, hi):  # prefix sum of the top m masses
            c = cums[m - 1] if m >= 1 else 0.0
            if abs(c - cut.target) >= tol:
                return False, f"count {m_g} vs {m_o}, prefix {m} off threshold by {abs(c - cut.target) / cut.W:.3g} W"
        return True, f"near-threshold: kept {m_g} vs oracle {m_o}"
    return True, f"near-tie swap: {sorted(g_sel ^ o_sel)[:6]}"
