"""Shared helpers for the GPU parity tests: device transfer of synthetic inputs
and element-by-element comparison of GPU outputs with the CPU oracle."""
from __future__ import annotations

import os

import numpy as np
import torch

# A decision is a near tie when the oracle's uniform lies within this distance
# of the accept threshold min(1, p/q) (the stated bar), or, for an inverse-CDF
# draw, within this fraction of the total mass of a bucket edge. The GPU does
# the accept test with normalisers good to ~1e-7 and every final draw in fp64.
NEAR_TIE_ACCEPT = 1e-6
NEAR_TIE_CDF = 1e-11
PROB_RTOL = 1e-5
RESID_RTOL = 1e-9

THREADS = max(1, min(16, os.cpu_count() or 1))


def f32(x: float) -> float:
    """x rounded to binary32 (how the C ABI carries temperature and top_p)."""
    return float(np.float32(x))


def to_dev(a: np.ndarray) -> torch.Tensor:
    """numpy float32 -> float32 device tensor; uint16 (bfloat16 bits) -> bfloat16."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def compare_linear(g: dict, o: dict, check_probs=True, check_resid=True):
    """Compare GPU outputs (torch) with oracle outputs (numpy), request by request.

    Returns (mismatched_requests_excused, total_decisions, near_ties). Raises
    AssertionError on any mismatch that is not a near tie, on probabilities
    outside PROB_RTOL and on residual masses outside RESID_RTOL.
    """
    gl = g["len"].cpu().numpy()
    gt = g["tokens"].cpu().numpy()
    ol, ot = o["len"], o["tokens"]
    B = len(ol)
    ma, mc = o["margin_acc"], o["margin_cdf"]
    near = (ma < NEAR_TIE_ACCEPT) | (mc < NEAR_TIE_CDF)
    excused = 0
    for b in range(B):
        if gl[b] == ol[b] and np.array_equal(gt[b], ot[b]):
            continue
        assert near[b], (f"request {b}: gpu len {gl[b]} tokens {gt[b].tolist()} vs oracle len {ol[b]} "
                         f"tokens {ot[b].tolist()} (margins acc {ma[b]:.3g} cdf {mc[b]:.3g})")
        excused += 1
    valid = (ol >= 0) & (gl == ol)
    if check_probs and g.get("probs") is not None:
        gp = g["probs"].cpu().numpy().astype(np.float64)
        op = o["probs"]
        for b in np.nonzero(valid)[0]:
            err = np.abs(gp[b] - op[b])
            tol = PROB_RTOL * np.abs(op[b]) + 2e-38
            assert np.all(err <= tol), f"request {b}: probs {gp[b].tolist()} vs {op[b].tolist()}"
    if check_resid and g.get("resid") is not None:
        gr = g["resid"].cpu().numpy()
        orr = o["resid"]
        same = valid & np.array([np.array_equal(gt[b], ot[b]) for b in range(B)])
        for b in np.nonzero(same)[0]:
            assert abs(gr[b] - orr[b]) <= RESID_RTOL * abs(orr[b]) + 1e-15, f"request {b}: resid {gr[b]} vs {orr[b]}"
    K = ot.shape[1] - 1
    decisions = sum(min(int(n) + 1, K) + 1 for n in ol if n >= 0)
    return excused, max(decisions, 1), int(near.sum())


def compare_tree(g: dict, o: dict):
    """Tree outputs: len, tokens and path identical per request, except requests
    whose oracle decisions include a near tie. Returns (excused, near_ties)."""
    gl = g["len"].cpu().numpy()
    gt = g["tokens"].cpu().numpy()
    gp = g["path"].cpu().numpy()
    ol, ot, op = o["len"], o["tokens"], o["path"]
    near = (o["margin_acc"] < NEAR_TIE_ACCEPT) | (o["margin_cdf"] < NEAR_TIE_CDF)
    excused = 0
    for b in range(len(ol)):
        if gl[b] == ol[b] and np.array_equal(gt[b], ot[b]) and np.array_equal(gp[b], op[b]):
            continue
        assert near[b], (f"request {b}: gpu len {gl[b]} path {gp[b].tolist()} tokens {gt[b].tolist()} vs oracle "
                         f"len {ol[b]} path {op[b].tolist()} tokens {ot[b].tolist()}")
        excused += 1
    return excused, int(near.sum())
