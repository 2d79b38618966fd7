"""Shared helpers for the GPU parity tests: device transfer of synthetic inputs
and element-by-element comparison of GPU outputs with the CPU oracle.

The excuse rule. GPU and oracle compute in different precisions, so they may
part at a decision that lies within a band of going the other way: a near
tie. A request whose outputs differ is excused only when the FIRST decision at
which the two can have parted is a near tie of the oracle, and, for an
inverse-CDF draw, only when the GPU's token is the one across that draw's
nearer edge. Decisions are ordered as the method takes them: filter cuts of
every row, then the drafts, then the accept tests in order (the first
rejection ends the walk), then the final draw. Every other mismatch fails.
Each comparison returns a Tally: decisions taken, oracle near ties among them,
and excused requests. Tests assert that excused requests stay within
max(1, 1e-4 of the decisions), and large tests assert that near ties make up
less than 1e-4 of the decisions.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

# Bands. Accept test: |u - min(1, p/q)| < 1e-6, the stated bar (the GPU's
# normalisers are good to ~1e-7). Inverse-CDF draws: 1e-11 of the drawn mass
# (the GPU draws in fp64). Top-p cuts: 1e-11 (fp64 sums on both sides, in
# different orders).
NEAR_TIE_ACCEPT = 1e-6
NEAR_TIE_CDF = 1e-11
NEAR_TIE_FILTER = 1e-11
PROB_RTOL = 1e-5
RESID_RTOL = 1e-9
MAX_NEAR_FRACTION = 1e-4

THREADS = max(1, min(16, os.cpu_count() or 1))


def f32(x: float) -> float:
    """x rounded to binary32 (how the C ABI carries temperature and top_p)."""
    return float(np.float32(x))


def to_dev(a: np.ndarray) -> torch.Tensor:
    """numpy float32 -> float32 device tensor; uint16 (bfloat16 bits) -> bfloat16."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def np_of(x):
    return x.cpu().numpy() if isinstance(x, torch.Tensor) else np.asarray(x)


class Tally:
    """Decisions taken by the oracle, near ties among them, excused requests."""

    def __init__(self, name: str = ""):
        self.name = name
        self.decisions = 0
        self.near = 0
        self.excused = 0
        self.requests = 0

    def __iadd__(self, o: "Tally"):
        self.decisions += o.decisions
        self.near += o.near
        self.excused += o.excused
        self.requests += o.requests
        return self

    def report(self) -> str:
        frac = self.near / max(self.decisions, 1)
        return (f"[parity {self.name}] requests {self.requests}, decisions {self.decisions}, near ties {self.near} "
                f"({frac:.2e}), excused {self.excused}")

    def check(self, near_fraction: bool = False) -> "Tally":
        """Excused requests within max(1, 1e-4 of the decisions) (and never
        more than the near ties); with near_fraction, near ties themselves
        below 1e-4 of the decisions."""
        print(self.report(), flush=True)
        assert self.excused <= self.near, self.report()
        assert self.excused <= max(1, math.floor(MAX_NEAR_FRACTION * self.decisions)), self.report()
        if near_fraction:
            assert self.near < MAX_NEAR_FRACTION * self.decisions, self.report()
        return self


def _first_diff(a, b) -> int:
    d = np.nonzero(np.asarray(a) != np.asarray(b))[0]
    return int(d[0]) if d.size else -1


def compare_linear(g: dict, o: dict, fused: bool = False, acc_band: float = NEAR_TIE_ACCEPT,
                   cdf_band: float = NEAR_TIE_CDF, check_probs: bool = True, check_resid: bool = True,
                   name: str = "") -> Tally:
    """Compare GPU outputs (torch) of a linear verification with the oracle's
    (numpy), request by request, under the excuse rule above. Probabilities
    must agree within PROB_RTOL and residual masses within RESID_RTOL wherever
    the decisions they depend on agree."""
    gl, gt = np_of(g["len"]), np_of(g["tokens"])
    gd = np_of(g["draft"]) if fused else None
    ol, ot, od = o["len"], o["tokens"], o["draft"]
    K = ot.shape[1] - 1
    t = Tally(name)
    t.requests = len(ol)
    gp = np_of(g["probs"]).astype(np.float64) if (check_probs and g.get("probs") is not None) else None
    gr = np_of(g["resid"]) if (check_resid and g.get("resid") is not None) else None
    for b in range(len(ol)):
        if ol[b] < 0:
            assert gl[b] == -1 and np.all(gt[b] == -1), f"request {b}: oracle error, gpu len {gl[b]}"
            if fused:
                assert np.all(gd[b] == -1), f"request {b}: drafts of an invalid request must be -1"
            continue
        ma, md, mf, mfl = o["m_acc"][b], o["m_draft"][b], o["m_final"][b], o["m_filter"][b]
        # decisions taken and near ties among them
        t.decisions += int(np.isfinite(ma).sum()) + int(np.isfinite(md).sum()) + int(np.isfinite(mf))
        t.near += int((ma < acc_band).sum()) + int((md < cdf_band).sum()) + int(mf < cdf_band)
        if np.isfinite(mfl):
            t.decisions += 2 * K + 1
            t.near += int(mfl < NEAR_TIE_FILTER)
        drafts_same = (not fused) or np.array_equal(gd[b], od[b])
        same = drafts_same and gl[b] == ol[b] and np.array_equal(gt[b], ot[b])
        if not same:
            msg = (f"request {b}: gpu len {gl[b]} tokens {gt[b].tolist()}"
                   + (f" drafts {gd[b].tolist()}" if fused else "")
                   + f" vs oracle len {ol[b]} tokens {ot[b].tolist()} drafts {od[b].tolist()}; margins acc "
                   f"{ma.tolist()} draft {md.tolist()} final {mf:.3g} filter {mfl:.3g}")
            if mfl < NEAR_TIE_FILTER:
                pass  # a row's top-p cut may have parted first
            elif not drafts_same:
                i = _first_diff(gd[b], od[b])
                assert md[i] < cdf_band and gd[b, i] == o["alt_draft"][b, i], "first difference: draft " + \
                    f"{i}; " + msg
            elif gl[b] != ol[b]:
                i = min(int(gl[b]), int(ol[b]))
                assert ma[i] < acc_band, f"first difference: accept test {i}; " + msg
            else:
                n = int(ol[b])
                assert mf < cdf_band and gt[b, n] == o["alt_final"][b], "first difference: final draw; " + msg
            t.excused += 1
        if mfl < NEAR_TIE_FILTER or not drafts_same:
            continue
        if gp is not None:
            err = np.abs(gp[b] - o["probs"][b])
            tol = PROB_RTOL * np.abs(o["probs"][b]) + 2e-38
            assert np.all(err <= tol), f"request {b}: probs {gp[b].tolist()} vs {o['probs'][b].tolist()}"
        if gr is not None and same:
            assert abs(gr[b] - o["resid"][b]) <= RESID_RTOL * abs(o["resid"][b]) + 1e-15, \
                f"request {b}: resid {gr[b]} vs {o['resid'][b]}"
    return t


def compare_drafts(g_tokens, o_tokens, om: dict, name: str = "") -> Tally:
    """Draft draws (psispec_draft_sample or tree node drafts) against the
    oracle's, each draw on its own: equal, or an oracle near tie (its row's
    top-p cut, or the draw itself with the GPU on the token across the near
    edge)."""
    gx, ox = np_of(g_tokens), np.asarray(o_tokens)
    t = Tally(name)
    t.requests = gx.shape[0]
    cdf, alt, flt = om["cdf"], om["alt"], om["filter"]
    t.decisions = int(np.isfinite(cdf).sum()) + int(np.isfinite(flt).sum())
    t.near = int((cdf < NEAR_TIE_CDF).sum()) + int((flt < NEAR_TIE_FILTER).sum())
    for idx in zip(*np.nonzero(gx != ox)):
        ok = flt[idx] < NEAR_TIE_FILTER or (cdf[idx] < NEAR_TIE_CDF and gx[idx] == alt[idx])
        assert ok, f"draft {idx}: gpu {gx[idx]} vs oracle {ox[idx]} (margin {cdf[idx]:.3g}, alt {alt[idx]})"
        t.excused += 1
    return t


def compare_tree(g: dict, o: dict, acc_band: float = NEAR_TIE_ACCEPT, cdf_band: float = NEAR_TIE_CDF,
                 name: str = "") -> Tally:
    """Tree outputs (linear-rule tree or deterministic candidates): len, path
    and tokens identical per request, except under the excuse rule: where the
    paths part, the first child test that can differ (the lower node id of
    the two children accepted, none counting as after every child) must be a
    near tie; with equal paths, the final draw must be one, the GPU on the
    token across its nearer edge."""
    gl, gt, gp = np_of(g["len"]), np_of(g["tokens"]), np_of(g["path"])
    ol, ot, op = o["len"], o["tokens"], o["path"]
    t = Tally(name)
    t.requests = len(ol)
    for b in range(len(ol)):
        if ol[b] < 0:
            assert gl[b] == -1 and np.all(gt[b] == -1), f"request {b}: oracle error, gpu len {gl[b]}"
            continue
        ma, mf, mfl = o["m_acc"][b], o["m_final"][b], o["m_filter"][b]
        t.decisions += int(np.isfinite(ma).sum()) + int(np.isfinite(mf)) + int(np.isfinite(mfl))
        t.near += int((ma < acc_band).sum()) + int(mf < cdf_band) + int(mfl < NEAR_TIE_FILTER)
        if gl[b] == ol[b] and np.array_equal(gt[b], ot[b]) and np.array_equal(gp[b], op[b]):
            continue
        msg = (f"request {b}: gpu len {gl[b]} path {gp[b].tolist()} tokens {gt[b].tolist()} vs oracle len {ol[b]} "
               f"path {op[b].tolist()} tokens {ot[b].tolist()}")
        if mfl < NEAR_TIE_FILTER:
            t.excused += 1
            continue
        L = max(int(gl[b]), int(ol[b]))
        k = next((i for i in range(L + 1) if (gp[b, i] if i < gl[b] else -1) != (op[b, i] if i < ol[b] else -1)), -1)
        if k >= 0:
            cg = int(gp[b, k]) if k < gl[b] else -1
            co = int(op[b, k]) if k < ol[b] else -1
            c = min(x for x in (cg, co) if x >= 0)
            assert ma[c] < acc_band, f"first difference: test of node {c} (margin {ma[c]:.3g}); " + msg
        else:
            n = int(ol[b])
            assert mf < cdf_band and gt[b, n] == o["alt_final"][b], \
                f"first difference: final draw (margin {mf:.3g}, alt {o['alt_final'][b]}); " + msg
        t.excused += 1
    return t
