"""Helpers for the oracle tests: independent reference quantities and exact
enumeration of the oracle's decisions by bisection over its uniforms.

The reference quantities here use scipy's softmax (an independent library
implementation of the softmax definition); the enumeration treats the oracle as
a black box driven through its uniform-override input.
"""
from __future__ import annotations

import ctypes

import numpy as np
from scipy.special import softmax

import oracle


def probs(a, temperature=1.0):
    return softmax(np.asarray(a, dtype=np.float64) / temperature)


def alpha(P, Q):
    """Acceptance probability of one position: sum_j min(P_j, Q_j)."""
    return float(np.minimum(P, Q).sum())


def residual(P, Q):
    w = np.maximum(P - Q, 0.0)
    s = w.sum()
    return w / s if s > 0 else P.copy()


class FastLinear:
    """Repeated oracle linear-verify calls on fixed logits with uniform overrides."""

    def __init__(self, p, q, temperature=1.0, top_k=0, top_p=1.0):
        self.p = np.ascontiguousarray(p)
        self.q = np.ascontiguousarray(q)
        self.B, K1, self.V = self.p.shape
        self.K = K1 - 1
        self.T, self.top_k, self.top_p = float(temperature), int(top_k), float(top_p)
        self.draft = np.zeros((self.B, self.K), dtype=np.int32)
        self.toks = np.zeros((self.B, self.K + 1), dtype=np.int32)
        self.len = np.zeros(self.B, dtype=np.int32)
        self.ovr = np.zeros((self.B, self.K + 1, 3), dtype=np.float64)
        self.dtype = oracle._dtype_code(self.p)
        self._args = None

    def run(self, draft, ovr):
        self.draft[...] = np.asarray(draft, dtype=np.int32).reshape(self.B, self.K)
        self.ovr[...] = ovr
        P = ctypes.c_void_p
        rc = oracle.lib().orc_verify_linear(
            self.p.ctypes.data_as(P), self.q.ctypes.data_as(P), self.dtype, self.B, self.K, self.V,
            self.draft.ctypes.data_as(P), self.T, self.top_k, self.top_p, 0, 0, 0,
            self.toks.ctypes.data_as(P), self.len.ctypes.data_as(P), None, None, None,
            self.ovr.ctypes.data_as(P), 1)
        assert rc == 0
        n = int(self.len[0])
        return n, tuple(int(t) for t in self.toks[0, :n + 1])


def threshold(pred, lo=0.0, hi=1.0, iters=60):
    """For pred monotone True->False on [lo, hi): the switch point."""
    if not pred(lo):
        return lo
    if pred(np.nextafter(hi, 0.0)):
        return hi
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if pred(mid):
            lo = mid
        else:
            hi = mid
        if hi - lo < 1e-16:
            break
    return 0.5 * (lo + hi)


def step_measure(f, a=0.0, b=None, tol=1e-15):
    """Measure of each value of a monotone step function f on [a, b)."""
    if b is None:
        b = np.nextafter(1.0, 0.0)
    out: dict = {}

    def rec(lo, hi, flo, fhi):
        if flo == fhi:
            out[flo] = out.get(flo, 0.0) + (hi - lo)
            return
        if hi - lo < tol:
            out[flo] = out.get(flo, 0.0) + 0.5 * (hi - lo)
            out[fhi] = out.get(fhi, 0.0) + 0.5 * (hi - lo)
            return
        mid = 0.5 * (lo + hi)
        fm = f(mid)
        rec(lo, mid, flo, fm)
        rec(mid, hi, fm, fhi)

    rec(a, b, f(a), f(b))
    total = sum(out.values())
    return {k: v / total for k, v in out.items()}


def chi2_pvalue(counts, expected, min_expected=5.0):
    """Pearson chi-square p-value, merging cells whose expectation is < min_expected."""
    from scipy.stats import chi2

    counts = np.asarray(counts, dtype=np.float64)
    expected = np.asarray(expected, dtype=np.float64)
    order = np.argsort(expected)
    c_m, e_m = [], []
    acc_c = acc_e = 0.0
    for i in order:
        acc_c += counts[i]
        acc_e += expected[i]
        if acc_e >= min_expected:
            c_m.append(acc_c)
            e_m.append(acc_e)
            acc_c = acc_e = 0.0
    if acc_e > 0:
        if e_m:
            c_m[-1] += acc_c
            e_m[-1] += acc_e
        else:
            c_m.append(acc_c)
            e_m.append(acc_e)
    c_m = np.array(c_m)
    e_m = np.array(e_m)
    if len(c_m) < 2:
        return 1.0
    stat = float(((c_m - e_m) ** 2 / e_m).sum())
    return float(chi2.sf(stat, len(c_m) - 1))


class FastTree:
    """Repeated oracle tree-verify calls on fixed logits with uniform overrides."""

    def __init__(self, p, q, parent, max_children, temperature=1.0):
        self.p = np.ascontiguousarray(p)
        self.q = np.ascontiguousarray(q)
        self.B, R, self.V = self.p.shape
        self.N = R - 1
        self.parent = np.ascontiguousarray(parent, dtype=np.int32)
        self.D = oracle.tree_depth(self.parent)
        self.maxC = int(max_children)
        self.T = float(temperature)
        self.tokens = np.zeros((self.B, self.N), dtype=np.int32)
        self.otok = np.zeros((self.B, self.D + 1), dtype=np.int32)
        self.opath = np.zeros((self.B, self.D), dtype=np.int32)
        self.olen = np.zeros(self.B, dtype=np.int32)
        self.ovr = np.zeros((self.B, R, 1 + self.maxC), dtype=np.float64)
        self.dtype = oracle._dtype_code(self.p)

    def run(self, tokens, ovr):
        self.tokens[...] = np.asarray(tokens, dtype=np.int32).reshape(self.B, self.N)
        self.ovr[...] = ovr
        P = ctypes.c_void_p
        rc = oracle.lib().orc_verify_tree(
            self.p.ctypes.data_as(P), self.q.ctypes.data_as(P), self.dtype, self.B, self.N, self.V,
            self.parent.ctypes.data_as(P), self.tokens.ctypes.data_as(P), self.T, 0, 1.0, 0, 0,
            self.otok.ctypes.data_as(P), self.opath.ctypes.data_as(P), self.olen.ctypes.data_as(P), None,
            self.ovr.ctypes.data_as(P), self.maxC, 1)
        assert rc == 0
        n = int(self.olen[0])
        return n, tuple(int(t) for t in self.otok[0, :n + 1]), tuple(int(x) for x in self.opath[0, :n])


class FastDetTree:
    """Repeated oracle calls of the verification of deterministic candidates
    (one request) on fixed logits and tree, with uniform overrides."""

    def __init__(self, p, parent, max_children, temperature=1.0):
        self.p = np.ascontiguousarray(p)
        _, R, self.V = self.p.shape
        self.N = R - 1
        self.parent = np.ascontiguousarray(parent, dtype=np.int32).reshape(1, self.N)
        self.maxC = int(max_children)
        self.T = float(temperature)
        self.tokens = np.zeros((1, self.N), dtype=np.int32)
        self.otok = np.zeros((1, self.N + 1), dtype=np.int32)
        self.opath = np.zeros((1, self.N), dtype=np.int32)
        self.olen = np.zeros(1, dtype=np.int32)
        self.ovr = np.zeros((1, R, 1 + self.maxC), dtype=np.float64)
        self.dtype = oracle._dtype_code(self.p)

    def run(self, tokens, ovr):
        self.tokens[...] = np.asarray(tokens, dtype=np.int32).reshape(1, self.N)
        self.ovr[...] = ovr
        P = ctypes.c_void_p
        rc = oracle.lib().orc_verify_tree_det(
            self.p.ctypes.data_as(P), self.dtype, 1, self.N, self.V, self.parent.ctypes.data_as(P),
            self.tokens.ctypes.data_as(P), self.T, 0, 0, self.otok.ctypes.data_as(P), self.opath.ctypes.data_as(P),
            self.olen.ctypes.data_as(P), None, self.ovr.ctypes.data_as(P), self.maxC, 1)
        assert rc == 0
        n = int(self.olen[0])
        return n, tuple(int(t) for t in self.otok[0, :n + 1]), tuple(int(x) for x in self.opath[0, :n])
