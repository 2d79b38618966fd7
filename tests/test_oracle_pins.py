"""Pins of the CPU oracle against facts fixed outside the oracle itself:
published known-answer vectors, closed forms, the textbook law of speculative
sampling, brute force on tiny inputs and exact enumeration of every random
branch. A plausible mistake in the oracle (a dropped term, a wrong sign or
index, a transposed operand, an off-by-one in the prefix) fails one of these.
"""
from __future__ import annotations

import itertools
import os

import numpy as np
import pytest
from scipy.special import logsumexp as sp_logsumexp

import oracle
import synth
from oracle_helpers import (FastDetTree, FastLinear, FastTree, alpha, chi2_pvalue, probs, residual, step_measure,
                            threshold)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- Philox --
def test_philox_known_answers():
    """Published Philox4x32-10 known-answer vectors (tests/golden)."""
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([int(w, 16) for w in line.split()])
    assert len(rows) == 3
    for r in rows:
        out = oracle.philox4x32_10(r[0:4], r[4:6])
        assert [int(x) for x in out] == r[6:10]


def test_uniform_layout_and_range():
    """U(seed, step, b, r, d) = word0 / 2^32 of Philox with counter (d, r, b, step)
    and key (lo32 seed, hi32 seed)."""
    seed = 0x0123456789ABCDEF
    for (step, b, r, d) in [(0, 0, 0, 0), (7, 3, 2, 1), (999, 255, 8, 0x40000000), (1, 2, 3, 4)]:
        w = oracle.philox4x32_10([d, r, b, step], [seed & 0xFFFFFFFF, seed >> 32])
        u = oracle.uniform(seed, step, b, r, d)
        assert u == int(w[0]) / 2.0 ** 32
        assert 0.0 <= u < 1.0


def test_uniform_chi_square():
    """The uniforms are uniform: chi-square over 64 bins of 2^17 draws."""
    n = 1 << 17
    us = np.array([oracle.uniform(0, 5, i & 0xFF, i >> 8, 1) for i in range(n)])
    counts = np.bincount((us * 64).astype(int), minlength=64)
    assert chi2_pvalue(counts, np.full(64, n / 64)) > 1e-3


# ------------------------------------------------------------- normaliser --
def test_logsumexp_closed_forms():
    V = 1000
    assert abs(oracle.logsumexp(np.full(V, 3.25)) - (3.25 + np.log(V))) < 1e-13
    z = np.full(17, -np.inf)
    z[5] = -2.5
    assert oracle.logsumexp(z) == -2.5
    assert oracle.logsumexp(np.array([0.0, np.log(3.0)])) == pytest.approx(np.log(4.0), abs=1e-15)
    assert oracle.logsumexp(np.full(4, -np.inf)) == -np.inf
    # far-apart values: no overflow, exact dominant term
    assert oracle.logsumexp(np.array([1000.0, 0.0])) == pytest.approx(1000.0 + np.log1p(np.exp(-1000.0)), abs=1e-12)


def test_logsumexp_against_library():
    rng = np.random.default_rng(3)
    for V in (1, 7, 1024, 151936):
        z = rng.normal(0, 3, V)
        ref = sp_logsumexp(z)
        assert abs(oracle.logsumexp(z) - ref) <= 1e-14 * max(1.0, abs(ref)) * max(1.0, np.log2(V))


# ----------------------------------------------------------- inverse CDF --
def test_sample_brute_force_grid():
    """Sweeping u over a fine grid reproduces w / W; zero weights are never drawn."""
    w = np.array([0.0, 0.3, 0.0, 1.2, 0.5, 0.0, 2.0, 0.0])
    G = 1 << 16
    counts = np.zeros_like(w)
    for k in range(G):
        j = oracle.sample(w, (k + 0.5) / G)[0]
        counts[j] += 1
    assert np.all(counts[w == 0] == 0)
    assert np.max(np.abs(counts / G - w / w.sum())) <= 1.0 / G


def test_sample_edges_and_margin():
    w = np.array([0.0, 1.0, 3.0])
    assert oracle.sample(w, 0.0)[0] == 1  # smallest j with C_j > 0
    j, m, _ = oracle.sample(w, 0.25)  # t = 1.0 = C_1 exactly -> next token
    assert j == 2 and m == 0.0
    j, m, _ = oracle.sample(w, 0.5)  # t = 2.0, inside [1, 4): margin min(1, 2)/4
    assert j == 2 and m == pytest.approx(0.25)
    assert oracle.sample(np.zeros(3), 0.5)[0] == -1


def test_sample_rounding_fallback():
    """If rounding leaves no C_j > u*W the largest positive-weight id is returned."""
    w = np.array([1e-300, 1.0, 0.0])
    j = oracle.sample(w, np.nextafter(1.0, 0.0))[0]
    assert j == 1


# ----------------------------------------------------------------- filters --
def _brute_filter(a, T, top_k, top_p):
    z = np.asarray(a, dtype=np.float64) / T
    V = len(z)
    keep = np.ones(V, dtype=bool)
    if 0 < top_k < V:
        order = sorted(range(V), key=lambda j: (-z[j], j))
        keep[:] = False
        keep[order[:top_k]] = True
    if top_p < 1.0:
        idx = [j for j in range(V) if keep[j] and np.isfinite(z[j])]
        m = max(z[j] for j in idx)
        e = {j: np.exp(z[j] - m) for j in idx}
        s = 0.0
        for j in idx:
            s += e[j]
        pr = {j: e[j] / s for j in idx}
        order = sorted(idx, key=lambda j: (-pr[j], j))
        cum, cnt = 0.0, len(order)
        for t, j in enumerate(order):
            cum += pr[j]
            if cum >= top_p:
                cnt = t + 1
                break
        kept = set(order[:cnt])
        keep = np.array([j in kept for j in range(V)])
    out = z.copy()
    out[~keep] = -np.inf
    return out


@pytest.mark.parametrize("seed", range(6))
def test_filters_brute_force(seed):
    rng = np.random.default_rng(seed)
    V = 40
    a = np.round(rng.normal(0, 2, V), 1)  # rounding makes ties
    for (T, k, pp) in [(1.0, 5, 1.0), (0.7, 0, 0.6), (1.3, 12, 0.9), (1.0, 1, 0.5), (2.0, 39, 0.99), (1.0, 3, 0.2)]:
        got = oracle.filter_row(a, T, k, pp)
        ref = _brute_filter(a, T, k, pp)
        assert np.array_equal(np.isfinite(got), np.isfinite(ref))
        assert np.array_equal(got[np.isfinite(got)], ref[np.isfinite(ref)])


def test_filter_disabled_is_identity():
    rng = np.random.default_rng(1)
    a = rng.normal(0, 3, 500)
    for k in (0, 500, 10_000):
        z = oracle.filter_row(a, 0.7, k, 1.0)
        assert np.array_equal(z, a / 0.7)


def test_top_k_ties_lower_id():
    a = np.array([1.0, 3.0, 2.0, 3.0, 3.0])
    z = oracle.filter_row(a, 1.0, 2, 1.0)
    assert list(np.isfinite(z)) == [False, True, False, True, False]


# ------------------------------------------------- single-position pins --
def _tiny_pair(seed, V=8, K=2, sd=1.5, noise=1.0):
    rng = np.random.default_rng(seed)
    a = rng.normal(0, sd, (1, K + 1, V))
    d = a[:, :K] + rng.normal(0, noise, (1, K, V))
    return a.astype(np.float32), d.astype(np.float32)


@pytest.mark.parametrize("seed", range(3))
def test_accept_probability_is_min_ratio(seed):
    """Bisection on the accept uniform recovers min(1, P(x)/Q(x)) for every x,
    and the draft-averaged acceptance equals sum min(P, Q) = 1 - TV(P, Q)."""
    p, q = _tiny_pair(seed, K=1)
    P, Q = probs(p[0, 0]), probs(q[0, 0])
    fl = FastLinear(p, q)
    acc = 0.0
    for x in range(8):
        def accepted(u):
            ovr = np.zeros((1, 2, 3))
            ovr[0, 0, 1] = u
            return fl.run([x], ovr)[0] == 1
        r = threshold(accepted)
        assert abs(r - min(1.0, P[x] / Q[x])) < 1e-12
        acc += Q[x] * r
    assert abs(acc - alpha(P, Q)) < 1e-12
    assert abs(acc - (1.0 - 0.5 * np.abs(P - Q).sum())) < 1e-12


@pytest.mark.parametrize("seed", range(3))
def test_residual_mass_identity(seed):
    """The reported residual mass is sum (P - Q)+ = 1 - alpha."""
    p, q = _tiny_pair(seed, V=64, K=3)
    draft = np.array([[int(np.argmin(probs(p[0, i]) / probs(q[0, i]))) for i in range(3)]], dtype=np.int32)
    r = oracle.verify_linear(p, q, draft, 1.0, seed=seed)
    n = int(r["len"][0])
    assert n < 3  # the draft with the smallest ratio is rejected with high probability
    P, Q = probs(p[0, n]), probs(q[0, n])
    assert abs(r["resid"][0] - (1.0 - alpha(P, Q))) < 1e-12


# ------------------------------------------- exact enumeration, K=2, V=8 --
@pytest.mark.parametrize("seed", [0, 1])
def test_linear_exact_enumeration(seed):
    """Every random branch of the oracle (all 64 draft pairs, accept tests,
    residual and bonus draws) enumerated exactly: the joint law of the emitted
    block equals the speculative-sampling law, and the first emitted token
    follows the target distribution exactly (losslessness)."""
    V, K = 8, 2
    p, q = _tiny_pair(seed, V=V, K=K)
    P = [probs(p[0, i]) for i in range(K + 1)]
    Q = [probs(q[0, i]) for i in range(K)]
    fl = FastLinear(p, q)
    HI = np.nextafter(1.0, 0.0)
    law: dict = {}
    for x0, x1 in itertools.product(range(V), range(V)):
        wx = Q[0][x0] * Q[1][x1]

        def run(ua0, ua1, uf):
            ovr = np.zeros((1, K + 1, 3))
            ovr[0, :, 1] = [ua0, ua1, 0.0]
            ovr[0, :, 0] = uf
            return fl.run([x0, x1], ovr)

        r0 = threshold(lambda u: run(u, 0.0, 0.5)[0] >= 1)
        r1 = threshold(lambda u: run(0.0, u, 0.5)[0] >= 2)
        branches = []
        if r0 < 1.0:
            branches.append((1.0 - r0, HI, 0.0))
        if r0 > 0.0 and r1 < 1.0:
            branches.append((r0 * (1.0 - r1), 0.0, HI))
        if r0 > 0.0 and r1 > 0.0:
            branches.append((r0 * r1, 0.0, 0.0))
        for (wb, ua0, ua1) in branches:
            meas = step_measure(lambda u: run(ua0, ua1, u)[1])
            for out, m in meas.items():
                law[out] = law.get(out, 0.0) + wx * wb * m
    assert abs(sum(law.values()) - 1.0) < 1e-12
    a0, a1 = alpha(P[0], Q[0]), alpha(P[1], Q[1])
    R0, R1 = residual(P[0], Q[0]), residual(P[1], Q[1])
    M0, M1 = np.minimum(P[0], Q[0]), np.minimum(P[1], Q[1])
    expect = {}
    for y in range(V):
        expect[(y,)] = (1 - a0) * R0[y]
    for v, y in itertools.product(range(V), range(V)):
        expect[(v, y)] = M0[v] * (1 - a1) * R1[y]
    for v, w_, y in itertools.product(range(V), range(V), range(V)):
        expect[(v, w_, y)] = M0[v] * M1[w_] * P[2][y]
    for k in set(law) | set(expect):
        assert abs(law.get(k, 0.0) - expect.get(k, 0.0)) < 1e-12, k
    first = np.zeros(V)
    for out, m in law.items():
        first[out[0]] += m
    assert np.max(np.abs(first - P[0])) < 1e-12
    # given that the first draft was accepted, the next token follows P[1]
    second = np.zeros(V)
    for out, m in law.items():
        if len(out) >= 2:
            second[out[1]] += m
    assert np.max(np.abs(second / second.sum() - P[1])) < 1e-12


# -------------------------------------------------- multi-round AR chain --
def _toy_logits(prefix, which, pos=0):
    code = 1
    for t in prefix:
        code = code * 9 + (t + 1)
    stream = code * 64 + pos * 2 + which
    return 1.6 * synth.normal(7, stream, 8)


def test_multi_round_toy_chain_lossless():
    """Full draft -> verify -> commit rounds on a toy AR model (V=8, 3 tokens):
    the law of the generated sequence equals prod_l p(y_l | y_<l) (chi-square
    over the 512 sequences)."""
    V, L, K = 8, 3, 2
    pcache: dict = {}

    def p_logits(prefix):
        key = tuple(prefix)
        if key not in pcache:
            pcache[key] = _toy_logits(prefix, 0)
        return pcache[key]

    def q_logits(prefix, i):
        return p_logits(list(prefix) + [0] * i) + 0.8 * _toy_logits(prefix, 1, i)

    runs = 12000
    counts = np.zeros(V ** L)
    for run in range(runs):
        s: list = []
        rnd = 0
        while len(s) < L:
            q = np.array([[q_logits(s, i) for i in range(K)]], dtype=np.float32)
            x, _ = oracle.draft_sample(q, 1.0, seed=run, step=rnd)
            p = np.array([[p_logits(s + list(x[0, :i])) for i in range(K + 1)]], dtype=np.float32)
            r = oracle.verify_linear(p, q, x, 1.0, seed=run, step=rnd)
            n = int(r["len"][0])
            s += [int(t) for t in r["tokens"][0, :n + 1]]
            rnd += 1
        y = s[:L]
        counts[(y[0] * V + y[1]) * V + y[2]] += 1
    expected = np.zeros(V ** L)
    for y in itertools.product(range(V), repeat=L):
        pr = 1.0
        for l in range(L):
            pr *= probs(np.float32(p_logits(list(y[:l]))).astype(np.float64))[y[l]]
        expected[(y[0] * V + y[1]) * V + y[2]] = pr * runs
    assert abs(expected.sum() - runs) < 1e-6 * runs
    assert chi2_pvalue(counts, expected) > 1e-3


# --------------------------------------------------- tiny workload laws --
def test_accept_length_law_tiny_workload():
    """Tiny workload, 2000 trials with fused drafts: the accept-length histogram
    follows P(n=k) = prod_{j<k} alpha_j (1 - alpha_k), P(n=K) = prod alpha_j;
    the first emitted token follows P_0; emitted per call is in [1, K+1]."""
    p, q = synth.linear_inputs("tiny", seed=0)
    K = q.shape[1]
    T = 1.0
    P = [probs(p[0, i], T) for i in range(K + 1)]
    Q = [probs(q[0, i], T) for i in range(K)]
    al = [alpha(P[i], Q[i]) for i in range(K)]
    law = []
    for k in range(K + 1):
        pr = np.prod(al[:k])
        law.append(pr * (1 - al[k]) if k < K else pr)
    trials = 2000
    hist = np.zeros(K + 1)
    first = np.zeros(p.shape[2])
    for t in range(trials):
        r = oracle.verify_linear(p, q, None, T, seed=0, step=t, fused=True)
        n = int(r["len"][0])
        assert 0 <= n <= K
        assert np.all(r["tokens"][0, :n] == r["draft"][0, :n])
        assert np.all(r["tokens"][0, n + 1:] == -1)
        hist[n] += 1
        first[r["tokens"][0, 0]] += 1
    assert chi2_pvalue(hist, np.array(law) * trials) > 1e-3
    assert chi2_pvalue(first, P[0] * trials) > 1e-3


def test_draft_sample_law():
    """Draft draws follow softmax(q / T): chi-square over 3000 steps."""
    rng = np.random.default_rng(5)
    q = rng.normal(0, 1.0, (1, 2, 16)).astype(np.float32)
    T = 0.7
    c = np.zeros((2, 16))
    for t in range(3000):
        x, _ = oracle.draft_sample(q, T, seed=9, step=t)
        c[0, x[0, 0]] += 1
        c[1, x[0, 1]] += 1
    for i in range(2):
        assert chi2_pvalue(c[i], probs(q[0, i], T) * 3000) > 1e-3


# ------------------------------------------------------ special cases --
def test_identical_rows_always_accept():
    """q_i == p_i: the ratio is exactly 1, so the position is always accepted
    (the AR-only first block position is such a row)."""
    p, _ = synth.linear_inputs("tiny", seed=3)
    q = np.ascontiguousarray(p[:, :4])
    for t in range(200):
        r = oracle.verify_linear(p, q, None, 1.0, seed=1, step=t, fused=True)
        assert r["len"][0] == 4
        assert np.all(r["probs"][0, :, 0] == r["probs"][0, :, 1])


def test_disjoint_supports_never_accept():
    """Disjoint supports: alpha = 0, every draft is rejected and y ~ P_0."""
    V = 16
    a = np.full((1, 3, V), -np.inf, dtype=np.float32)
    d = np.full((1, 2, V), -np.inf, dtype=np.float32)
    a[:, :, :8] = np.random.default_rng(0).normal(0, 1, (1, 3, 8))
    d[:, :, 8:] = np.random.default_rng(1).normal(0, 1, (1, 2, 8))
    P0 = probs(a[0, 0])
    first = np.zeros(V)
    for t in range(3000):
        r = oracle.verify_linear(a, d, None, 1.0, seed=2, step=t, fused=True)
        assert r["len"][0] == 0
        assert r["resid"][0] == pytest.approx(1.0, abs=1e-15)
        first[r["tokens"][0, 0]] += 1
    assert np.all(first[8:] == 0)
    assert chi2_pvalue(first[:8], P0[:8] * 3000) > 1e-3


def test_greedy_rules():
    """Temperature 0: accept iff the draft equals the target argmax (lowest id
    on ties); the final token is the target argmax of the stop row."""
    V, K = 10, 3
    a = np.zeros((1, K + 1, V), dtype=np.float32)
    a[0, 0, [2, 7]] = 5.0  # tie -> 2
    a[0, 1, 4] = 3.0
    a[0, 2, 9] = 1.0
    a[0, 3, 0] = 2.0
    d = np.zeros((1, K, V), dtype=np.float32)
    for drafts, n, y in [([2, 4, 9], 3, 0), ([2, 4, 1], 2, 9), ([7, 4, 9], 0, 2), ([2, 5, 9], 1, 4)]:
        r = oracle.verify_linear(a, d, np.array([drafts]), 0.0)
        assert r["len"][0] == n
        assert list(r["tokens"][0, :n + 1]) == drafts[:n] + [y]


def test_top_k_one_equals_greedy():
    """top_k = 1 stochastic sampling with fused drafts is greedy decoding."""
    p, q = synth.linear_inputs("tiny", seed=4)
    g = oracle.verify_linear(p, q, None, 0.0, fused=True)
    for t in range(20):
        s = oracle.verify_linear(p, q, None, 1.0, top_k=1, seed=3, step=t, fused=True)
        assert np.array_equal(s["tokens"], g["tokens"]) and np.array_equal(s["len"], g["len"])


def test_unfiltered_equivalences():
    """top_k = V, top_p = 1 is the unfiltered sampler, bit for bit."""
    p, q = synth.linear_inputs("tiny", seed=6)
    V = p.shape[2]
    for t in range(10):
        a = oracle.verify_linear(p, q, None, 0.9, seed=1, step=t, fused=True)
        b = oracle.verify_linear(p, q, None, 0.9, top_k=V, top_p=1.0, seed=1, step=t, fused=True)
        for k in ("tokens", "len", "probs", "resid"):
            assert np.array_equal(a[k], b[k])


def test_request_errors():
    p, q = synth.linear_inputs("tiny", seed=2, B=1)
    p = np.repeat(p, 5, axis=0)
    q = np.repeat(q, 5, axis=0)
    p[1, 4, 17] = np.nan  # NaN in the bonus row
    q[2, 0, 3] = np.inf  # +inf
    p[3, 2, :] = -np.inf  # all -inf row
    drafts = np.zeros((5, 4), dtype=np.int32)
    drafts[4, 1] = 1024  # out of range
    r = oracle.verify_linear(p, q, drafts, 1.0)
    assert list(r["len"]) [1:] == [-1, -1, -1, -1]
    assert r["len"][0] >= 0
    assert np.all(r["tokens"][1:] == -1)
    q2 = q.copy()
    q2[0, 1, :5] = -np.inf  # partial -inf is fine
    assert oracle.verify_linear(p[:1], q2[:1], drafts[:1], 1.0)["len"][0] >= 0


# --------------------------------------------------------------- tree --
def test_chain_tree_equals_linear():
    """A chain tree (node i's parent is i-1) gives bit-for-bit the linear
    verifier's output under the shared random-number layout."""
    pl, ql = synth.linear_inputs("tiny", seed=8, B=3)
    B, K1, V = pl.shape
    K = K1 - 1
    qt = np.concatenate([ql, ql[:, -1:]], axis=1)  # tree has a draft row for every context row
    parent = np.arange(-1, K - 1, dtype=np.int32)
    for t in range(40):
        lin = oracle.verify_linear(pl, ql, None, 1.0, seed=5, step=t, fused=True)
        tr = oracle.verify_tree(pl, qt, parent, lin["draft"], 1.0, seed=5, step=t)
        assert np.array_equal(tr["len"], lin["len"])
        assert np.array_equal(tr["tokens"], lin["tokens"])


def test_tree_root_candidates_exact():
    """Root with 3 i.i.d. candidates (V=8): enumerating every candidate triple
    (weights Q_root^3) and every uniform, the first emitted token follows P_root
    exactly; then, below an accepted child, enumerating the grandchild drawn from
    that child's draft row, the next token follows P of the child's row."""
    V = 8
    rng = np.random.default_rng(11)
    parent = np.array([-1, -1, -1, 0, 1, 2], dtype=np.int32)
    N = len(parent)
    a = rng.normal(0, 1.5, (1, N + 1, V)).astype(np.float32)
    d = (a + rng.normal(0, 1.0, (1, N + 1, V))).astype(np.float32)
    P = [probs(a[0, r]) for r in range(N + 1)]
    Q = [probs(d[0, r]) for r in range(N + 1)]
    HI = np.nextafter(1.0, 0.0)
    ft = FastTree(a, d, parent, max_children=3)

    def ovr_of(ua, uf_root, child_u=0.5, child_uf=0.5):
        o = np.zeros((1, N + 1, 4))
        o[0, 0, 1:4] = ua
        o[0, 0, 0] = uf_root
        o[0, 1:, 1] = child_u
        o[0, 1:, 0] = child_uf
        return o

    first = np.zeros(V)
    for c in itertools.product(range(V), repeat=3):
        wx = Q[0][c[0]] * Q[0][c[1]] * Q[0][c[2]]
        toks = [c[0], c[1], c[2], 0, 0, 0]
        def took(ua, node):
            path = ft.run(toks, ovr_of(ua, 0.5))[2]
            return len(path) >= 1 and path[0] == node
        r_a = threshold(lambda u: took([u, HI, HI], 0))
        r_b = threshold(lambda u: took([HI, u, HI], 1))
        r_c = threshold(lambda u: took([HI, HI, u], 2))
        first[c[0]] += wx * r_a
        first[c[1]] += wx * (1 - r_a) * r_b
        first[c[2]] += wx * (1 - r_a) * (1 - r_b) * r_c
        wr = (1 - r_a) * (1 - r_b) * (1 - r_c)
        if wr > 0:
            for t, m in step_measure(lambda u: ft.run(toks, ovr_of([HI, HI, HI], u))[1][0]).items():
                first[t] += wx * wr * m
    assert np.max(np.abs(first - P[0])) < 1e-12

    # second level below an accepted child 0 (row 1), grandchild node 3 ~ Q[1]
    c0 = int(np.argmax(P[0]))
    second = np.zeros(V)
    for g in range(V):
        toks = [c0, 0, 0, g, 0, 0]
        r_g = threshold(lambda u: ft.run(toks, ovr_of([0.0, HI, HI], 0.5, child_u=u))[0] >= 2)
        second[g] += Q[1][g] * r_g
        if r_g < 1:
            meas = step_measure(lambda u: ft.run(toks, ovr_of([0.0, HI, HI], 0.5, child_u=HI, child_uf=u))[1][1])
            for t, m in meas.items():
                second[t] += Q[1][g] * (1 - r_g) * m
    assert np.max(np.abs(second - P[1])) < 1e-12


def test_recursive_residual_closed_form():
    """The recursive update r <- norm(max(0, r - Q)) after j rejections equals
    (P - c_j Q)+ / G(c_j) with G(c) = sum max(0, P - c Q), c_0 = 0,
    c_{j+1} = c_j + G(c_j) (the form the GPU walk evaluates)."""
    rng = np.random.default_rng(2)
    for _ in range(20):
        V = 50
        P = probs(rng.normal(0, 2, V))
        Q = probs(rng.normal(0, 2, V))
        r = P.copy()
        c = 0.0
        for j in range(6):
            G = np.maximum(P - c * Q, 0).sum()
            assert np.max(np.abs(r - np.maximum(P - c * Q, 0) / G)) < 1e-12
            w = np.maximum(r - Q, 0)
            if w.sum() <= 0:
                break
            r = w / w.sum()
            c = c + G


def test_tree_depth_and_malformed():
    assert oracle.tree_depth(synth.branch_chain_parent(4, 8)) == 8
    assert oracle.tree_depth(np.array([-1, 0, 0, 1])) == 3
    assert oracle.tree_depth(np.array([-1, 2])) == -1
    assert oracle.tree_depth(np.array([0])) == -1


def test_tree_greedy():
    """Temperature 0: descend into the first child equal to the target argmax."""
    V = 6
    parent = np.array([-1, -1, 0, 1], dtype=np.int32)
    a = np.zeros((1, 5, V), dtype=np.float32)
    a[0, 0, 3] = 1.0  # root argmax 3
    a[0, 2, 5] = 1.0  # row of node 1: argmax 5
    d = np.zeros((1, 5, V), dtype=np.float32)
    r = oracle.verify_tree(a, d, parent, np.array([[1, 3, 4, 5]]), 0.0)
    assert r["len"][0] == 2 and list(r["path"][0]) == [1, 3] and list(r["tokens"][0]) == [3, 5, 0]
    r = oracle.verify_tree(a, d, parent, np.array([[1, 2, 4, 5]]), 0.0)
    assert r["len"][0] == 0 and list(r["tokens"][0]) == [3, -1, -1]


def test_tree_draft_chain_equals_linear_draft():
    """On a chain, node i is the only child of row i, so the tree drafts are the
    linear drafts of rows 0..K-1 (draw id 0x40000000 at every row)."""
    _, ql = synth.linear_inputs("tiny", seed=3, B=3)
    K = ql.shape[1]
    qt = np.concatenate([ql, ql[:, -1:]], axis=1)
    parent = np.arange(-1, K - 1, dtype=np.int32)
    for t in range(5):
        d, _ = oracle.draft_sample(ql, 1.0, seed=9, step=t)
        assert np.array_equal(oracle.tree_draft(qt, parent, 1.0, seed=9, step=t), d)


def test_tree_draft_brute_force():
    """Several children of one row: child j is the inverse-CDF pick of
    softmax(filter(q_r / T)) at U(seed, step, b, r, 0x40000000 + j), checked with
    a numpy cumulative sum; greedy gives the argmax; a bad row gives -1."""
    rng = np.random.default_rng(4)
    V = 300
    parent = np.array([-1, -1, -1, 0, 0, 2], dtype=np.int32)
    N = len(parent)
    q = rng.normal(0, 2.0, (2, N + 1, V)).astype(np.float32)
    rows = parent + 1
    sib = [int(np.sum(parent[:n] == parent[n])) for n in range(N)]
    for T, top_k in ((0.8, 0), (1.3, 17)):
        got = oracle.tree_draft(q, parent, T, top_k=top_k, seed=21, step=2)
        for b in range(2):
            for n in range(N):
                z = q[b, rows[n]].astype(np.float64) / T
                if top_k:
                    keep = np.argsort(-z, kind="stable")[:top_k]
                    zz = np.full(V, -np.inf)
                    zz[keep] = z[keep]
                    z = zz
                w = np.exp(z - z.max())
                u = oracle.uniform(21, 2, b, int(rows[n]), 0x40000000 + sib[n])
                want = int(np.argmax(np.cumsum(w) > u * w.sum()))
                assert got[b, n] == want
    g = oracle.tree_draft(q, parent, 0.0)
    assert np.array_equal(g, np.argmax(q[:, rows, :], axis=2))
    qb = q.copy()
    qb[1, 6, 5] = np.nan  # a leaf row: still makes the request invalid
    g = oracle.tree_draft(qb, parent, 1.0)
    assert np.all(g[1] == -1) and np.all(g[0] >= 0)


# ------------------------------------------- Tree Sampler (deterministic) --
def _brute_candidates(q, cands, nodes, T):
    """Every prefix over the top-`cands` tokens of each position, sorted by the
    recursive key (-log score, length, key of the parent, rank), first `nodes`."""
    K, V = q.shape
    z = q.astype(np.float64) / T
    lq = z - sp_logsumexp(z, axis=1, keepdims=True)
    ranks = [sorted(range(V), key=lambda j, i=i: (-z[i, j], j))[:cands] for i in range(K)]
    keys = {(): ()}
    score = {(): 0.0}
    items = []
    frontier = [()]
    for length in range(1, K + 1):
        nxt = []
        for pre in frontier:
            for r in range(cands):
                path = pre + (r,)
                score[path] = score[pre] + lq[length - 1, ranks[length - 1][r]]
                keys[path] = (-score[path], length, keys[pre], r)
                items.append(path)
                nxt.append(path)
        frontier = nxt
    items.sort(key=lambda p: keys[p])
    kept = items[:nodes]
    pos = {p: n for n, p in enumerate(kept)}
    parent = [pos[p[:-1]] if len(p) > 1 else -1 for p in kept]
    tokens = [ranks[len(p) - 1][p[-1]] for p in kept]
    return np.array(parent), np.array(tokens)


@pytest.mark.parametrize("K,cands,nodes,seed", [(3, 3, 10, 0), (4, 2, 12, 1), (2, 4, 9, 2), (3, 3, 27, 3),
                                                (5, 2, 20, 4)])
def test_tree_candidates_brute_force(K, cands, nodes, seed):
    """The best-first enumeration keeps exactly the first `nodes` prefixes of
    the stated order, as a sort of every prefix does."""
    rng = np.random.default_rng(seed)
    V = 7
    q = rng.normal(0.0, 2.0, (3, K, V)).astype(np.float32)
    par, tok, mg = oracle.tree_candidates(q, cands, nodes, 0.8)
    for b in range(3):
        bp, bt = _brute_candidates(q[b], cands, nodes, np.float64(0.8))
        assert np.array_equal(par[b], bp) and np.array_equal(tok[b], bt)
        assert np.all(mg[b] > 0.0)


def test_tree_candidates_special_cases():
    rng = np.random.default_rng(9)
    q = rng.normal(0.0, 2.0, (2, 4, 50)).astype(np.float32)
    # one position: its top tokens in order, all children of the root
    par, tok, _ = oracle.tree_candidates(q[:, :1], 6, 5, 1.0)
    for b in range(2):
        order = sorted(range(50), key=lambda j: (-q[b, 0, j], j))
        assert list(tok[b]) == order[:5] and list(par[b]) == [-1] * 5
    # one candidate per position: the chain of per-position argmaxes
    par, tok, _ = oracle.tree_candidates(q, 1, 4, 1.0)
    for b in range(2):
        assert list(par[b]) == [-1, 0, 1, 2]
        assert list(tok[b]) == [int(np.argmax(q[b, i])) for i in range(4)]
    # more nodes than prefixes exist: the rest are -1
    par, tok, _ = oracle.tree_candidates(q[:, :2], 2, 9, 1.0)
    assert (par[:, 6:] == -1).all() and (tok[:, 6:] == -1).all() and (par[:, :6] >= -1).all()
    # prefixes of probability zero are never kept: two finite tokens per position
    q2 = np.full((1, 2, 6), -np.inf, dtype=np.float32)
    q2[0, :, :2] = [[1.0, 0.5], [0.0, -1.0]]
    par, tok, _ = oracle.tree_candidates(q2, 4, 9, 1.0)
    # log scores: [0] -0.474, [0,0] -0.787, [1] -0.974, [1,0] -1.287, [0,1] -1.787, [1,1] -2.287
    assert list(par[0]) == [-1, 0, -1, 2, 0, 2, -1, -1, -1] and list(tok[0]) == [0, 0, 1, 0, 1, 1, -1, -1, -1]
    # invariants: parent before child, scores non-increasing
    par, tok, _ = oracle.tree_candidates(q, 8, 40, 0.7)
    z = q.astype(np.float64) / np.float64(0.7)
    lq = z - sp_logsumexp(z, axis=2, keepdims=True)
    for b in range(2):
        depth, sc = [], []
        for n in range(40):
            assert -1 <= par[b, n] < n
            d = 0 if par[b, n] < 0 else depth[par[b, n]] + 1
            depth.append(d)
            sc.append((0.0 if par[b, n] < 0 else sc[par[b, n]]) + lq[b, d, tok[b, n]])
        assert all(sc[n] >= sc[n + 1] - 1e-12 for n in range(39))


def test_tree_candidates_ties():
    """Equal logits: siblings are ordered by token id, and a parent's equal-score
    child comes after it (the kept set stays prefix-closed)."""
    q = np.zeros((1, 3, 5), dtype=np.float32)  # every token equally likely at every position
    par, tok, _ = oracle.tree_candidates(q, 2, 6, 1.0)
    bp, bt = _brute_candidates(q[0], 2, 6, np.float64(1.0))
    assert np.array_equal(par[0], bp) and np.array_equal(tok[0], bt)
    assert list(par[0]) == [-1, -1, 0, 0, 1, 1] and list(tok[0]) == [0, 1, 0, 1, 0, 1]


def test_tree_det_chain_equals_linear_point_mass():
    """A chain of deterministic candidates is linear verification with drafts
    that are point masses at those tokens: same decisions, same draws (the
    draw ids coincide), bit for bit."""
    rng = np.random.default_rng(5)
    B, K, V = 6, 4, 40
    p = rng.normal(0.0, 2.0, (B, K + 1, V)).astype(np.float32)
    toks = rng.integers(0, V, (B, K)).astype(np.int32)
    p[np.arange(B)[:, None], np.arange(K)[None, :], toks] += 6.0  # let many drafts be accepted
    q = np.full((B, K, V), -np.inf, dtype=np.float32)
    q[np.arange(B)[:, None], np.arange(K)[None, :], toks] = 0.0
    parent = np.tile(np.arange(-1, K - 1, dtype=np.int32), (B, 1))
    lens = []
    for step in range(8):
        for T in (1.0, 0.6):
            d = oracle.verify_tree_det(p, parent, toks, T, seed=3, step=step)
            lin = oracle.verify_linear(p, q, toks, T, seed=3, step=step)
            assert np.array_equal(d["len"], lin["len"])
            assert np.array_equal(d["tokens"][:, :K + 1], lin["tokens"])
            lens.extend(d["len"].tolist())
    assert len(set(lens)) >= 3


def test_tree_det_first_token_law():
    """Root with three deterministic candidates (one of them at a -inf logit):
    the first emitted token follows P_root, and after candidate c the next one
    follows the row of c (lossless, chi-square over 20,000 draws)."""
    rng = np.random.default_rng(11)
    V = 6
    p = rng.normal(0.0, 1.0, (1, 4, V)).astype(np.float32)
    p[0, 0, 5] = -np.inf
    parent = np.array([[-1, -1, -1]], dtype=np.int32)
    toks = np.array([[2, 0, 5]], dtype=np.int32)
    P0 = probs(p[0, 0])
    n = 20000
    first = np.zeros(V)
    second = {c: np.zeros(V) for c in range(3)}
    reps = 200
    pr = np.repeat(p, reps, axis=0)
    par = np.repeat(parent, reps, axis=0)
    tk = np.repeat(toks, reps, axis=0)
    for step in range(n // reps):
        o = oracle.verify_tree_det(pr, par, tk, 1.0, seed=7, step=step)
        for b in range(reps):
            first[o["tokens"][b, 0]] += 1
            if o["len"][b] == 1:
                second[o["path"][b, 0]][o["tokens"][b, 1]] += 1
    assert first[5] == 0
    assert chi2_pvalue(first, n * P0) > 1e-3
    for c in range(2):
        m = second[c].sum()
        assert m > 500
        assert chi2_pvalue(second[c], m * probs(p[0, c + 1])) > 1e-3


@pytest.mark.parametrize("toks", [(2, 5, 1), (3, 3, 4), (0, 0, 0), (6, 7, 6), (4, 1, 2)])
def test_tree_det_root_exact(toks):
    """Exact enumeration over the uniforms (bisection on each accept test,
    measure of each final token over the final uniform): for a root with three
    fixed candidates, repeated tokens included (token 7's logit is -inf), the
    first emitted token follows P_root exactly; below an accepted first child
    with one fixed grandchild, the next token follows that child's row."""
    V = 8
    rng = np.random.default_rng(13)
    parent = np.array([-1, -1, -1, 0, 1, 2], dtype=np.int32)
    N = len(parent)
    p = rng.normal(0.0, 1.2, (1, N + 1, V)).astype(np.float32)
    p[0, 0, 7] = -np.inf
    P = [probs(p[0, r]) for r in range(N + 1)]
    HI = np.nextafter(1.0, 0.0)
    ft = FastDetTree(p, parent, max_children=3)

    def ovr_of(ua, uf_root, child_u=0.5, child_uf=0.5):
        o = np.zeros((1, N + 1, 4))
        o[0, 0, 1:4] = ua
        o[0, 0, 0] = uf_root
        o[0, 1:, 1] = child_u
        o[0, 1:, 0] = child_uf
        return o

    tk = [toks[0], toks[1], toks[2], 0, 0, 0]

    def took(ua, node):
        path = ft.run(tk, ovr_of(ua, 0.5))[2]
        return len(path) >= 1 and path[0] == node

    r_a = threshold(lambda u: took([u, HI, HI], 0))
    r_b = threshold(lambda u: took([HI, u, HI], 1))
    r_c = threshold(lambda u: took([HI, HI, u], 2))
    first = np.zeros(V)
    first[toks[0]] += r_a
    first[toks[1]] += (1 - r_a) * r_b
    first[toks[2]] += (1 - r_a) * (1 - r_b) * r_c
    rest = (1 - r_a) * (1 - r_b) * (1 - r_c)
    if rest > 0:
        for t, m in step_measure(lambda u: ft.run(tk, ovr_of([HI, HI, HI], u))[1][0]).items():
            first[t] += rest * m
    assert np.max(np.abs(first - P[0])) < 1e-12
    if toks[1] == toks[0]:
        assert r_b == 0.0  # a rejected token has probability 0 for its later siblings

    # second level: below an accepted child 0 (row 1), its fixed child node 3
    second = np.zeros(V)
    for g in range(V):
        tk2 = [toks[0], toks[1], toks[2], g, 0, 0]
        r_g = threshold(lambda u: ft.run(tk2, ovr_of([0.0, HI, HI], 0.5, child_u=u))[0] >= 2)
        sec = np.zeros(V)
        sec[g] += r_g
        if r_g < 1:
            meas = step_measure(lambda u: ft.run(tk2, ovr_of([0.0, HI, HI], 0.5, child_u=HI, child_uf=u))[1][1])
            for t, m in meas.items():
                sec[t] += (1 - r_g) * m
        assert np.max(np.abs(sec - P[1])) < 1e-12, g


def test_tree_det_greedy_and_errors():
    rng = np.random.default_rng(2)
    V = 9
    p = rng.normal(0.0, 1.0, (3, 4, V)).astype(np.float32)
    g0 = [int(np.argmax(p[b, 0])) for b in range(3)]
    parent = np.array([[-1, -1, 1]] * 3, dtype=np.int32)
    toks = np.array([[(g0[0] + 1) % V, g0[0], 3], [(g0[1] + 1) % V, (g0[1] + 2) % V, 1], [0, 1, 2]],
                    dtype=np.int32)
    parent[2, 2] = 2  # malformed: parent not before the node
    o = oracle.verify_tree_det(p, parent, toks, 0.0)
    assert o["len"][0] >= 1 and o["path"][0, 0] == 1 and o["tokens"][0, 0] == g0[0]
    g2 = int(np.argmax(p[0, 2]))
    assert o["tokens"][0, 1] == (3 if g2 == 3 else g2) and o["len"][0] == (2 if g2 == 3 else 1)
    assert o["len"][1] == 0 and o["tokens"][1, 0] == g0[1]
    assert o["len"][2] == -1 and (o["tokens"][2] == -1).all()


# ------------------------------------------------------ TV distillation loss --
def _tv_ref(a, d, T=1.0):
    """scipy softmaxes; TV = 1 - sum min(p, q) (an identity, not the oracle's sum)."""
    P, Q = probs(a, T), probs(d, T)
    return 1.0 - np.minimum(P, Q).sum()


def test_tv_loss_closed_forms():
    rng = np.random.default_rng(3)
    a = rng.normal(0, 2, (3, 50)).astype(np.float32)
    loss, g = oracle.tv_loss(a, a.copy(), 1.0)
    assert np.all(loss == 0.0) and np.all(g == 0.0)  # identical rows
    p = np.full((2, 10), -np.inf, dtype=np.float32)
    q = np.full((2, 10), -np.inf, dtype=np.float32)
    p[:, :4] = rng.normal(0, 1, (2, 4))
    q[:, 4:] = rng.normal(0, 1, (2, 6))
    loss, _ = oracle.tv_loss(p, q, 1.0)
    assert np.allclose(loss, 1.0, rtol=0, atol=1e-15)  # disjoint supports
    # two tokens: TV = |sigmoid(x / T) - sigmoid(y / T)|
    from scipy.special import expit
    xs = rng.normal(0, 3, 20).astype(np.float32)
    ys = rng.normal(0, 3, 20).astype(np.float32)
    z = np.zeros(20, dtype=np.float32)
    for T in (1.0, 0.6):
        loss, _ = oracle.tv_loss(np.stack([xs, z], 1), np.stack([ys, z], 1), T)
        ref = np.abs(expit(xs.astype(np.float64) / T) - expit(ys.astype(np.float64) / T))
        assert np.allclose(loss, ref, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("dtype,T", [("f32", 1.0), ("bf16", 1.0), ("f32", 0.7)])
def test_tv_loss_is_one_minus_acceptance(dtype, T):
    """TV(p, q) = 1 - sum min(p, q): one minus the acceptance probability of a
    drawn draft (the quantity the TV term is chosen to govern)."""
    p, q = synth.pair(4, 3, 3, 3000, dtype, seed=8, sd_a=2.0, mode=0, sd_noise=1.0)
    loss, _ = oracle.tv_loss(p, q, T, grad=False)
    a, d = _as64(p).reshape(12, -1), _as64(q).reshape(12, -1)
    ref = np.array([_tv_ref(a[r], d[r], T) for r in range(12)])
    assert np.allclose(loss, ref, rtol=1e-12, atol=1e-14)


def _as64(x):
    return (synth.bf16_to_f32(x) if x.dtype == np.uint16 else x).astype(np.float64)


def test_tv_grad_finite_differences():
    """The gradient with respect to the student logits against central
    differences of the loss (scipy softmaxes in fp64) at random points away
    from the kinks p_v = q_v."""
    rng = np.random.default_rng(4)
    R, V = 5, 9
    a = rng.normal(0, 1.5, (R, V)).astype(np.float32)
    d = rng.normal(0, 1.5, (R, V)).astype(np.float32)
    w = rng.uniform(0.5, 2.0, R)
    for T in (1.0, 0.8):
        _, g = oracle.tv_loss(a, d, T, row_weights=w)
        h = 1e-6
        for r in range(R):
            fd = np.zeros(V)
            for j in range(V):
                dp = d[r].astype(np.float64).copy()
                dm = dp.copy()
                dp[j] += h
                dm[j] -= h
                fd[j] = (_tv_ref(a[r], dp, T) - _tv_ref(a[r], dm, T)) / (2 * h)
            assert np.allclose(g[r], w[r] * fd, rtol=1e-6, atol=1e-8), (r, g[r], w[r] * fd)


def test_tv_grad_invariants_and_errors():
    p, q = synth.pair(3, 2, 2, 500, "bf16", seed=5, sd_a=2.0, mode=0, sd_noise=1.0)
    loss, g = oracle.tv_loss(p, q, 1.0)
    assert np.allclose(g.sum(axis=1), 0.0, atol=1e-15)  # adding a constant to a row changes nothing
    assert np.all((loss > 0) & (loss < 1))
    _, g2 = oracle.tv_loss(p, q, 1.0, row_weights=np.full(6, 3.0))
    assert np.allclose(g2, 3.0 * g, rtol=1e-15, atol=0)
    qf = synth.bf16_to_f32(q).copy()
    qf[0, 1, 7] = np.nan
    qf[1, 0, :] = -np.inf
    pf = synth.bf16_to_f32(p).copy()
    pf[2, 1, 3] = np.inf
    loss, g = oracle.tv_loss(pf, qf, 1.0)
    bad = [1, 2, 5]
    assert np.all(np.isnan(loss[bad])) and np.all(np.isnan(g[bad]))
    ok = [0, 3, 4]
    assert np.all(np.isfinite(loss[ok])) and np.all(np.isfinite(g[ok]))


# ------------------------------------------------- multi-round generation --
def _toy(V, dtype="f32"):
    return lambda kind, ctx, pos: synth.toy_logits(ctx, pos, V=V, kind=kind, dtype=dtype)


@pytest.mark.parametrize("T,block", [(1.0, 4), (0.7, 3)])
def test_generate_law(T, block):
    """Losslessness across rounds: the joint law of the first three generated
    tokens of 30,000 independent requests equals the toy target model's own
    autoregressive law (chi-square over the 125 outcomes, exact probabilities
    from scipy softmaxes of the target logits)."""
    V, B = 5, 30000
    model = _toy(V)
    prompt = np.tile(np.array([[3, 1]], dtype=np.int32), (B, 1))
    g = oracle.generate(model, prompt, block, V, T, seed=21, rounds=2, nthreads=8)
    assert np.all(g["len"] >= 3)
    s = g["seq"][:, :3]
    counts = np.zeros(V ** 3)
    np.add.at(counts, s[:, 0] * V * V + s[:, 1] * V + s[:, 2], 1)
    exp = np.zeros(V ** 3)
    for a in range(V):
        pa = probs(model(0, np.array([[3, 1]]), None)[0], T)[a]
        for b in range(V):
            pb = probs(model(0, np.array([[1, a]]), None)[0], T)[b]
            pc = probs(model(0, np.array([[a, b]]), None)[0], T)
            exp[a * V * V + b * V:a * V * V + b * V + V] = pa * pb * pc
    assert abs(exp.sum() - 1.0) < 1e-12
    assert chi2_pvalue(counts, B * exp) > 1e-3


def test_generate_round_bounds():
    """Each round commits between 2 and block + 1 tokens (so tokens per forward
    pass, with one draft and one verify pass per round, lie in [1, (block+1)/2]),
    and the committed sequence is the concatenation of the rounds."""
    V, B, block, R = 300, 64, 8, 6
    g = oracle.generate(_toy(V, "bf16"), synth.randint(4, 0, 2 * B, V).reshape(B, 2), block, V, 1.0, seed=5,
                        rounds=R, nthreads=8)
    rt = g["round_tokens"]
    assert rt.min() >= 2 and rt.max() <= block + 1 and len(set(rt.ravel().tolist())) >= 3
    assert np.array_equal(g["len"], rt.sum(axis=1))
    tpf = g["len"].sum() / (2 * R * B)
    assert 1.0 <= tpf <= (block + 1) / 2
    for b in range(B):
        assert np.all(g["seq"][b, :g["len"][b]] >= 0) and np.all(g["seq"][b, g["len"][b]:] == -1)


def test_generate_greedy_is_the_argmax_chain():
    """Temperature 0: the generated sequence is the target's greedy chain
    (argmax of the toy target at each context, lowest id on ties)."""
    V, B, block, R = 200, 8, 5, 4
    model = _toy(V)
    prompt = synth.randint(9, 0, 2 * B, V).reshape(B, 2)
    g = oracle.generate(model, prompt, block, V, 0.0, seed=0, rounds=R)
    for b in range(B):
        t1, t2 = int(prompt[b, 0]), int(prompt[b, 1])
        chain = []
        while len(chain) < g["len"][b]:
            a = model(0, np.array([[t1, t2]]), None)[0]
            x = int(np.argmax(a))
            chain.append(x)
            t1, t2 = t2, x
        assert chain == g["seq"][b, :g["len"][b]].tolist()


def test_lmhead_logits_small_loops():
    """z[r, v] = sum_k h[r, k] w[v, k] on a non-square case, written as loops
    over bf16 inputs (catches a transposed operand or a wrong decode)."""
    rng = np.random.default_rng(14)
    h = synth.f32_to_bf16(rng.normal(0, 1, (2, 3, 16)).astype(np.float32))
    w = synth.f32_to_bf16(rng.normal(0, 0.5, (7, 16)).astype(np.float32))
    z = oracle.lmhead_logits(h, w, chunk=3)
    hf, wf = synth.bf16_to_f32(h).astype(np.float64), synth.bf16_to_f32(w).astype(np.float64)
    assert z.shape == (2, 3, 7) and z.dtype == np.float32
    for a in range(2):
        for r in range(3):
            for v in range(7):
                ref = 0.0
                for k in range(16):
                    ref += hf[a, r, k] * wf[v, k]
                assert z[a, r, v] == np.float32(ref)
