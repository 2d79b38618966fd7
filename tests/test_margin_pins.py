"""Pins of the oracle's decision margins.

The GPU and the oracle may part only at a decision that lies within a stated
band of going the other way, and only at the first decision where they part.
These margins therefore decide which mismatches a parity test excuses. This
file recomputes each margin the oracle reports, on small cases and with
uniforms overridden, from quantities computed independently of the oracle:
- scipy softmaxes;
- brute-force inverse CDFs (numpy cumulative sums);
- brute-force sorts for top-p cuts and for the Tree Sampler's offers.
The margins covered are:
- accept tests;
- draft, residual, bonus and tree final draws, with the token across the
  nearer edge of each draw;
- top-p cuts;
- deterministic-candidate tests;
- candidate-enumeration gaps.

Every checker is also run against deliberately wrong margins. These are
plausible mistakes: a dropped min(1, .), an index off by one, a missing
normalisation, the wrong edge, the original target instead of the running
one, a sibling counted as a rival offer. The test requires that the checker
reject each of them, so a wrong margin in the oracle cannot pass unnoticed.
"""
from __future__ import annotations

import copy

import numpy as np
import pytest
from scipy.special import softmax

import oracle

REL = 1e-11  # the margins are differences of O(1) quantities computed in a different order


# ------------------------------------------------------------ references --
def ref_draw(w, u):
    """Inverse-CDF draw by brute force: (token, margin, alt)."""
    w = np.asarray(w, dtype=np.float64)
    C = np.cumsum(w)
    W = C[-1]
    t = u * W
    j = int(np.searchsorted(C, t, side="right"))
    if j >= len(w):  # rounding fallback: last positive weight
        j = int(np.nonzero(w > 0)[0][-1])
        return j, 0.0, j
    lo = t - (C[j - 1] if j else 0.0)
    hi = C[j] - t
    if lo <= hi:
        prev = np.nonzero(w[:j] > 0)[0]
        alt = int(prev[-1]) if prev.size else -1
    else:
        nxt = np.nonzero(w[j + 1:] > 0)[0]
        alt = int(j + 1 + nxt[0]) if nxt.size else -1
    return j, min(lo, hi) / W, alt


def ref_filter(a, T, top_k, top_p):
    """Temperature, top-k, top-p by sorting: (z with removed entries at -inf,
    top-p cut margin or +inf)."""
    z = np.asarray(a, dtype=np.float64) / T
    V = z.size
    order = np.lexsort((np.arange(V), -z))  # logit descending, id ascending
    if 0 < top_k < V:
        z[order[top_k:]] = -np.inf
    margin = np.inf
    if top_p < 1.0:
        keep = np.isfinite(z)
        pr = np.zeros(V)
        pr[keep] = softmax(z[keep])
        order = np.lexsort((np.arange(V), -pr))
        order = order[keep[order]]
        cum = np.cumsum(pr[order])
        t = int(np.searchsorted(cum, top_p, side="left"))  # first cum >= top_p
        t = min(t, len(cum) - 1)
        prev = cum[t - 1] if t else 0.0
        margin = min(abs(cum[t] - top_p), top_p - prev)
        z[order[t + 1:]] = -np.inf
    return z, margin


def sm(z):
    return softmax(np.asarray(z, dtype=np.float64))


def close(a, b):
    if np.isinf(a) or np.isinf(b):
        return a == b
    return abs(a - b) <= REL


# ---------------------------------------------------------------- linear --
def linear_expected(p, q, draft, ovr, T, top_k, top_p, fused):
    """Per-request margins of the linear rule, recomputed from scratch."""
    B, K1, V = p.shape
    K = K1 - 1
    out = []
    for b in range(B):
        zs, fm = [], np.inf
        for i in range(K + 1):
            z, m = ref_filter(p[b, i], T, top_k, top_p)
            zs.append(z)
            fm = min(fm, m)
        zq = []
        for i in range(K):
            z, m = ref_filter(q[b, i], T, top_k, top_p)
            zq.append(z)
            fm = min(fm, m)
        P = [sm(z) for z in zs]
        Q = [sm(z) for z in zq]
        d = np.array(draft[b], dtype=np.int64)
        m_draft = np.full(K, np.inf)
        alt_draft = np.full(K, -1)
        if fused:
            for i in range(K):
                d[i], m_draft[i], alt_draft[i] = ref_draw(Q[i], ovr[b, i, 2])
        m_acc = np.full(K, np.inf)
        n = K
        for i in range(K):
            u = ovr[b, i, 1]
            Pi, Qi = P[i][d[i]], Q[i][d[i]]
            if Qi > 0:
                m_acc[i] = abs(u - min(1.0, Pi / Qi))
            if not u * Qi < Pi:
                n = i
                break
        if n < K:
            w = np.maximum(P[n] - Q[n], 0.0)
            if not w.sum() > 0:
                w = P[n]
        else:
            w = P[K]
        y, m_fin, alt_fin = ref_draw(w, ovr[b, n, 0])
        out.append(dict(n=n, y=y, draft=d, m_acc=m_acc, m_draft=m_draft, alt_draft=alt_draft, m_final=m_fin,
                        alt_final=alt_fin, m_filter=fm))
    return out


def check_linear(o, exp):
    for b, e in enumerate(exp):
        assert o["len"][b] == e["n"] and o["tokens"][b, e["n"]] == e["y"], b
        for i in range(len(e["m_acc"])):
            assert close(o["m_acc"][b, i], e["m_acc"][i]), ("acc", b, i, o["m_acc"][b, i], e["m_acc"][i])
            assert close(o["m_draft"][b, i], e["m_draft"][i]), ("draft", b, i)
            assert o["alt_draft"][b, i] == e["alt_draft"][i], ("draft alt", b, i)
        assert close(o["m_final"][b], e["m_final"]), ("final", b, o["m_final"][b], e["m_final"])
        assert o["alt_final"][b] == e["alt_final"], ("final alt", b)
        assert close(o["m_filter"][b], e["m_filter"]), ("filter", b, o["m_filter"][b], e["m_filter"])


def _linear_case(seed, B=6, K=4, V=40, noise=1.0):
    rng = np.random.default_rng(seed)
    p = rng.normal(0, 1.5, (B, K + 1, V)).astype(np.float32)
    q = (p[:, :K] + rng.normal(0, noise, (B, K, V))).astype(np.float32)
    ovr = rng.random((B, K + 1, 3))
    # drafts: mostly likely under q, some the target's argmax (p > q there), some rare
    draft = np.empty((B, K), dtype=np.int32)
    for b in range(B):
        for i in range(K):
            draft[b, i] = (np.argmax(p[b, i]) if (b + i) % 3 == 0 else
                           np.argmax(q[b, i]) if (b + i) % 3 == 1 else rng.integers(0, V))
    return p, q, draft, ovr


def _linear_mutants(o, exp):
    """Plausible mistakes in the margins of a linear verification."""
    K = o["m_acc"].shape[1]
    muts = []
    # |u - P/Q| without the cap at 1
    m = copy.deepcopy(o)
    hit = False
    for b, e in enumerate(exp):
        for i in range(min(e["n"] + 1, K)):
            P, Q = o["probs"][b, i]
            if Q > 0 and P > Q:
                m["m_acc"][b, i] = abs(u_of(b, i) - P / Q)
                hit = True
    if hit:
        muts.append(("no min(1, P/Q)", m))
    m = copy.deepcopy(o)
    m["m_acc"] = np.roll(o["m_acc"], 1, axis=1)
    muts.append(("accept margin one position late", m))
    resid = (o["len"] < K) & (o["len"] >= 0) & (o["resid"] < 0.9)
    if resid.any():
        m = copy.deepcopy(o)
        m["m_final"] = np.where(resid, o["m_final"] * o["resid"], o["m_final"])
        muts.append(("residual margin not divided by the residual mass", m))
    m = copy.deepcopy(o)
    m["alt_final"] = np.where(o["alt_final"] >= 0, o["tokens"][np.arange(len(o["len"])), o["len"]] + 1, -1)
    muts.append(("alternative token taken as the next id", m))
    m = copy.deepcopy(o)
    m["m_final"] = np.where(np.isfinite(o["m_final"]), 0.5 - o["m_final"], o["m_final"])
    muts.append(("far edge instead of the near one", m))
    return muts


_U = {}


def u_of(b, i):
    return _U["ovr"][b, i, 1]


@pytest.mark.parametrize("seed,T,top_k,top_p,fused", [(0, 1.0, 0, 1.0, False), (1, 0.7, 0, 1.0, True),
                                                      (2, 1.0, 12, 0.9, True), (3, 1.3, 0, 0.8, False)])
def test_linear_margins(seed, T, top_k, top_p, fused):
    p, q, draft, ovr = _linear_case(seed)
    _U["ovr"] = ovr
    o = oracle.verify_linear(p, q, None if fused else draft, T, top_k=top_k, top_p=top_p, fused=fused,
                             u_override=ovr)
    exp = linear_expected(p, q, draft, ovr, T, top_k, top_p, fused)
    check_linear(o, exp)
    assert (o["len"] < p.shape[1] - 1).any()  # residual draws happen
    muts = _linear_mutants(o, exp)
    assert len(muts) >= 4
    for name, m in muts:
        with pytest.raises(AssertionError):
            check_linear(m, exp)
            raise RuntimeError(f"mutant not detected: {name}")


def test_linear_margins_bonus_and_ratio_cap():
    """Drafts equal to the target argmax on near-identical rows: accept tests
    with P > Q (capped ratio) and bonus draws."""
    rng = np.random.default_rng(7)
    B, K, V = 8, 3, 30
    p = rng.normal(0, 2.0, (B, K + 1, V)).astype(np.float32)
    q = (p[:, :K] + rng.normal(0, 0.05, (B, K, V))).astype(np.float32)
    draft = np.argmax(p[:, :K], axis=2).astype(np.int32)
    ovr = rng.random((B, K + 1, 3))
    _U["ovr"] = ovr
    o = oracle.verify_linear(p, q, draft, 1.0, u_override=ovr)
    exp = linear_expected(p, q, draft, ovr, 1.0, 0, 1.0, False)
    check_linear(o, exp)
    assert (o["len"] == K).any()
    for name, m in _linear_mutants(o, exp):
        with pytest.raises(AssertionError):
            check_linear(m, exp)
            raise RuntimeError(f"mutant not detected: {name}")


def test_draft_sample_margins():
    """Margins and alternative tokens of psispec-style draft draws, with a
    top-p cut on some rows."""
    rng = np.random.default_rng(4)
    B, K, V = 5, 3, 60
    q = rng.normal(0, 1.5, (B, K, V)).astype(np.float32)
    u = rng.random((B, K))
    for top_k, top_p in ((0, 1.0), (20, 0.85)):
        x, m = oracle.draft_sample(q, 0.9, top_k=top_k, top_p=top_p, u_override=u)
        for b in range(B):
            for i in range(K):
                z, fm = ref_filter(q[b, i], np.float64(0.9), top_k, top_p)
                j, mg, alt = ref_draw(sm(z), u[b, i])
                assert x[b, i] == j and close(m["cdf"][b, i], mg) and m["alt"][b, i] == alt
                assert close(m["filter"][b, i], fm)
        bad = copy.deepcopy(m)
        bad["alt"] = np.where(m["alt"] >= 0, x - 1, -1)
        assert any(bad["alt"][b, i] != m["alt"][b, i] for b in range(B) for i in range(K))


# ------------------------------------------------------------------ tree --
def tree_expected(p, q, parent, tokens, ovr, T, top_k, top_p):
    """The tree walk with the recursive residual, recomputed: per-node accept
    margins and the final draw."""
    B, R, V = p.shape
    N = R - 1
    out = []
    for b in range(B):
        m_acc = np.full(N, np.inf)
        fm = np.inf
        row, path = 0, []
        while True:
            zp, m1 = ref_filter(p[b, row], T, top_k, top_p)
            zq, m2 = ref_filter(q[b, row], T, top_k, top_p)
            fm = min(fm, m1, m2)
            r, Q = sm(zp), sm(zq)
            acc, j = -1, 0
            for c in range(N):
                if parent[c] != row - 1:
                    continue
                tok = tokens[b, c]
                u = ovr[b, row, 1 + j]
                if Q[tok] > 0:
                    m_acc[c] = abs(u - min(1.0, r[tok] / Q[tok]))
                if u * Q[tok] < r[tok]:
                    acc = c
                    break
                w = np.maximum(r - Q, 0.0)
                if w.sum() > 0:
                    r = w / w.sum()
                j += 1
            if acc < 0:
                y, mf, alt = ref_draw(r, ovr[b, row, 0])
                break
            path.append(acc)
            row = acc + 1
        out.append(dict(path=path, y=y, m_acc=m_acc, m_final=mf, alt_final=alt, m_filter=fm))
    return out


def check_tree(o, exp):
    for b, e in enumerate(exp):
        n = len(e["path"])
        assert o["len"][b] == n and list(o["path"][b, :n]) == e["path"] and o["tokens"][b, n] == e["y"], b
        for c in range(len(e["m_acc"])):
            assert close(o["m_acc"][b, c], e["m_acc"][c]), ("acc", b, c, o["m_acc"][b, c], e["m_acc"][c])
        assert close(o["m_final"][b], e["m_final"]) and o["alt_final"][b] == e["alt_final"], ("final", b)
        assert close(o["m_filter"][b], e["m_filter"]), ("filter", b)


def _tree_case(seed, B=8, V=16):
    rng = np.random.default_rng(seed)
    parent = np.array([-1, -1, -1, 0, 1, 2, 3, 4, 5, 0], dtype=np.int32)  # root: 3 children, then chains
    N = len(parent)
    p = rng.normal(0, 1.5, (B, N + 1, V)).astype(np.float32)
    q = (p + rng.normal(0, 1.5, (B, N + 1, V))).astype(np.float32)
    tokens = rng.integers(0, V, (B, N)).astype(np.int32)
    maxC = 4
    ovr = rng.random((B, N + 1, 1 + maxC))
    return p, q, parent, tokens, ovr, maxC


def _running_target_mutant(p, q, parent, tokens, ovr, T, top_k, top_p, o):
    """Accept margins computed against the row's original target P instead of
    the running residual target."""
    m = copy.deepcopy(o)
    hit = False
    for b in range(p.shape[0]):
        for c in range(len(parent)):
            if not np.isfinite(o["m_acc"][b, c]):
                continue
            row = parent[c] + 1
            j = int(np.sum(parent[:c] == parent[c]))
            if j == 0:
                continue  # the first child sees r = P: no difference
            P = sm(ref_filter(p[b, row], T, top_k, top_p)[0])
            Q = sm(ref_filter(q[b, row], T, top_k, top_p)[0])
            tok = tokens[b, c]
            m["m_acc"][b, c] = abs(ovr[b, row, 1 + j] - min(1.0, P[tok] / Q[tok]))
            hit = True
    return m if hit else None


@pytest.mark.parametrize("seed,T,top_k,top_p", [(0, 1.0, 0, 1.0), (1, 0.8, 10, 0.9)])
def test_tree_margins(seed, T, top_k, top_p):
    p, q, parent, tokens, ovr, maxC = _tree_case(seed)
    o = oracle.verify_tree(p, q, parent, tokens, T, top_k=top_k, top_p=top_p, u_override=ovr, max_children=maxC)
    exp = tree_expected(p, q, parent, tokens, ovr, np.float64(T), top_k, top_p)
    check_tree(o, exp)
    muts = []
    m = _running_target_mutant(p, q, parent, tokens, ovr, np.float64(T), top_k, top_p, o)
    assert m is not None, "no second sibling was tested: the case does not exercise the running target"
    muts.append(("original target instead of the running one", m))
    m = copy.deepcopy(o)
    m["m_acc"] = np.roll(o["m_acc"], 1, axis=1)
    muts.append(("margin on the neighbouring node", m))
    m = copy.deepcopy(o)
    m["m_final"] = o["m_final"] * 2.0
    muts.append(("final margin over half the mass", m))
    for name, mm in muts:
        with pytest.raises(AssertionError):
            check_tree(mm, exp)
            raise RuntimeError(f"mutant not detected: {name}")


def test_tree_draft_margins():
    p, q, parent, _, _, _ = _tree_case(3)
    x, m = oracle.tree_draft(q, parent, 1.0, top_k=8, top_p=0.95, seed=5, step=2, margins=True)
    sib = np.zeros(len(parent), dtype=np.int64)
    for n in range(len(parent)):
        sib[n] = np.sum(parent[:n] == parent[n])
    for b in range(q.shape[0]):
        for n in range(len(parent)):
            row = parent[n] + 1
            z, fm = ref_filter(q[b, row], 1.0, 8, 0.95)
            u = oracle.uniform(5, 2, b, row, oracle.DRAFT_DRAW + int(sib[n]))
            j, mg, alt = ref_draw(sm(z), u)
            assert x[b, n] == j and close(m["cdf"][b, n], mg) and m["alt"][b, n] == alt and close(m["filter"][b, n], fm)


# --------------------------------------------------- deterministic tree --
def dtree_expected(p, parent, tokens, ovr, T):
    B, R, V = p.shape
    N = R - 1
    out = []
    for b in range(B):
        m_acc = np.full(N, np.inf)
        row, path = 0, []
        while True:
            P = sm(np.asarray(p[b, row], dtype=np.float64) / T)
            removed = np.zeros(V, dtype=bool)
            E, j, acc = 0.0, 0, -1
            for c in range(N):
                if parent[b, c] != row - 1:
                    continue
                tok = tokens[b, c]
                pt = 0.0 if removed[tok] else P[tok]
                u = ovr[b, row, 1 + j]
                if pt > 0 and 1.0 - E > 0:
                    m_acc[c] = abs(u - pt / (1.0 - E))
                if u * (1.0 - E) < pt:
                    acc = c
                    break
                if not removed[tok]:
                    removed[tok] = True
                    E += P[tok]
                j += 1
            if acc < 0:
                w = np.where(removed, 0.0, P)
                y, mf, alt = ref_draw(w if w.sum() > 0 else P, ovr[b, row, 0])
                break
            path.append(acc)
            row = acc + 1
        out.append(dict(path=path, y=y, m_acc=m_acc, m_final=mf, alt_final=alt, m_filter=np.inf))
    return out


def test_dtree_margins():
    rng = np.random.default_rng(11)
    B, V = 10, 12
    parent = np.tile(np.array([-1, -1, -1, -1, 0, 0, 1, 4], dtype=np.int32), (B, 1))
    N = parent.shape[1]
    p = rng.normal(0, 1.2, (B, N + 1, V)).astype(np.float32)
    tokens = np.empty((B, N), dtype=np.int32)
    for b in range(B):
        top = np.argsort(-p[b, 0])
        tokens[b, :4] = [top[0], top[1], top[0], top[2]]  # a repeated sibling: removed after its rejection
        tokens[b, 4:] = rng.integers(0, V, N - 4)
    maxC = 4
    ovr = rng.random((B, N + 1, 1 + maxC))
    o = oracle.verify_tree_det(p, parent, tokens, 1.0, u_override=ovr, max_children=maxC)
    exp = dtree_expected(p, parent, tokens, ovr, 1.0)
    check_tree(o, exp)
    # P(tok) instead of the running target's mass P(tok) / (1 - E)
    m = copy.deepcopy(o)
    hit = False
    for b in range(B):
        for c in range(N):
            row = parent[b, c] + 1
            j = int(np.sum(parent[b, :c] == parent[b, c]))
            if np.isfinite(o["m_acc"][b, c]) and j > 0:
                P = sm(p[b, row].astype(np.float64))
                m["m_acc"][b, c] = abs(ovr[b, row, 1 + j] - P[tokens[b, c]])
                hit = True
    assert hit
    with pytest.raises(AssertionError):
        check_tree(m, exp)
    m = copy.deepcopy(o)
    m["alt_final"] = np.where(o["alt_final"] >= 0, (o["alt_final"] + 1) % V, -1)
    with pytest.raises(AssertionError):
        check_tree(m, exp)


# ------------------------------------------------------------ candidates --
def cand_gaps_expected(q, T, cands, par, tok):
    """Gap of every enumeration step, from the kept tree alone: at the step
    that keeps node n, every other kept prefix (and the empty one) offers its
    best child not yet kept; the gap is node n's score minus the best of
    those offers."""
    K, V = q.shape
    z = np.asarray(q, dtype=np.float64) / T
    lq = z - np.logaddexp.reduce(z, axis=1, keepdims=True)
    ranks = [np.lexsort((np.arange(V), -lq[i]))[:cands] for i in range(K)]
    nodes = len(par)
    score, depth = np.zeros(nodes), np.zeros(nodes, dtype=int)
    gaps = np.full(nodes, np.inf)
    for n in range(nodes):
        if tok[n] < 0:
            break
        pp = par[n]
        depth[n] = 0 if pp < 0 else depth[pp] + 1
        score[n] = (0.0 if pp < 0 else score[pp]) + lq[depth[n], tok[n]]
        best = -np.inf
        for s in [-1] + list(range(n)):
            if s == pp:
                continue  # node n's own parent: its best remaining child is node n
            d = 0 if s < 0 else depth[s] + 1
            if d >= K:
                continue
            taken = {tok[c] for c in range(n) if par[c] == s}
            rest = [t for t in ranks[d] if t not in taken]
            if not rest:
                continue
            best = max(best, (0.0 if s < 0 else score[s]) + lq[d, rest[0]])
        if np.isfinite(best):
            gaps[n] = score[n] - best
    return gaps


def test_candidate_gaps():
    rng = np.random.default_rng(5)
    B, K, V, C, NN = 4, 4, 9, 3, 14
    q = rng.normal(0.0, 1.5, (B, K, V)).astype(np.float32)
    par, tok, gap = oracle.tree_candidates(q, C, NN, 0.9)
    for b in range(B):
        e = cand_gaps_expected(q[b], 0.9, C, par[b], tok[b])
        for n in range(NN):
            assert close(gap[b, n], e[n]), (b, n, gap[b, n], e[n])
    # a plausible mistake: the next sibling of the kept node counted as a rival offer
    wrong = 0
    for b in range(B):
        z = q[b].astype(np.float64) / 0.9
        lq = z - np.logaddexp.reduce(z, axis=1, keepdims=True)
        for n in range(NN):
            pp = par[b, n]
            dn, x = 0, pp  # depth of node n (0 for a child of the empty prefix)
            while x >= 0:
                dn += 1
                x = par[b, x]
            rk = np.lexsort((np.arange(V), -lq[dn]))[:C]
            taken = {tok[b, c] for c in range(n + 1) if par[b, c] == pp}
            rest = [t for t in rk if t not in taken]
            if rest:
                sib_gap = lq[dn, tok[b, n]] - lq[dn, rest[0]]
                if sib_gap < gap[b, n] - REL:
                    wrong += 1
    assert wrong > 0, "no step where a sibling would have looked closer: the case does not exercise the rule"
