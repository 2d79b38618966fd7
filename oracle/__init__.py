"""ctypes binding of the plain CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the slow, obviously-correct double-precision
reference the GPU library is checked against. Only the test suite, the smoke
check and the CPU-baseline leg of the benchmark may import this module; the
GPU library and its Python binding never do.

Function-level citations live in oracle.c. The functions here only marshal
numpy arrays into the C entry points.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1
DRAFT_DRAW = 0x40000000


def build() -> str:
    """Compiles oracle.c into liboracle.so (gcc, no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fPIC", "-shared",
           "-o", _LIB, _SRC, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, u32, u64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_double
        L.orc_philox4x32_10.argtypes = [P, P, P]
        L.orc_philox4x32_10.restype = None
        L.orc_uniform.argtypes = [u64, u32, u32, u32, u32]
        L.orc_uniform.restype = f64
        L.orc_decode_row.argtypes = [P, ctypes.c_int, i64, ctypes.c_int, P]
        L.orc_decode_row.restype = ctypes.c_int
        L.orc_filter_row.argtypes = [P, ctypes.c_int, f64, ctypes.c_int, f64, P]
        L.orc_filter_row.restype = None
        L.orc_logsumexp.argtypes = [P, ctypes.c_int]
        L.orc_logsumexp.restype = f64
        L.orc_sample.argtypes = [P, ctypes.c_int, f64, P, P]
        L.orc_sample.restype = ctypes.c_int
        L.orc_tree_depth.argtypes = [P, ctypes.c_int]
        L.orc_tree_depth.restype = ctypes.c_int
        L.orc_draft_sample.argtypes = [P, ctypes.c_int, i64, ctypes.c_int, ctypes.c_int, f64, ctypes.c_int, f64,
                                       u64, u32, P, P, P, P, P, ctypes.c_int]
        L.orc_draft_sample.restype = ctypes.c_int
        L.orc_verify_linear.argtypes = [P, P, ctypes.c_int, i64, ctypes.c_int, ctypes.c_int, P, f64, ctypes.c_int,
                                        f64, u64, u32, ctypes.c_int, P, P, P, P, P, P, ctypes.c_int]
        L.orc_verify_linear.restype = ctypes.c_int
        L.orc_verify_tree.argtypes = [P, P, ctypes.c_int, i64, ctypes.c_int, ctypes.c_int, P, P, f64, ctypes.c_int,
                                      f64, u64, u32, P, P, P, P, P, ctypes.c_int, ctypes.c_int]
        L.orc_verify_tree.restype = ctypes.c_int
        L.orc_tree_draft.argtypes = [P, ctypes.c_int, i64, ctypes.c_int, ctypes.c_int, P, f64, ctypes.c_int, f64, u64,
                                     u32, P, P, P, P, ctypes.c_int]
        L.orc_tree_draft.restype = ctypes.c_int
        L.orc_tree_candidates.argtypes = [P, ctypes.c_int, i64, ctypes.c_int, ctypes.c_int, f64, ctypes.c_int,
                                          ctypes.c_int, P, P, P, ctypes.c_int]
        L.orc_tree_candidates.restype = ctypes.c_int
        L.orc_verify_tree_det.argtypes = [P, ctypes.c_int, i64, ctypes.c_int, ctypes.c_int, P, P, f64, u64, u32,
                                          P, P, P, P, P, ctypes.c_int, ctypes.c_int]
        L.orc_verify_tree_det.restype = ctypes.c_int
        L.orc_tv_loss.argtypes = [P, P, ctypes.c_int, i64, ctypes.c_int, f64, P, P, P, ctypes.c_int]
        L.orc_tv_loss.restype = ctypes.c_int
        del i32
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class _LinMargins(ctypes.Structure):
    # orc_lin_margins: acc, draft, fin, filter (double*), draft_alt, fin_alt (int32_t*)
    _fields_ = [("acc", ctypes.c_void_p), ("draft", ctypes.c_void_p), ("fin", ctypes.c_void_p),
                ("filter", ctypes.c_void_p), ("draft_alt", ctypes.c_void_p), ("fin_alt", ctypes.c_void_p)]


class _TreeMargins(ctypes.Structure):
    # orc_tree_margins: acc, fin, filter (double*), fin_alt (int32_t*)
    _fields_ = [("acc", ctypes.c_void_p), ("fin", ctypes.c_void_p), ("filter", ctypes.c_void_p),
                ("fin_alt", ctypes.c_void_p)]


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:  # raw bfloat16 bits
        return BF16
    raise TypeError("logits must be float32 or uint16 (bfloat16 bits)")


def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def uniform(seed, step, b, r, d) -> float:
    return lib().orc_uniform(seed, step, b, r, d)


def logsumexp(z) -> float:
    z = np.ascontiguousarray(z, dtype=np.float64)
    return lib().orc_logsumexp(_ptr(z), z.size)


def sample(w, u):
    """Inverse-CDF draw; returns (index, margin, alt): margin is the distance
    of u*W to the nearer edge of the chosen interval over W, alt the token
    across that edge (-1 if none)."""
    w = np.ascontiguousarray(w, dtype=np.float64)
    m = ctypes.c_double(0.0)
    a = ctypes.c_int(0)
    j = lib().orc_sample(_ptr(w), w.size, float(u), ctypes.byref(m), ctypes.byref(a))
    return j, m.value, a.value


def filter_row(a, temperature, top_k=0, top_p=1.0, with_margin=False):
    """Temperature, top-k, top-p on one row of logits; returns z (removed ->
    -inf), and with_margin=True also the top-p cut's margin (+inf if none)."""
    z = np.array(a, dtype=np.float64, copy=True)
    m = ctypes.c_double(0.0)
    lib().orc_filter_row(_ptr(z), z.size, float(temperature), int(top_k), float(top_p), ctypes.byref(m))
    return (z, m.value) if with_margin else z


def decode_row(logits, row):
    """Decodes row `row` of a 2-D logit array; returns (values, bad)."""
    a = np.ascontiguousarray(logits)
    V = a.shape[-1]
    out = np.zeros(V, dtype=np.float64)
    bad = lib().orc_decode_row(_ptr(a), _dtype_code(a), int(row), V, _ptr(out))
    return out, bool(bad)


def tree_depth(parent) -> int:
    p = np.ascontiguousarray(parent, dtype=np.int32)
    return lib().orc_tree_depth(_ptr(p), p.size)


def draft_sample(q, temperature, top_k=0, top_p=1.0, seed=0, step=0, u_override=None, nthreads=1):
    """q: [B, K, V] float32 or uint16 (bf16 bits). Returns (tokens [B,K], m)
    where m holds per-draft arrays [B,K]: "cdf" the draw's margin, "alt" the
    token across its nearer edge, "filter" its row's top-p cut margin (+inf
    where there is no such decision)."""
    q = np.ascontiguousarray(q)
    B, K, V = q.shape
    out = np.zeros((B, K), dtype=np.int32)
    mg = np.zeros((B, K), dtype=np.float64)
    alt = np.zeros((B, K), dtype=np.int32)
    mf = np.zeros((B, K), dtype=np.float64)
    ovr = None if u_override is None else np.ascontiguousarray(u_override, dtype=np.float64).reshape(B, K)
    rc = lib().orc_draft_sample(_ptr(q), _dtype_code(q), B, K, V, float(temperature), int(top_k), float(top_p),
                                int(seed), int(step), _ptr(out), _ptr(mg), _ptr(alt), _ptr(mf), _ptr(ovr),
                                int(nthreads))
    if rc != 0:
        raise ValueError("orc_draft_sample rejected its arguments")
    return out, dict(cdf=mg, alt=alt, filter=mf)


def verify_linear(p, q, draft_tokens, temperature, top_k=0, top_p=1.0, seed=0, step=0, fused=False,
                  u_override=None, nthreads=1):
    """p: [B, K+1, V], q: [B, K, V] (float32 or uint16 bf16 bits), draft_tokens [B, K].

    u_override: optional [B, K+1, 3] uniforms (slot 0 final draw, 1 accept test,
    2 draft draw at each row) replacing the Philox stream.
    Returns a dict with tokens, len, probs, resid, draft and the margins of
    every decision: m_acc [B,K] (accept tests; +inf where none was taken),
    m_draft / alt_draft [B,K] (drafts drawn in the call), m_final / alt_final
    [B] (final draw) and m_filter [B] (smallest top-p cut margin of the
    request's rows).
    """
    p = np.ascontiguousarray(p)
    q = np.ascontiguousarray(q)
    B, K1, V = p.shape
    K = K1 - 1
    assert q.shape == (B, K, V) and p.dtype == q.dtype
    draft = np.array(draft_tokens, dtype=np.int32, copy=True).reshape(B, K) if draft_tokens is not None \
        else np.zeros((B, K), dtype=np.int32)
    toks = np.zeros((B, K + 1), dtype=np.int32)
    ln = np.zeros(B, dtype=np.int32)
    probs = np.zeros((B, K, 2), dtype=np.float64)
    resid = np.zeros(B, dtype=np.float64)
    r = dict(m_acc=np.zeros((B, K)), m_draft=np.zeros((B, K)), alt_draft=np.zeros((B, K), dtype=np.int32),
             m_final=np.zeros(B), alt_final=np.zeros(B, dtype=np.int32), m_filter=np.zeros(B))
    mg = _LinMargins(_ptr(r["m_acc"]).value, _ptr(r["m_draft"]).value, _ptr(r["m_final"]).value,
                     _ptr(r["m_filter"]).value, _ptr(r["alt_draft"]).value, _ptr(r["alt_final"]).value)
    ovr = None if u_override is None else np.ascontiguousarray(u_override, dtype=np.float64).reshape(B, K + 1, 3)
    rc = lib().orc_verify_linear(_ptr(p), _ptr(q), _dtype_code(p), B, K, V, _ptr(draft), float(temperature),
                                 int(top_k), float(top_p), int(seed), int(step), int(bool(fused)), _ptr(toks),
                                 _ptr(ln), _ptr(probs), _ptr(resid), ctypes.byref(mg), _ptr(ovr), int(nthreads))
    if rc != 0:
        raise ValueError("orc_verify_linear rejected its arguments")
    r.update(tokens=toks, len=ln, probs=probs, resid=resid, draft=draft)
    return r


def tree_draft(q, parent, temperature, top_k=0, top_p=1.0, seed=0, step=0, nthreads=1, margins=False):
    """Node tokens [B, N] of a candidate tree: the j-th child of row r drawn from
    row r of q [B, N+1, V] with draw id 0x40000000 + j (argmax when greedy).
    margins=True also returns a dict of per-node arrays [B, N]: "cdf" the
    draw's margin, "alt" the token across its nearer edge, "filter" the top-p
    cut margin of its row."""
    q = np.ascontiguousarray(q)
    B, R, V = q.shape
    N = R - 1
    par = np.ascontiguousarray(parent, dtype=np.int32)
    out = np.zeros((B, N), dtype=np.int32)
    mg = np.zeros((B, N))
    alt = np.zeros((B, N), dtype=np.int32)
    mf = np.zeros((B, N))
    rc = lib().orc_tree_draft(_ptr(q), _dtype_code(q), B, N, V, _ptr(par), float(temperature), int(top_k),
                              float(top_p), int(seed), int(step), _ptr(out), _ptr(mg), _ptr(alt), _ptr(mf),
                              int(nthreads))
    if rc != 0:
        raise ValueError("orc_tree_draft rejected its arguments")
    return (out, dict(cdf=mg, alt=alt, filter=mf)) if margins else out


def _tree_margin_arrays(B, N):
    r = dict(m_acc=np.zeros((B, N)), m_final=np.zeros(B), alt_final=np.zeros(B, dtype=np.int32),
             m_filter=np.zeros(B))
    mg = _TreeMargins(_ptr(r["m_acc"]).value, _ptr(r["m_final"]).value, _ptr(r["m_filter"]).value,
                      _ptr(r["alt_final"]).value)
    return r, mg


def verify_tree(p, q, parent, node_tokens, temperature, top_k=0, top_p=1.0, seed=0, step=0, u_override=None,
                max_children=None, nthreads=1):
    """p, q: [B, N+1, V]; parent [N]; node_tokens [B, N].

    u_override: optional [B, N+1, 1+max_children] (slot 0 final draw, slot 1+j
    accept test of child j). Returns a dict with tokens, path, len and the
    margins: m_acc [B,N] (the accept test of each node, +inf if never tested),
    m_final / alt_final [B] (final draw), m_filter [B] (top-p cuts).
    """
    p = np.ascontiguousarray(p)
    q = np.ascontiguousarray(q)
    B, R, V = p.shape
    N = R - 1
    par = np.ascontiguousarray(parent, dtype=np.int32)
    nt = np.ascontiguousarray(node_tokens, dtype=np.int32).reshape(B, N)
    D = tree_depth(par)
    if D < 0:
        raise ValueError("malformed tree")
    toks = np.zeros((B, D + 1), dtype=np.int32)
    path = np.zeros((B, D), dtype=np.int32)
    ln = np.zeros(B, dtype=np.int32)
    r, mg = _tree_margin_arrays(B, N)
    maxC = 0
    ovr = None
    if u_override is not None:
        maxC = int(max_children)
        ovr = np.ascontiguousarray(u_override, dtype=np.float64).reshape(B, R, 1 + maxC)
    rc = lib().orc_verify_tree(_ptr(p), _ptr(q), _dtype_code(p), B, N, V, _ptr(par), _ptr(nt), float(temperature),
                               int(top_k), float(top_p), int(seed), int(step), _ptr(toks), _ptr(path), _ptr(ln),
                               ctypes.byref(mg), _ptr(ovr), maxC, int(nthreads))
    if rc != 0:
        raise ValueError("orc_verify_tree rejected its arguments")
    r.update(tokens=toks, path=path, len=ln)
    return r


def tree_candidates(q, cands, nodes, temperature, nthreads=1):
    """Tree Sampler candidates from draft logits q [B, K, V]: per request the
    `nodes` best prefixes over the top-`cands` tokens of each position.

    Returns (parent [B, nodes], tokens [B, nodes], gap [B, nodes]); gap[b, n]
    is the smallest log-score gap between the offer kept as node n and any
    other offer of that step (+inf when there was no other offer)."""
    q = np.ascontiguousarray(q)
    B, K, V = q.shape
    par = np.zeros((B, nodes), dtype=np.int32)
    tok = np.zeros((B, nodes), dtype=np.int32)
    mg = np.zeros((B, nodes), dtype=np.float64)
    rc = lib().orc_tree_candidates(_ptr(q), _dtype_code(q), B, K, V, float(temperature), int(cands), int(nodes),
                                   _ptr(par), _ptr(tok), _ptr(mg), int(nthreads))
    if rc != 0:
        raise ValueError("orc_tree_candidates rejected its arguments")
    return par, tok, mg


def verify_tree_det(p, parent, node_tokens, temperature, seed=0, step=0, u_override=None, max_children=None,
                    nthreads=1):
    """Verification of deterministic candidates: p [B, N+1, V], per-request
    parent [B, N] and node_tokens [B, N]. u_override: optional
    [B, N+1, 1+max_children] uniforms (slot 0 final draw, slot 1+j accept test
    of child j) replacing the Philox stream. Returns a dict with tokens
    [B, N+1], path [B, N], len [B] and the margins m_acc [B, N], m_final /
    alt_final [B] (m_filter is +inf: no filters)."""
    p = np.ascontiguousarray(p)
    B, R, V = p.shape
    N = R - 1
    par = np.ascontiguousarray(parent, dtype=np.int32).reshape(B, N)
    nt = np.ascontiguousarray(node_tokens, dtype=np.int32).reshape(B, N)
    toks = np.zeros((B, N + 1), dtype=np.int32)
    path = np.zeros((B, N), dtype=np.int32)
    ln = np.zeros(B, dtype=np.int32)
    r, mg = _tree_margin_arrays(B, N)
    ovr, maxC = None, 0
    if u_override is not None:
        maxC = int(max_children)
        ovr = np.ascontiguousarray(u_override, dtype=np.float64).reshape(B, N + 1, 1 + maxC)
    rc = lib().orc_verify_tree_det(_ptr(p), _dtype_code(p), B, N, V, _ptr(par), _ptr(nt), float(temperature),
                                   int(seed), int(step), _ptr(toks), _ptr(path), _ptr(ln), ctypes.byref(mg),
                                   _ptr(ovr), maxC, int(nthreads))
    if rc != 0:
        raise ValueError("orc_verify_tree_det rejected its arguments")
    r.update(tokens=toks, path=path, len=ln)
    return r


def tv_loss(p, q, temperature=1.0, row_weights=None, grad=True, nthreads=1):
    """Total-variation distillation loss of teacher logits p and student logits
    q ([R, V] or [..., V], float32 or uint16 bf16 bits): loss [R] = 1/2 sum |p - q|
    of the two softmaxes, and (grad=True) its gradient [R, V] with respect to the
    student logits, each row scaled by row_weights (default 1). fp64."""
    p = np.ascontiguousarray(p)
    q = np.ascontiguousarray(q)
    assert p.shape == q.shape and p.dtype == q.dtype
    V = p.shape[-1]
    R = int(np.prod(p.shape[:-1]))
    loss = np.zeros(R, dtype=np.float64)
    g = np.zeros((R, V), dtype=np.float64) if grad else None
    w = None if row_weights is None else np.ascontiguousarray(row_weights, dtype=np.float64).reshape(R)
    rc = lib().orc_tv_loss(_ptr(p), _ptr(q), _dtype_code(p), R, V, float(temperature), _ptr(w), _ptr(loss), _ptr(g),
                           int(nthreads))
    if rc != 0:
        raise ValueError("orc_tv_loss rejected its arguments")
    return loss, g


def generate(model, prompt, block, V, temperature, seed, rounds, nthreads=1):
    """Multi-round Psi-Spec generation ("Uno" research explainer, §3.3): each
    round draws the block's first token from the AR (target) model at the
    committed context (it is always kept), draws the other block - 1 positions
    from the drafter in parallel, scores them with the target model in one
    pass, verifies them (linear rule) and commits the first token, the
    accepted drafts and the final token; rejected drafts are dropped. So a
    round commits between 2 and block + 1 tokens and, with one draft pass and
    one verify pass per round, tokens per forward pass lie in [1, (block+1)/2].

    model(kind, ctx [rows, 2] int32, pos [rows] int32 or None) -> logits
    [rows, V] (float32 or bf16 bits): kind 0 is the target at context (t1, t2)
    (the last two tokens), kind 1 the drafter at block position pos.
    prompt [B, 2] int32: the last two tokens of each request's context.
    Random numbers: the first token of round r is drawn as draft 0 of a
    one-row draft call with step 2r; the drafts and the verification use
    step 2r + 1. Returns dict(seq [B, rounds * (block + 1)] (-1 padded),
    len [B], round_tokens [B, rounds], n [B, rounds] (accepted drafts) and the
    margins of every decision of every round: m_first / alt_first [B, rounds]
    (the first token's draw), m_draft / alt_draft [B, rounds, block - 1] (the
    drafts), m_acc [B, rounds, block - 1] (accept tests, +inf where none was
    taken) and m_final / alt_final [B, rounds] (the final draw))."""
    prompt = np.ascontiguousarray(prompt, dtype=np.int32).reshape(-1, 2)
    B = prompt.shape[0]
    K = block - 1
    L = rounds * (block + 1)
    seq = np.full((B, L), -1, dtype=np.int32)
    ln = np.zeros(B, dtype=np.int32)
    rt = np.zeros((B, rounds), dtype=np.int32)
    nacc = np.zeros((B, rounds), dtype=np.int32)
    mf, af = np.zeros((B, rounds)), np.zeros((B, rounds), dtype=np.int32)
    md_, ad_ = np.zeros((B, rounds, K)), np.zeros((B, rounds, K), dtype=np.int32)
    ma = np.zeros((B, rounds, K))
    mfin, afin = np.zeros((B, rounds)), np.zeros((B, rounds), dtype=np.int32)
    t1, t2 = prompt[:, 0].copy(), prompt[:, 1].copy()
    for r in range(rounds):
        # first position: the target model itself
        p0 = model(0, np.stack([t1, t2], 1), None).reshape(B, 1, V)
        x0, m0 = draft_sample(p0, temperature, seed=seed, step=2 * r, nthreads=nthreads)
        x0 = x0[:, 0]
        # drafts at positions 1 .. K, from the committed context and x0
        cq = np.repeat(np.stack([t2, x0], 1), K, axis=0)
        pq = np.tile(np.arange(1, K + 1, dtype=np.int32), B)
        q = model(1, cq, pq).reshape(B, K, V)
        d, md = draft_sample(q, temperature, seed=seed, step=2 * r + 1, nthreads=nthreads)
        # target rows: row i scores draft i given (prefix, x0, d_0 .. d_{i-1}); row K is the bonus row
        hist = np.concatenate([t2[:, None], x0[:, None], d], axis=1)  # [B, K + 2]
        cp = np.stack([hist[:, :K + 1], hist[:, 1:K + 2]], axis=2).reshape(-1, 2)
        p = model(0, cp, None).reshape(B, K + 1, V)
        v = verify_linear(p, q, d, temperature, seed=seed, step=2 * r + 1, nthreads=nthreads)
        mf[:, r], af[:, r] = m0["cdf"][:, 0], m0["alt"][:, 0]
        md_[:, r], ad_[:, r] = md["cdf"], md["alt"]
        ma[:, r], mfin[:, r], afin[:, r] = v["m_acc"], v["m_final"], v["alt_final"]
        for b in range(B):
            n = int(v["len"][b])
            toks = [int(x0[b])] + [int(t) for t in v["tokens"][b, :n + 1]]
            seq[b, ln[b]:ln[b] + len(toks)] = toks
            ln[b] += len(toks)
            rt[b, r] = len(toks)
            nacc[b, r] = n
            t1[b], t2[b] = seq[b, ln[b] - 2], seq[b, ln[b] - 1]
    return dict(seq=seq, len=ln, round_tokens=rt, n=nacc, m_first=mf, alt_first=af, m_draft=md_, alt_draft=ad_,
                m_acc=ma, m_final=mfin, alt_final=afin)


def lmhead_logits(h, w, chunk=16384):
    """Logits of hidden states through the shared output head ("Uno" research
    explainer, §3.1: the AR and diffusion paths share the base model and its
    head): z = h W^T, h [..., H] and w [V, H] in bf16 bits (uint16) or float32,
    exact products summed in fp64 (numpy matmul), returned rounded to float32.
    The vocabulary is processed `chunk` rows at a time."""
    def f64(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            x = (x.astype(np.uint32) << 16).view(np.float32)
        return x.astype(np.float64)

    hh = f64(h)
    lead, H = hh.shape[:-1], hh.shape[-1]
    hh = hh.reshape(-1, H)
    V = w.shape[0]
    out = np.empty((hh.shape[0], V), dtype=np.float32)
    for v0 in range(0, V, chunk):
        out[:, v0:v0 + chunk] = (hh @ f64(w[v0:v0 + chunk]).T).astype(np.float32)
    return out.reshape(*lead, V)
