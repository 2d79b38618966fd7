"""GPU parity of psispec_verify_linear / psispec_draft_sample against the CPU
oracle, element by element on the same seeded inputs: accepted lengths and
tokens bit-exact except counted near ties, probabilities within 1e-5
relative, residual masses within 1e-9 relative."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import THREADS, compare_linear, f32, to_dev
from oracle_helpers import alpha, chi2_pvalue, probs

pytestmark = pytest.mark.gpu


def _psi():
    import lossless_speculative_verification_amd as psi
    return psi


def _run_pair(p, q, draft, T, seed, step, fused, top_k=0, top_p=1.0):
    # the C ABI carries temperature and top_p as binary32: give the oracle the same values
    T, top_p = f32(T), f32(top_p)
    psi = _psi()
    pd, qd = to_dev(p), to_dev(q)
    dd = None if draft is None else torch.from_numpy(np.ascontiguousarray(draft, dtype=np.int32)).cuda()
    g = psi.verify_linear(pd, qd, dd, temperature=T, top_k=top_k, top_p=top_p, seed=seed, step=step, fused=fused)
    torch.cuda.synchronize()
    o = oracle.verify_linear(p, q, draft, T, top_k=top_k, top_p=top_p, seed=seed, step=step, fused=fused,
                             nthreads=THREADS)
    return g, o


def test_tiny_trials_fused():
    """Tiny workload (B=1, K=4, V=1024, fp32, T=1), fused drafts, 300 trials with step = trial."""
    p, q = synth.linear_inputs("tiny", seed=0)
    ex_total = dec_total = 0
    for t in range(300):
        g, o = _run_pair(p, q, None, 1.0, 0, t, True)
        assert np.array_equal(g["draft"].cpu().numpy(), o["draft"]) or o["margin_cdf"][0] < 1e-11
        ex, dec, _ = compare_linear(g, o)
        ex_total += ex
        dec_total += dec
    assert ex_total <= max(1, 1e-4 * dec_total)


def test_tiny_replicas_one_call():
    """2000 replicas of the tiny workload in one call (request id keys the
    random stream): parity with the oracle on every replica."""
    p, q = synth.linear_inputs("tiny", seed=0)
    B = 2000
    p = np.ascontiguousarray(np.repeat(p, B, axis=0))
    q = np.ascontiguousarray(np.repeat(q, B, axis=0))
    g, o = _run_pair(p, q, None, 1.0, 0, 0, True)
    ex, dec, _ = compare_linear(g, o)
    assert ex <= max(1, 1e-4 * dec)


@pytest.mark.parametrize("rho", [0.5, 0.8, 0.95])
def test_highconc_full_size(rho):
    """High-concurrency workload at full size (B=256, K=8, V=151936, bf16, T=1)
    in the benchmark's launch configuration, drafts drawn by the oracle."""
    p, q = synth.linear_inputs("highconc", seed=0, rho=rho)
    ex_total = dec_total = 0
    for step in range(2):
        d, _ = oracle.draft_sample(q, 1.0, seed=0, step=step, nthreads=THREADS)
        g, o = _run_pair(p, q, d, 1.0, 0, step, False)
        ex, dec, _ = compare_linear(g, o)
        ex_total += ex
        dec_total += dec
    assert ex_total <= max(1, 1e-4 * dec_total)


def test_qwen_fused_full_size():
    """Qwen3-8B-shaped workload (B=64, K=8, V=151936, bf16, T=0.7) with fused drafts."""
    p, q = synth.linear_inputs("qwen", seed=0)
    g, o = _run_pair(p, q, None, 0.7, 0, 3, True)
    gd = g["draft"].cpu().numpy()
    mism = np.nonzero(gd != o["draft"])[0]
    assert all(o["margin_cdf"][b] < 1e-11 for b in mism)
    ex, dec, _ = compare_linear(g, o)
    assert ex <= max(1, 1e-4 * dec)


def test_draft_sample_parity():
    psi = _psi()
    for (wl, T, B) in [("tiny", 1.0, 64), ("qwen", 0.7, 8)]:
        p, q = synth.linear_inputs(wl, seed=1, B=B)
        for step in range(3):
            g = psi.draft_sample(to_dev(q), temperature=T, seed=7, step=step).cpu().numpy()
            o, mg = oracle.draft_sample(q, f32(T), seed=7, step=step, nthreads=THREADS)
            bad = g != o
            assert np.all(mg[bad] < 1e-11), (np.argwhere(bad), mg[bad])


def test_fused_equals_draft_then_verify():
    """Fusing the draft draw into verification gives the same bits as
    psispec_draft_sample followed by a non-fused verify."""
    psi = _psi()
    p, q = synth.linear_inputs("qwen", seed=2, B=16)
    pd, qd = to_dev(p), to_dev(q)
    for step in range(2):
        f = psi.verify_linear(pd, qd, None, temperature=0.7, seed=5, step=step, fused=True)
        d = psi.draft_sample(qd, temperature=0.7, seed=5, step=step)
        n = psi.verify_linear(pd, qd, d, temperature=0.7, seed=5, step=step)
        torch.cuda.synchronize()
        assert torch.equal(f["draft"], d)
        for k in ("tokens", "len", "probs", "resid"):
            assert torch.equal(f[k], n[k])


def test_deterministic_repeat():
    psi = _psi()
    p, q = synth.linear_inputs("highconc", seed=4, B=32)
    pd, qd = to_dev(p), to_dev(q)
    d = psi.draft_sample(qd, temperature=1.0, seed=1, step=0)
    a = psi.verify_linear(pd, qd, d, temperature=1.0, seed=1, step=0)
    a = {k: v.clone() for k, v in a.items() if v is not None}
    b = psi.verify_linear(pd, qd, d, temperature=1.0, seed=1, step=0)
    torch.cuda.synchronize()
    for k in ("tokens", "len", "probs", "resid"):
        assert torch.equal(a[k], b[k])


@pytest.mark.parametrize("dtype,V", [("f32", 1000), ("bf16", 1001), ("bf16", 5000), ("f32", 1), ("bf16", 7)])
def test_ragged_and_unaligned_vocab(dtype, V):
    """Vocabulary sizes that are not multiples of the vector width or of the
    chunk (unaligned path, ragged tails, V = 1)."""
    B, K = 24, 3
    p, q = synth.pair(B, K + 1, K, V, dtype, seed=9, sd_a=2.0, mode=0, sd_noise=0.7)
    for step in range(2):
        g, o = _run_pair(p, q, None, 1.0, 3, step, True)
        ex, dec, _ = compare_linear(g, o)
        assert ex <= 1


@pytest.mark.parametrize("K", [1, 64])
def test_k_extremes(K):
    B, V = 8, 2048
    p, q = synth.pair(B, K + 1, K, V, "bf16", seed=K, sd_a=1.0, mode=1, rho=0.98, sd_noise=1.0)
    g, o = _run_pair(p, q, None, 1.0, 0, 0, True)
    ex, dec, _ = compare_linear(g, o)
    assert ex <= 1


def test_request_errors_and_special_rows():
    """NaN, +inf, all -inf rows and out-of-range drafts give len -1 on exactly
    those requests; identical target/draft rows are always accepted."""
    B, K, V = 8, 4, 3000
    p, q = synth.pair(B, K + 1, K, V, "f32", seed=3, sd_a=2.0, mode=0, sd_noise=0.5)
    p[1, 4, 17] = np.nan
    q[2, 0, 3] = np.inf
    p[3, 2, :] = -np.inf
    q[5, 1, :100] = -np.inf  # partially -inf is fine
    q[6] = p[6, :K]  # identical rows: always accepted
    d, _ = oracle.draft_sample(q, 1.0, seed=0, step=0)
    d[4, 1] = V  # out of range
    d[7, 0] = -3
    g, o = _run_pair(p, q, d, 1.0, 0, 0, False)
    gl = g["len"].cpu().numpy()
    assert list(gl[[1, 2, 3, 4, 7]]) == [-1] * 5
    assert np.all(g["tokens"].cpu().numpy()[[1, 2, 3, 4, 7]] == -1)
    assert gl[6] == K
    compare_linear(g, o)


def _bf16_bits(f: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _bf16_float(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_bf16_weight_window_edges(T):
    """bfloat16 rows full of logits that are zero or below 2^-26 in magnitude
    (weights outside the table, corrected exactly), logits at the edges of the
    table window (+-63.25 inside, -63.5 and beyond outside), rows whose
    maximum disables the table (above 63.25, or too small a spread), and
    pairs that mix both kinds: lengths, tokens and residual masses match."""
    B, K, V = 32, 4, 4096
    p, q = synth.pair(B, K + 1, K, V, "bf16", seed=21, sd_a=2.0, mode=0, sd_noise=1.0)
    fp, fq = _bf16_float(p).copy(), _bf16_float(q).copy()
    rng = np.random.default_rng(77)
    tiny = np.array([0.0, -0.0, 2.0 ** -30, -(2.0 ** -30), 2.0 ** -27, -(2.0 ** -40)], np.float32)
    edge = np.array([-63.25, -63.5, -64.0, -70.0, -1.0e4], np.float32)
    for f in (fp, fq):
        m = rng.random(f.shape) < 0.08
        f[m] = rng.choice(tiny, size=int(m.sum()))
        m = rng.random(f.shape) < 0.01
        f[m] = rng.choice(edge, size=int(m.sum()))
    for b in range(B):
        kind = b % 4
        if kind == 1:  # draft rows peak at the top of the window
            fq[b, :, 5] = 63.25
        elif kind == 2:  # target rows peak above the window: no table for the pair
            fp[b, :, 9] = 63.5
        elif kind == 3:  # too small a spread for the table
            fp[b] *= np.float32(0.25)
            fq[b] *= np.float32(0.25)
    p, q = _bf16_bits(fp), _bf16_bits(fq)
    for step in range(3):
        g, o = _run_pair(p, q, None, T, 4, step, True)
        ex, dec, _ = compare_linear(g, o)
        assert ex <= 1
        assert int((o["len"] < K).sum()) > 0  # residual draws happen


def test_greedy_parity():
    """Greedy mode (temperature 0) on the filtered/greedy workload shape, fused
    drafts (argmax of q) and given drafts."""
    p, q = synth.linear_inputs("greedy", seed=0, B=32)
    g, o = _run_pair(p, q, None, 0.0, 0, 0, True)
    assert np.array_equal(g["tokens"].cpu().numpy(), o["tokens"])
    assert np.array_equal(g["len"].cpu().numpy(), o["len"])
    rng = np.random.default_rng(0)
    d = o["draft"].copy()
    flip = rng.random(d.shape) < 0.2
    d[flip] = rng.integers(0, p.shape[2], flip.sum())
    g, o = _run_pair(p, q, d, 0.0, 0, 0, False)
    assert np.array_equal(g["tokens"].cpu().numpy(), o["tokens"])
    assert np.array_equal(g["len"].cpu().numpy(), o["len"])
    assert np.array_equal(g["probs"].cpu().numpy(), o["probs"].astype(np.float32))


def test_gpu_law_many_replicas():
    """10^5 replicas of a V=8, K=2 case in one call: accept-length histogram
    matches the closed form and the first token follows P_0 (chi-square)."""
    psi = _psi()
    rng = np.random.default_rng(21)
    a = rng.normal(0, 1.5, (1, 3, 8)).astype(np.float32)
    d = (a[:, :2] + rng.normal(0, 1.0, (1, 2, 8))).astype(np.float32)
    B = 100_000
    pd = to_dev(np.repeat(a, B, axis=0))
    qd = to_dev(np.repeat(d, B, axis=0))
    g = psi.verify_linear(pd, qd, None, temperature=1.0, seed=123, step=0, fused=True)
    n = g["len"].cpu().numpy()
    first = g["tokens"][:, 0].cpu().numpy()
    P = [probs(a[0, i]) for i in range(3)]
    Q = [probs(d[0, i]) for i in range(2)]
    al = [alpha(P[i], Q[i]) for i in range(2)]
    law = np.array([1 - al[0], al[0] * (1 - al[1]), al[0] * al[1]])
    assert chi2_pvalue(np.bincount(n, minlength=3), law * B) > 1e-3
    assert chi2_pvalue(np.bincount(first, minlength=8), P[0] * B) > 1e-3
