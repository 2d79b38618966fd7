"""GPU parity of filtered sampling (temperature -> top-k -> top-p ->
renormalise) against the CPU oracle: verification and draft sampling, at the
filtered workload's full size and on small cases with ties."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import THREADS, Tally, compare_drafts, compare_linear, f32, to_dev

pytestmark = pytest.mark.gpu


def _psi():
    import lossless_speculative_verification_amd as psi
    return psi


def _run(p, q, draft, T, top_k, top_p, seed, step, fused):
    psi = _psi()
    T, top_p = f32(T), f32(top_p)
    dd = None if draft is None else torch.from_numpy(np.ascontiguousarray(draft, dtype=np.int32)).cuda()
    g = psi.verify_linear(to_dev(p), to_dev(q), dd, temperature=T, top_k=top_k, top_p=top_p, seed=seed, step=step,
                          fused=fused)
    torch.cuda.synchronize()
    o = oracle.verify_linear(p, q, draft, T, top_k=top_k, top_p=top_p, seed=seed, step=step, fused=fused,
                             nthreads=THREADS)
    return g, o


def test_filtered_full_size():
    """Filtered workload at full size: B=128, K=16, V=128256, fp32, T=1, top_k=50, top_p=0.95, fused drafts."""
    p, q = synth.linear_inputs("filtered", seed=0)
    tot = Tally("filtered full size x2")
    for step in range(2):
        g, o = _run(p, q, None, 1.0, 50, 0.95, 0, step, True)
        tot += compare_linear(g, o, fused=True)
    tot.check()


@pytest.mark.parametrize("dtype,V,T,top_k,top_p", [
    ("f32", 3000, 1.0, 5, 1.0), ("f32", 3000, 0.7, 40, 0.6), ("bf16", 5000, 1.3, 256, 0.99),
    ("bf16", 1001, 1.0, 3, 0.3), ("f32", 777, 2.0, 17, 0.999), ("bf16", 20000, 1.0, 100, 0.9)])
def test_filtered_small(dtype, V, T, top_k, top_p):
    B, K = 24, 4
    p, q = synth.pair(B, K + 1, K, V, dtype, seed=V, sd_a=2.0, mode=0, sd_noise=0.6)
    tot = Tally(f"filtered {dtype} V={V} k={top_k} p={top_p}")
    for step in range(3):
        g, o = _run(p, q, None, T, top_k, top_p, 11, step, True)
        tot += compare_linear(g, o, fused=True)
    tot.check()


def test_filtered_ties():
    """Logits rounded to a coarse grid (many exact ties): top-k keeps the lower ids."""
    B, K, V = 16, 3, 4000
    p, q = synth.pair(B, K + 1, K, V, "f32", seed=5, sd_a=2.0, mode=0, sd_noise=0.5)
    p = np.round(p * 2) / 2
    q = np.round(q * 2) / 2
    for step in range(4):
        g, o = _run(p.astype(np.float32), q.astype(np.float32), None, 1.0, 30, 0.8, 2, step, True)
        assert np.array_equal(g["draft"].cpu().numpy(), o["draft"])
        compare_linear(g, o, fused=True, name="filtered ties").check()
        assert np.array_equal(g["tokens"].cpu().numpy(), o["tokens"])


def test_filtered_candidate_overflow():
    """Rows whose top-k candidates overflow: constant rows (every logit ties,
    so every chunk is read again and the whole row is streamed) and rows with
    300 copies of their maximum spread over three chunks (the lowest ids win
    the ties across chunks)."""
    B, K, V = 8, 3, 40000
    p, q = synth.pair(B, K + 1, K, V, "f32", seed=13, sd_a=2.0, mode=0, sd_noise=0.5)
    rng = np.random.default_rng(3)
    p[0] = 1.5
    q[0] = 1.5
    for r in range(K + 1):
        p[1, r, rng.choice(V, 300, replace=False)] = p[1, r].max() + 1.0
    for r in range(K):
        q[1, r, rng.choice(V, 300, replace=False)] = q[1, r].max() + 1.0
    q[2] = -0.25
    for step in range(3):
        g, o = _run(p, q, None, 1.0, 20, 0.53, 5, step, True)
        assert np.array_equal(g["draft"].cpu().numpy(), o["draft"])
        compare_linear(g, o, fused=True, name="filtered overflow").check()
        assert np.array_equal(g["tokens"].cpu().numpy(), o["tokens"])
        assert int(g["len"][0]) == K  # identical constant rows always accept


def test_filtered_chunk_bound_raised():
    """Chunks whose large logits sit in a few threads' elements: the first
    bound admits hundreds of candidates and is raised by bisection (distinct
    values) or leaves the chunk to be read again (tied values)."""
    B, K, V = 4, 2, 40000
    p, q = synth.pair(B, K + 1, K, V, "f32", seed=17, sd_a=2.0, mode=0, sd_noise=0.5)
    # fp32 chunk of 16384 logits: thread t holds vectors t + 256 k (k < 16) of
    # 4 logits, i.e. logits (t + 256 k) * 4 + e
    idx = np.array([(t + 256 * k) * 4 + e for t in range(13) for k in range(16) for e in range(4)])
    for b in range(B):
        for r in range(K + 1):
            for ch in (0, 1):
                vals = 9.0 + 0.001 * np.arange(idx.size) if (b + r) % 2 == 0 else np.full(idx.size, 9.5)
                p[b, r, ch * 16384 + idx] = vals.astype(np.float32)
    for step in range(3):
        g, o = _run(p, q, None, 1.0, 50, 0.9, 8, step, True)
        assert np.array_equal(g["draft"].cpu().numpy(), o["draft"])
        compare_linear(g, o, fused=True, name="filtered chunk bound").check()
        assert np.array_equal(g["tokens"].cpu().numpy(), o["tokens"])


def test_top_k_one_matches_greedy():
    """top_k = 1 stochastic verification with fused drafts equals greedy mode."""
    psi = _psi()
    p, q = synth.linear_inputs("greedy", seed=3, B=16)
    pd, qd = to_dev(p), to_dev(q)
    a = psi.verify_linear(pd, qd, None, temperature=1.0, top_k=1, seed=4, step=0, fused=True)
    b = psi.verify_linear(pd, qd, None, temperature=0.0, fused=True)
    torch.cuda.synchronize()
    assert torch.equal(a["tokens"], b["tokens"]) and torch.equal(a["len"], b["len"])


def test_filtered_draft_sample():
    psi = _psi()
    p, q = synth.linear_inputs("filtered", seed=1, B=8)
    tot = Tally("filtered draft sample")
    for step in range(3):
        g = psi.draft_sample(to_dev(q), temperature=1.0, top_k=50, top_p=f32(0.95), seed=3, step=step)
        o, om = oracle.draft_sample(q, 1.0, top_k=50, top_p=f32(0.95), seed=3, step=step, nthreads=THREADS)
        tot += compare_drafts(g, o, om)
    tot.check()


def test_filtered_errors():
    B, K, V = 6, 3, 2000
    p, q = synth.pair(B, K + 1, K, V, "f32", seed=8, sd_a=2.0, mode=0, sd_noise=0.5)
    p[1, 2, 5] = np.nan
    q[2, 0, :] = -np.inf
    p[3, 3, 7] = np.inf
    g, o = _run(p, q, None, 1.0, 20, 0.9, 0, 0, True)
    gl = g["len"].cpu().numpy()
    assert list(gl[[1, 2, 3]]) == [-1, -1, -1]
    compare_linear(g, o, fused=True, name="filtered errors").check()
