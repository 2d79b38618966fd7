"""GPU parity of filters whose kept set has no small bound (top-p without a
top-k, top_k above 256, top_k >= V with a top-p) against the CPU oracle:
verification with fused drafts, draft sampling alone, ties at the cut,
constant rows, invalid rows, and the filtered workload's full size with
top_k = 0, top_p = 0.95."""
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


def test_wide_full_size_top_p_alone():
    """Filtered workload shape, B=128, K=16, V=128256, fp32, T=1, with
    top_k = 0 and top_p = 0.95 (the kept set runs to thousands of tokens)."""
    p, q = synth.linear_inputs("filtered", seed=0)
    tot = Tally("top-p alone full size x2")
    for step in range(2):
        print(f"[wide] full size step {step}", flush=True)
        g, o = _run(p, q, None, 1.0, 0, 0.95, 0, step, True)
        tot += compare_linear(g, o, fused=True)
    tot.check()


@pytest.mark.parametrize("dtype,V,T,top_k,top_p", [
    ("f32", 3000, 1.0, 0, 0.9),        # top-p alone
    ("bf16", 5000, 1.3, 0, 0.99),
    ("f32", 777, 2.0, 300, 0.999),     # ragged V, top-k above 256 and top-p
    ("bf16", 20000, 1.0, 1000, 1.0),   # top-k above 256 alone
    ("bf16", 4099, 0.7, 5000, 0.5),    # top_k >= V: top-p alone
    ("f32", 70000, 1.0, 257, 0.95),
    ("bf16", 9000, 1.0, 0, 0.01),      # the cut keeps one or two tokens
    ("f32", 2048, 0.5, 0, 0.999999)])  # the cut lies deep in the tail
def test_wide_small(dtype, V, T, top_k, top_p):
    B, K = 24, 4
    p, q = synth.pair(B, K + 1, K, V, dtype, seed=V + top_k, sd_a=2.0, mode=0, sd_noise=0.6)
    tot = Tally(f"wide {dtype} V={V} k={top_k} p={top_p}")
    for step in range(3):
        print(f"[wide] {dtype} V={V} k={top_k} p={top_p} step {step}", flush=True)
        g, o = _run(p, q, None, T, top_k, top_p, 11, step, True)
        tot += compare_linear(g, o, fused=True)
    tot.check()


@pytest.mark.parametrize("top_k,top_p", [(0, 0.8), (300, 1.0), (300, 0.7), (0, 0.3)])
def test_wide_ties(top_k, top_p):
    """Logits on a coarse grid: many tokens share the cut's logit, and the
    lower ids among them are kept."""
    B, K, V = 16, 3, 4000
    p, q = synth.pair(B, K + 1, K, V, "f32", seed=5, sd_a=2.0, mode=0, sd_noise=0.5)
    p = (np.round(p * 2) / 2).astype(np.float32)
    q = (np.round(q * 2) / 2).astype(np.float32)
    for step in range(4):
        print(f"[wide] ties k={top_k} p={top_p} step {step}", flush=True)
        g, o = _run(p, q, None, 1.0, top_k, top_p, 2, step, True)
        compare_linear(g, o, fused=True, name=f"wide ties k={top_k} p={top_p}").check()


def test_wide_constant_rows():
    """Constant rows: every token ties, so top-p keeps the first
    ceil(top_p V) ids and top-k the first top_k ids."""
    B, K, V = 6, 3, 3000
    p, q = synth.pair(B, K + 1, K, V, "f32", seed=21, sd_a=2.0, mode=0, sd_noise=0.5)
    p[0] = 0.75
    q[0] = 0.75
    q[1] = -2.0
    p[2, :, :] = 1.0
    for top_k, top_p in ((0, 0.6), (700, 1.0), (400, 0.5)):
        g, o = _run(p, q, None, 1.0, top_k, top_p, 9, 0, True)
        compare_linear(g, o, fused=True, name=f"wide constant k={top_k} p={top_p}").check()
        assert int(g["len"][0]) == K  # identical rows always accept
        kept = min(top_k or V, int(np.ceil(np.float32(top_p) * (top_k or V) - 1e-9)))
        assert 0 <= int(g["tokens"][0, K]) < kept + 1  # + 1: the running sum may round below top_p


def test_wide_draft_sample():
    psi = _psi()
    p, q = synth.linear_inputs("filtered", seed=1, B=8)
    for top_k, top_p in ((0, 0.95), (1000, 0.9), (500, 1.0)):
        tot = Tally(f"wide draft sample k={top_k} p={top_p}")
        for step in range(2):
            g = psi.draft_sample(to_dev(q), temperature=1.0, top_k=top_k, top_p=f32(top_p), seed=3, step=step)
            o, om = oracle.draft_sample(q, 1.0, top_k=top_k, top_p=f32(top_p), seed=3, step=step, nthreads=THREADS)
            tot += compare_drafts(g, o, om)
        tot.check()


def test_wide_given_drafts():
    """Drafts passed in (not fused): the cuts of the q rows still decide Q(x)."""
    B, K, V = 12, 5, 6000
    p, q = synth.pair(B, K + 1, K, V, "bf16", seed=4, sd_a=2.0, mode=0, sd_noise=0.6)
    rng = np.random.default_rng(0)
    draft = rng.integers(0, V, size=(B, K), dtype=np.int32)
    draft[:, 0] = np.argmax(synth.bf16_to_f32(q[:, 0]), axis=-1)  # a kept token at position 0
    tot = Tally("wide given drafts")
    for step in range(3):
        g, o = _run(p, q, draft, 1.0, 0, 0.9, 6, step, False)
        tot += compare_linear(g, o, fused=False)
    tot.check()


def test_wide_errors():
    B, K, V = 6, 3, 2000
    p, q = synth.pair(B, K + 1, K, V, "f32", seed=8, sd_a=2.0, mode=0, sd_noise=0.5)
    p[1, 2, 5] = np.nan
    q[2, 0, :] = -np.inf
    p[3, 3, 7] = np.inf
    g, o = _run(p, q, None, 1.0, 0, 0.9, 0, 0, True)
    gl = g["len"].cpu().numpy()
    assert list(gl[[1, 2, 3]]) == [-1, -1, -1]
    compare_linear(g, o, fused=True, name="wide errors").check()
