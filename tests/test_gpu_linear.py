"""GPU parity of psispec_verify_linear / psispec_draft_sample against the CPU
oracle, element by element on the same seeded inputs: accepted lengths and
tokens bit-exact except requests whose first differing decision is an oracle
near tie (gpu_helpers), counted; probabilities within 1e-5 relative, residual
masses within 1e-9 relative."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import PROB_RTOL, RESID_RTOL, THREADS, Tally, compare_drafts, compare_linear, f32, to_dev
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
    tot = Tally("tiny x300")
    for t in range(300):
        g, o = _run_pair(p, q, None, 1.0, 0, t, True)
        tot += compare_linear(g, o, fused=True)
    tot.check()


def test_tiny_replicas_one_call():
    """2000 replicas of the tiny workload in one call (request id keys the
    random stream): parity with the oracle on every replica."""
    p, q = synth.linear_inputs("tiny", seed=0)
    B = 2000
    p = np.ascontiguousarray(np.repeat(p, B, axis=0))
    q = np.ascontiguousarray(np.repeat(q, B, axis=0))
    g, o = _run_pair(p, q, None, 1.0, 0, 0, True)
    compare_linear(g, o, fused=True, name="tiny 2000 replicas").check()


@pytest.mark.parametrize("rho", [0.5, 0.8, 0.95])
def test_highconc_full_size(rho):
    """High-concurrency workload at full size (B=256, K=8, V=151936, bf16, T=1)
    in the benchmark's launch configuration, over steps 0..19: the drafts of
    each step drawn on the GPU (psispec_draft_sample, 2048 draws) and checked
    against the oracle's, then verified on both sides from the GPU's drafts.
    Near ties must make up less than 1e-4 of the decisions."""
    psi = _psi()
    p, q = synth.linear_inputs("highconc", seed=0, rho=rho)
    pd, qd = to_dev(p), to_dev(q)
    td, tv = Tally(f"highconc rho {rho} drafts"), Tally(f"highconc rho {rho} verify")
    for step in range(20):
        gd = psi.draft_sample(qd, temperature=1.0, seed=0, step=step)
        g = psi.verify_linear(pd, qd, gd, temperature=1.0, seed=0, step=step)
        torch.cuda.synchronize()
        od, om = oracle.draft_sample(q, 1.0, seed=0, step=step, nthreads=THREADS)
        td += compare_drafts(gd, od, om)
        d = gd.cpu().numpy()
        o = oracle.verify_linear(p, q, d, 1.0, seed=0, step=step, nthreads=THREADS)
        tv += compare_linear(g, o)
    td.check(near_fraction=True)
    tv.check(near_fraction=True)
    both = Tally(f"highconc rho {rho}")
    both += td
    both += tv
    both.check(near_fraction=True)
    assert both.decisions >= 40960


def test_qwen_fused_full_size():
    """Qwen3-8B-shaped workload (B=64, K=8, V=151936, bf16, T=0.7) with fused drafts, 4 steps."""
    p, q = synth.linear_inputs("qwen", seed=0)
    tot = Tally("qwen fused x4")
    for step in range(4):
        g, o = _run_pair(p, q, None, 0.7, 0, 3 + step, True)
        tot += compare_linear(g, o, fused=True)
    tot.check()


def test_draft_sample_parity():
    psi = _psi()
    tot = Tally("draft sample")
    for (wl, T, B) in [("tiny", 1.0, 64), ("qwen", 0.7, 8)]:
        p, q = synth.linear_inputs(wl, seed=1, B=B)
        for step in range(3):
            g = psi.draft_sample(to_dev(q), temperature=T, seed=7, step=step)
            o, om = oracle.draft_sample(q, f32(T), seed=7, step=step, nthreads=THREADS)
            tot += compare_drafts(g, o, om)
    tot.check()


@pytest.mark.parametrize("wl,T", [("qwen", 0.7), ("tiny", 1.0)])
def test_fused_equals_draft_then_verify(wl, T):
    """Fusing the draft draw into verification draws the same drafts, bit for
    bit, as psispec_draft_sample, and verifies them to the same lengths and
    tokens as a non-fused verify. The draft rows' normalisers differ in their
    last bits (bfloat16 fused drafting sums exact fp64 weights in its one pass
    over each draft row; the non-fused call uses the binary32-grade
    statistics), so probabilities agree to 1e-5 and residual masses to 1e-9."""
    psi = _psi()
    p, q = synth.linear_inputs(wl, seed=2, B=16)
    pd, qd = to_dev(p), to_dev(q)
    for step in range(3):
        f = psi.verify_linear(pd, qd, None, temperature=T, seed=5, step=step, fused=True)
        d = psi.draft_sample(qd, temperature=T, seed=5, step=step)
        n = psi.verify_linear(pd, qd, d, temperature=T, seed=5, step=step)
        torch.cuda.synchronize()
        assert torch.equal(f["draft"], d)
        for k in ("tokens", "len"):
            assert torch.equal(f[k], n[k])
        np.testing.assert_allclose(f["probs"].cpu().numpy(), n["probs"].cpu().numpy(), rtol=PROB_RTOL, atol=0)
        np.testing.assert_allclose(f["resid"].cpu().numpy(), n["resid"].cpu().numpy(), rtol=RESID_RTOL, atol=0)


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
    tot = Tally(f"ragged {dtype} V={V}")
    for step in range(2):
        g, o = _run_pair(p, q, None, 1.0, 3, step, True)
        tot += compare_linear(g, o, fused=True)
    tot.check()


@pytest.mark.parametrize("K", [1, 64])
def test_k_extremes(K):
    B, V = 8, 2048
    p, q = synth.pair(B, K + 1, K, V, "bf16", seed=K, sd_a=1.0, mode=1, rho=0.98, sd_noise=1.0)
    g, o = _run_pair(p, q, None, 1.0, 0, 0, True)
    compare_linear(g, o, fused=True, name=f"K={K}").check()


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
    compare_linear(g, o, name="request errors").check()


def test_bf16_draft_row_errors():
    """bfloat16 draft rows holding a positive or a negative NaN, +inf, or only
    -inf make their request invalid, both in draft sampling alone and with the
    drafts fused into verification (one pass over each draft row); a partly
    -inf draft row is valid."""
    psi = _psi()
    B, K, V = 8, 3, 5000
    p, q = synth.pair(B, K + 1, K, V, "bf16", seed=12, sd_a=2.0, mode=0, sd_noise=0.7)
    q[1, 0, 17] = 0x7FC0   # NaN
    q[2, 2, 4000] = 0xFFC1  # NaN with the sign bit set
    q[3, 1, 9] = 0x7F80    # +inf
    q[4, 0, :] = 0xFF80    # all -inf
    q[5, 2, :2500] = 0xFF80  # partly -inf: valid
    bad = [1, 2, 3, 4]
    for step in range(2):
        d = psi.draft_sample(to_dev(q), temperature=1.0, seed=3, step=step).cpu().numpy()
        o, om = oracle.draft_sample(q, 1.0, seed=3, step=step, nthreads=THREADS)
        assert np.all(d[bad] == -1) and np.all(o[bad] == -1)
        compare_drafts(d, o, om, name="bf16 draft row errors").check()
        g, og = _run_pair(p, q, None, 1.0, 3, step, True)
        assert list(g["len"].cpu().numpy()[bad]) == [-1] * 4
        assert np.all(g["len"].cpu().numpy()[[0, 5, 6, 7]] >= 0)
        compare_linear(g, og, fused=True, name="bf16 fused draft row errors").check()


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
    edge = np.array([-63.25, -63.5, -63.75, -64.0, -70.0, -1.0e4], np.float32)
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
    tot = Tally(f"bf16 window edges T={T}")
    for step in range(3):
        g, o = _run_pair(p, q, None, T, 4, step, True)
        tot += compare_linear(g, o, fused=True)
        assert int((o["len"] < K).sum()) > 0  # residual draws happen
    tot.check()


def test_bf16_window_top_one_workgroup_resolve():
    """Requests enough for one resolve workgroup each (B=192), bfloat16 rows
    inside the table window except for a few logits just above it in
    magnitude (-63.5 and -63.75, the last two codes before -64, which weigh
    zero under the table rule) and fewer still beyond it (-64, -1e4): most
    16-byte vector pairs have every code inside the window, some carry the
    codes just above it, a few take the general slot computation. Given
    drafts, three steps: lengths, tokens and residual masses match."""
    B, K, V = 192, 4, 4096
    p, q = synth.pair(B, K + 1, K, V, "bf16", seed=23, sd_a=3.0, mode=0, sd_noise=1.0)
    fp, fq = _bf16_float(p).copy(), _bf16_float(q).copy()
    rng = np.random.default_rng(78)
    for f in (fp, fq):
        m = rng.random(f.shape) < 0.004
        f[m] = rng.choice(np.array([-63.5, -63.75], np.float32), size=int(m.sum()))
        m = rng.random(f.shape) < 0.0005
        f[m] = rng.choice(np.array([-64.0, -1.0e4], np.float32), size=int(m.sum()))
    p, q = _bf16_bits(fp), _bf16_bits(fq)
    drafts, _ = oracle.draft_sample(q, 1.0, seed=5, step=0, nthreads=THREADS)
    tot = Tally("bf16 window top, one workgroup per request")
    for step in range(3):
        g, o = _run_pair(p, q, drafts, 1.0, 5, step, False)
        tot += compare_linear(g, o, fused=False)
        assert int((o["len"] < K).sum()) > 0  # residual draws happen
    tot.check()


def test_greedy_parity():
    """Greedy mode (temperature 0) on the filtered/greedy workload at full size
    (B=128, K=16, V=128256, fp32): fused drafts (argmax of q), then given
    drafts with a fifth of them replaced. Argmaxes compare exact values, so
    everything must match exactly."""
    p, q = synth.linear_inputs("greedy", seed=0)
    assert p.shape == (128, 17, 128256)
    g, o = _run_pair(p, q, None, 0.0, 0, 0, True)
    assert np.array_equal(g["draft"].cpu().numpy(), o["draft"])
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
    assert int((o["len"] < 16).sum()) > 0  # rejections happen


def test_gpu_law_many_replicas():
    """10^6 replicas of a V=8, K=2 case in one call: the accept-length
    histogram matches the closed form (1 - a_0, a_0 (1 - a_1), a_0 a_1), the
    first emitted token follows P_0 and, on the replicas that reach position 1,
    the second emitted token follows P_1 (chi-square)."""
    psi = _psi()
    rng = np.random.default_rng(21)
    a = rng.normal(0, 1.5, (1, 3, 8)).astype(np.float32)
    d = (a[:, :2] + rng.normal(0, 1.0, (1, 2, 8))).astype(np.float32)
    B = 1_000_000
    pd = to_dev(np.repeat(a, B, axis=0))
    qd = to_dev(np.repeat(d, B, axis=0))
    g = psi.verify_linear(pd, qd, None, temperature=1.0, seed=123, step=0, fused=True)
    n = g["len"].cpu().numpy()
    tok = g["tokens"].cpu().numpy()
    P = [probs(a[0, i]) for i in range(3)]
    Q = [probs(d[0, i]) for i in range(2)]
    al = [alpha(P[i], Q[i]) for i in range(2)]
    law = np.array([1 - al[0], al[0] * (1 - al[1]), al[0] * al[1]])
    assert chi2_pvalue(np.bincount(n, minlength=3), law * B) > 1e-3
    assert chi2_pvalue(np.bincount(tok[:, 0], minlength=8), P[0] * B) > 1e-3
    reach = n >= 1
    assert chi2_pvalue(np.bincount(tok[reach, 1], minlength=8), P[1] * int(reach.sum())) > 1e-3


def test_philox_sweep_against_oracle():
    """The GPU's Philox4x32-10 uniforms equal the oracle's on 1,048,576
    counters. With equal logits over V = 65536 tokens an inverse-CDF draw lands
    on floor(u * 65536), so each draft draw shows the top 16 bits of
    U(seed, step, b, i, 0x40000000); identical target rows accept every draft,
    so the bonus draw shows those of U(seed, step, b, K, 0)."""
    psi = _psi()
    B, K, V = 256, 15, 65536
    seed = 0x0123456789ABCDEF
    p = torch.zeros((B, K + 1, V), dtype=torch.float32, device="cuda")
    q = torch.zeros((B, K, V), dtype=torch.float32, device="cuda")
    bad = 0
    for step in range(256):
        g = psi.verify_linear(p, q, None, temperature=1.0, seed=seed, step=step, fused=True)
        torch.cuda.synchronize()
        drafts = g["draft"].cpu().numpy()
        assert np.all(g["len"].cpu().numpy() == K)
        bonus = g["tokens"].cpu().numpy()[:, K]
        want_d = np.array([[int(oracle.uniform(seed, step, b, i, oracle.DRAFT_DRAW) * V) for i in range(K)]
                           for b in range(B)])
        want_b = np.array([int(oracle.uniform(seed, step, b, K, 0) * V) for b in range(B)])
        bad += int((drafts != want_d).sum() + (bonus != want_b).sum())
    assert bad == 0


def test_timing_hook_two_events_per_kernel():
    """The benchmark timing hook: an armed verification call launches each of
    its kernels with a start and a stop event, two per kernel (statistics pass
    and resolve at one workgroup per request: four); the durations are
    positive, and the outputs equal those of the same call unarmed."""
    psi = _psi()
    B, K, V = 192, 4, 4096
    p, q = synth.pair(B, K + 1, K, V, "bf16", seed=31, sd_a=3.0, mode=0, sd_noise=1.0)
    pd, qd = to_dev(p), to_dev(q)
    drafts, _ = oracle.draft_sample(q, 1.0, seed=2, step=0, nthreads=THREADS)
    dd = torch.from_numpy(drafts.astype(np.int32)).cuda()
    plain = psi.verify_linear(pd, qd, dd, temperature=1.0, seed=2, step=0)
    timer = psi.KernelTimer(3, 4)
    for i in range(3):
        timer.arm(i)
        g = psi.verify_linear(pd, qd, dd, temperature=1.0, seed=2, step=0)
        timer.note()
    timer.disarm()
    torch.cuda.synchronize()
    assert timer.recorded == [4, 4, 4]
    dur = timer.durations()
    assert dur.shape == (3, 4) and np.isfinite(dur[:, :2]).all() and (dur[:, :2] > 0).all()
    assert np.isnan(dur[:, 2:]).all()  # two kernels: the last two slots stay unused
    assert torch.equal(g["tokens"], plain["tokens"]) and torch.equal(g["len"], plain["len"])
