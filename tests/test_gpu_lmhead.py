"""GPU parity of linear verification fused with the LM head: hidden states and
a vocabulary matrix in, the verification's tokens and lengths out, against the
oracle's logits (exact products summed in fp64) fed to the oracle's linear
verification. Ragged vocabularies and row counts, several temperatures, and
the Qwen3-8B head shape (H = 4096, V = 151,936)."""
from __future__ import annotations

import numpy as np
import pytest
import torch
from scipy.special import softmax

import oracle
import synth
from gpu_helpers import THREADS, Tally, f32

pytestmark = pytest.mark.gpu

# The GPU's logits carry the fp32 accumulation error of an H-term dot product
# of bf16 values, bounded in tests/test_lmhead_error.py by emulating fp32
# accumulation on the CPU: at most 5e-5 absolute at H = 4096 for these inputs,
# summing one product at a time). A probability moves by at most twice that,
# relative, and a ratio P/Q or a CDF edge by at most four times that, so an
# accept test may differ only where |u - min(1, P/Q)| < BAND_ACC, and a final
# draw may land on any token whose interval of the oracle's CDF comes within
# BAND_CDF of the mass of u*W (the draw is then checked for validity, not
# identity).
BAND_ACC = 2.5e-4
BAND_CDF = 2.5e-4


def _psi():
    import lossless_speculative_verification_amd as psi
    return psi


def _bf16(x: np.ndarray) -> np.ndarray:
    return synth.f32_to_bf16(np.ascontiguousarray(x, dtype=np.float32))


def _dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def inputs(B, K, H, V, seed, sd_w=0.05, noise=0.3):
    """Target hidden states ~ N(0, 1), draft hidden states = target + noise,
    vocabulary rows ~ N(0, sd_w^2) with a few rows scaled up (heavy tokens)."""
    rng = np.random.default_rng(seed)
    ht = rng.normal(0, 1, (B, K + 1, H)).astype(np.float32)
    hd = ht[:, :K] + rng.normal(0, noise, (B, K, H)).astype(np.float32)
    w = rng.normal(0, sd_w, (V, H)).astype(np.float32)
    heavy = rng.choice(V, size=min(V, 20), replace=False)
    w[heavy] *= 3.0
    return _bf16(ht), _bf16(hd), _bf16(w)


def _final_weights(zp, zq, b, n, K, T):
    """The oracle's final-draw weights of request b (fp64, from its logits)."""
    P = softmax(zp[b, n].astype(np.float64) / T)
    if n == K:
        return P
    w = np.maximum(P - softmax(zq[b, n].astype(np.float64) / T), 0.0)
    return w if w.sum() > 0 else P


def check(B, K, H, V, T, seed, steps=3) -> Tally:
    """Per request: the GPU's accepted length equals the oracle's unless the
    first accept test where they part is within BAND_ACC; with equal lengths,
    the GPU's final token is the oracle's, or one whose CDF interval lies
    within BAND_CDF of the oracle's target mass u*W."""
    psi = _psi()
    ht, hd, w = inputs(B, K, H, V, seed)
    zp = oracle.lmhead_logits(ht, w)
    zq = oracle.lmhead_logits(hd, w)
    dt, dd, dw = _dev(ht), _dev(hd), _dev(w)
    t = Tally(f"lmhead B={B} K={K} H={H} V={V} T={T}")
    for step in range(steps):
        x, _ = oracle.draft_sample(zq, T, seed=seed, step=step, nthreads=THREADS)
        g = psi.verify_lmhead(dt, dd, dw, torch.from_numpy(x).cuda(), temperature=T, seed=seed, step=step)
        torch.cuda.synchronize()
        o = oracle.verify_linear(zp, zq, x, T, seed=seed, step=step, nthreads=THREADS)
        gl, gt = g["len"].cpu().numpy(), g["tokens"].cpu().numpy()
        t.requests += B
        for b in range(B):
            ma, mf = o["m_acc"][b], o["m_final"][b]
            t.decisions += int(np.isfinite(ma).sum()) + 1
            t.near += int((ma < BAND_ACC).sum()) + int(mf < BAND_CDF)
            if gl[b] == o["len"][b] and np.array_equal(gt[b], o["tokens"][b]):
                continue
            msg = (f"request {b} step {step}: gpu {gl[b]} {gt[b].tolist()} vs oracle {o['len'][b]} "
                   f"{o['tokens'][b].tolist()} (accept margins {ma.tolist()})")
            if gl[b] != o["len"][b]:
                i = min(int(gl[b]), int(o["len"][b]))
                assert ma[i] < BAND_ACC, msg
                t.excused += 1
                continue
            n = int(gl[b])
            wts = _final_weights(zp, zq, b, n, K, T)
            C = np.cumsum(wts) / wts.sum()
            u = oracle.uniform(seed, step, b, n, 0)
            j = int(gt[b, n])
            lo, hi = (C[j - 1] if j else 0.0), C[j]
            assert wts[j] > 0 and lo - BAND_CDF <= u < hi + BAND_CDF, msg + f"; final token {j} at [{lo}, {hi}), u {u}"
    return t


@pytest.mark.parametrize("B,K,H,V,T,seed", [
    (3, 4, 128, 3000, 1.0, 0), (5, 8, 256, 4096, 0.7, 1), (2, 1, 128, 700, 1.0, 2), (7, 3, 384, 257, 1.3, 3),
    (20, 8, 512, 32768, 1.0, 4),
    # 680 rows (the last row tile partial, down to part of a 16-row block),
    # 588 tiles: workgroups walk two or three tiles each
    (40, 8, 256, 50000, 1.0, 7)])
def test_lmhead_parity(B, K, H, V, T, seed):
    check(B, K, H, V, f32(T), seed).check()


def test_lmhead_qwen_shape():
    """Qwen3-8B head: H = 4096, V = 151,936, 64 requests of K = 8, two steps."""
    check(64, 8, 4096, 151936, 1.0, 5, steps=2).check()


def test_lmhead_rejects_bad_shapes():
    psi = _psi()
    x = torch.zeros((2, 2), dtype=torch.int32, device="cuda")
    for H in (96, 192):  # not multiples of 128
        ht, hd, w = inputs(2, 2, H, 100, 6)
        with pytest.raises(psi.PsiSpecError):
            psi.verify_lmhead(_dev(ht), _dev(hd), _dev(w), x)
