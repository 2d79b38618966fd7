"""GPU parity of linear verification fused with the LM head: hidden states and
a vocabulary matrix in, the verification's tokens and lengths out, against the
oracle's logits (exact products summed in fp64) fed to the oracle's linear
verification. Ragged vocabularies and row counts, several temperatures, and
the Qwen3-8B head shape (H = 4096, V = 151,936)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import THREADS, f32

pytestmark = pytest.mark.gpu

# The GPU's logits carry the fp32 accumulation error of an H-term dot product
# of bf16 values (~sqrt(H) 2^-24 times the partial sums, about 1e-5 absolute
# at H = 4096 for these inputs), so a ratio P/Q moves by about 2e-5 relative
# and a cumulative position by about 1e-5 of the mass: decisions whose oracle
# margin is inside these bands may differ.
BAND_ACC = 1e-4
BAND_CDF = 1e-4


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


def check(B, K, H, V, T, seed, steps=3):
    psi = _psi()
    ht, hd, w = inputs(B, K, H, V, seed)
    zp = oracle.lmhead_logits(ht, w)
    zq = oracle.lmhead_logits(hd, w)
    dt, dd, dw = _dev(ht), _dev(hd), _dev(w)
    excused = decisions = 0
    for step in range(steps):
        x, _ = oracle.draft_sample(zq, T, seed=seed, step=step, nthreads=THREADS)
        g = psi.verify_lmhead(dt, dd, dw, torch.from_numpy(x).cuda(), temperature=T, seed=seed, step=step)
        torch.cuda.synchronize()
        o = oracle.verify_linear(zp, zq, x, T, seed=seed, step=step, nthreads=THREADS)
        gl, gt = g["len"].cpu().numpy(), g["tokens"].cpu().numpy()
        for b in range(B):
            decisions += 1
            if gl[b] == o["len"][b] and np.array_equal(gt[b], o["tokens"][b]):
                continue
            assert o["margin_acc"][b] < BAND_ACC or o["margin_cdf"][b] < BAND_CDF, (
                f"request {b} step {step}: gpu {gl[b]} {gt[b].tolist()} vs oracle {o['len'][b]} "
                f"{o['tokens'][b].tolist()} (margins {o['margin_acc'][b]:.3g} {o['margin_cdf'][b]:.3g})")
            excused += 1
    return excused, decisions


@pytest.mark.parametrize("B,K,H,V,T,seed", [
    (3, 4, 128, 3000, 1.0, 0), (5, 8, 256, 4096, 0.7, 1), (2, 1, 64, 700, 1.0, 2), (7, 3, 192, 257, 1.3, 3),
    (20, 8, 512, 32768, 1.0, 4)])
def test_lmhead_parity(B, K, H, V, T, seed):
    excused, decisions = check(B, K, H, V, f32(T), seed)
    assert excused <= max(1, decisions // 50)


def test_lmhead_qwen_shape():
    """Qwen3-8B head: H = 4096, V = 151,936, four requests of K = 8."""
    excused, decisions = check(4, 8, 4096, 151936, 1.0, 5, steps=2)
    assert excused <= 1


def test_lmhead_rejects_bad_shapes():
    psi = _psi()
    ht, hd, w = inputs(2, 2, 96, 100, 6)  # H not a multiple of 64
    x = torch.zeros((2, 2), dtype=torch.int32, device="cuda")
    with pytest.raises(psi.PsiSpecError):
        psi.verify_lmhead(_dev(ht), _dev(hd), _dev(w), x)
