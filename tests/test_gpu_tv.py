"""GPU parity of the total-variation distillation loss (forward and the
gradient with respect to the student logits) against the CPU oracle: small,
ragged and unaligned shapes, both dtypes, temperatures, row weights, forward
only, identical and invalid rows, and 512 full-vocabulary rows."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import THREADS, f32, to_dev

pytestmark = pytest.mark.gpu

# p and q are evaluated in binary32 from binary32-grade normalisers: each is
# good to ~1e-6 relative (exponent rounding on the tails included), so the
# loss to LOSS_ATOL and each gradient element to GRAD_RTOL; an element whose
# p and q agree within TIE_RTOL may take the other sign (and moves its row's
# mean term by its own q), so such rows compare at TIE_GRAD_RTOL.
LOSS_ATOL = 5e-6
GRAD_RTOL = 2e-5
TIE_RTOL = 1e-5
TIE_GRAD_RTOL = 1e-3
BF16_ULP = 2.0 ** -8


def _psi():
    import lossless_speculative_verification_amd as psi
    return psi


def _f64(x):
    return (synth.bf16_to_f32(x) if x.dtype == np.uint16 else x).astype(np.float64)


def _probs(x, T):
    with np.errstate(invalid="ignore"):  # rows of NaN or +inf are never compared
        z = _f64(x) / T
        m = np.max(z, axis=-1, keepdims=True)
        e = np.exp(z - m)
        return e / e.sum(axis=-1, keepdims=True)


def check(p, q, T=1.0, w=None, grad=True, rows=None):
    """GPU loss and gradient against the oracle on rows `rows` (all by default)."""
    psi = _psi()
    R, V = p.shape[0] * (p.shape[1] if p.ndim == 3 else 1), p.shape[-1]
    p2, q2 = p.reshape(R, V), q.reshape(R, V)
    wd = None if w is None else torch.from_numpy(np.asarray(w, dtype=np.float32)).cuda()
    g = psi.tv_loss(to_dev(p2), to_dev(q2), temperature=T, row_weights=wd, grad=grad)
    torch.cuda.synchronize()
    rows = np.arange(R) if rows is None else np.asarray(rows)
    ol, og = oracle.tv_loss(p2[rows], q2[rows], T, row_weights=None if w is None else np.asarray(w, np.float32)[rows],
                            grad=grad, nthreads=THREADS)
    gl = g["loss"].cpu().numpy()[rows]
    nan = np.isnan(ol)
    assert np.array_equal(np.isnan(gl), nan)
    assert np.all(np.abs(gl[~nan] - ol[~nan]) <= LOSS_ATOL), np.max(np.abs(gl[~nan] - ol[~nan]))
    if not grad:
        assert g["grad"] is None
        return gl, ol
    gg = g["grad"].cpu()
    gg = (gg.view(torch.int16).numpy().view(np.uint16) if gg.dtype == torch.bfloat16 else gg.numpy())
    gg = _f64(gg)[rows]
    bf16 = p.dtype == np.uint16
    P, Q = _probs(p2[rows], T), _probs(q2[rows], T)
    for k in range(len(rows)):
        if nan[k]:
            assert np.all(np.isnan(gg[k]))
            continue
        tie = np.abs(P[k] - Q[k]) <= TIE_RTOL * np.maximum(P[k], Q[k])
        rtol = TIE_GRAD_RTOL if tie.any() else GRAD_RTOL
        if bf16:
            rtol += BF16_ULP
        err = np.abs(gg[k] - og[k])
        tol = rtol * np.abs(og[k]) + 1e-12 * np.max(np.abs(og[k])) + 1e-37
        bad = (err > tol) & ~tie
        assert not bad.any(), (k, np.nonzero(bad)[0][:8], gg[k][bad][:4], og[k][bad][:4])
    return gl, ol


@pytest.mark.parametrize("R,V,dtype,T,seed", [
    (6, 5000, "bf16", 1.0, 0), (4, 3001, "f32", 0.7, 1), (5, 777, "bf16", 1.3, 2), (3, 151936, "bf16", 1.0, 3),
    (8, 1, "f32", 1.0, 4), (2, 16, "bf16", 0.5, 5), (7, 20000, "f32", 1.0, 6)])
def test_tv_parity(R, V, dtype, T, seed):
    p, q = synth.pair(R, 1, 1, V, dtype, seed=seed, sd_a=2.0, mode=1, rho=0.8, sd_noise=2.0)
    check(p, q, f32(T))


def test_tv_weights_and_forward_only():
    p, q = synth.pair(6, 1, 1, 4096, "bf16", seed=11, sd_a=3.0, n_heavy=20, boost=8.0, mode=1, rho=0.9,
                      sd_noise=3.0)
    w = np.linspace(0.1, 2.0, 6).astype(np.float32)
    check(p, q, 1.0, w=w)
    check(p, q, 1.0, grad=False)


def test_tv_identical_and_invalid_rows():
    p, q = synth.pair(6, 1, 1, 3000, "f32", seed=12, sd_a=2.0, mode=0, sd_noise=1.0)
    q[0] = p[0]                  # identical rows: loss 0, gradient 0
    q[1, 0, 5] = np.nan
    p[2, 0, :] = -np.inf
    p[3, 0, 9] = np.inf
    gl, ol = check(p, q, 1.0)
    assert gl[0] == 0.0 and np.all(np.isnan(gl[1:4])) and np.all(np.isfinite(gl[4:]))
    psi = _psi()
    g = psi.tv_loss(to_dev(p.reshape(6, -1)), to_dev(q.reshape(6, -1)), temperature=1.0)
    assert torch.all(g["grad"][0] == 0)


def test_tv_many_rows():
    """512 rows of 151936 bf16 logits: the first and last rows and a sample of
    the rest against the oracle."""
    R, V = 512, 151936
    p, q = synth.pair(R, 1, 1, V, "bf16", seed=13, sd_a=3.0, n_heavy=20, boost=8.0, mode=1, rho=0.85, sd_noise=3.0)
    rows = [0, 1, 219, 220, 221, 439, 440, 441, 511] + list(range(37, R, 97))
    check(p, q, 1.0, w=np.full(R, 1.0 / R, dtype=np.float32), rows=sorted(set(rows)))
