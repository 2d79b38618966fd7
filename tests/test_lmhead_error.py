"""The error bound behind the LM-head parity bands, checked on the CPU.

The fused LM-head verifier forms each logit as an H-term dot product of
bfloat16 values on matrix cores. Each product is exact in fp32, but the sum
accumulates in fp32. The oracle sums the exact products in fp64. Its logits
differ from the GPU's by the fp32 accumulation error delta. Through the
log-normaliser a probability then moves by at most 2 delta, relative. A ratio
P/Q moves by at most 4 delta, and so does an interval edge of a final draw's
CDF, as a fraction of the mass. The parity test's bands BAND_ACC and BAND_CDF
must therefore exceed 4 delta.

This test measures delta on the parity test's own input distribution, at the
Qwen3-8B hidden size H = 4096. The accumulation is emulated plainly in numpy
float32, one product at a time in index order. That is the slowest-converging
order: the matrix cores add 16 products per step, which halves the error (see
the second model below).
"""
from __future__ import annotations

import numpy as np

from test_gpu_lmhead import BAND_ACC, BAND_CDF, inputs

import synth


def _dots(ht, w, chunk):
    """fp32 accumulation of the exact products (in steps of `chunk` products
    summed first in fp32), and the fp64 sum, for every pair of rows."""
    h = synth.bf16_to_f32(ht).reshape(-1, ht.shape[-1])
    v = synth.bf16_to_f32(w)
    H = h.shape[1]
    exact = h.astype(np.float64) @ v.astype(np.float64).T
    acc = np.zeros(exact.shape, dtype=np.float32)
    for c in range(0, H, chunk):
        s = np.zeros(exact.shape, dtype=np.float32)
        for k in range(c, c + chunk):
            s += np.outer(h[:, k], v[:, k]).astype(np.float32)  # products of bf16 values are exact in fp32
        acc += s
    return acc.astype(np.float64), exact


def test_lmhead_logit_error_within_bands():
    ht, _, w = inputs(4, 8, 4096, 512, seed=5)  # 36 hidden rows x 512 vocabulary rows
    for chunk in (1, 16):
        acc, exact = _dots(ht, w, chunk)
        delta = float(np.max(np.abs(acc - exact)))
        print(f"fp32 accumulation in steps of {chunk}: max logit error {delta:.3g} "
              f"(logit sd {exact.std():.3g})", flush=True)
        assert 4 * delta < BAND_ACC and 4 * delta < BAND_CDF
