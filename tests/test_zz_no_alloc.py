"""psispec_verify_linear_noalloc (the entry point that allocates nothing and
uses the library's fixed device scratch) against psispec_verify_linear with a
caller workspace: the same kernels on the same inputs must give the same bits.
Two calls in a row, the second smaller than the first; then greedy and
filtered calls within the scratch limit; a request error; and a call past the
limit, refused before anything is enqueued."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import f32, to_dev

pytestmark = pytest.mark.gpu


def _psi():
    import lossless_speculative_verification_amd as psi
    return psi


def _same(a: dict, b: dict, keys=("tokens", "len", "probs", "resid", "draft")):
    for k in keys:
        if a.get(k) is None and b.get(k) is None:
            continue
        assert torch.equal(a[k], b[k]), k


def _pair_calls(p, q, draft, **kw):
    psi = _psi()
    pd, qd = to_dev(p), to_dev(q)
    d1 = None if draft is None else torch.from_numpy(np.ascontiguousarray(draft, dtype=np.int32)).cuda()
    d2 = None if d1 is None else d1.clone()
    ref = psi.verify_linear(pd, qd, d1, **kw)
    got = psi.verify_linear_noalloc(pd, qd, d2, **kw)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_workspace_entry_two_calls():
    """Qwen3-8B-shaped call (B=64, K=8, V=151936 bf16, T=0.7, fused drafts),
    then a smaller fp32 call (B=8, K=4, V=5000): identical outputs."""
    p, q = synth.linear_inputs("qwen", seed=3)
    ref, got = _pair_calls(p, q, None, temperature=f32(0.7), seed=11, step=2, fused=True)
    _same(ref, got)
    assert int((got["len"] < 8).sum()) > 0
    p, q = synth.pair(8, 5, 4, 5000, "f32", seed=4, sd_a=2.0, mode=0, sd_noise=0.7)
    ref, got = _pair_calls(p, q, None, temperature=1.0, seed=12, step=3, fused=True)
    _same(ref, got)


def test_noalloc_greedy_filtered_and_errors():
    psi = _psi()
    p, q = synth.pair(16, 5, 4, 3000, "bf16", seed=5, sd_a=2.0, mode=0, sd_noise=0.8)
    ref, got = _pair_calls(p, q, None, temperature=0.0, fused=True)
    _same(ref, got)
    ref, got = _pair_calls(p, q, None, temperature=1.0, top_k=40, top_p=f32(0.9), seed=3, step=1, fused=True)
    _same(ref, got)
    p2 = p.copy()
    p2[3, 2, 7] = 0x7fc0  # a NaN logit: request 3 is an error
    ref, got = _pair_calls(p2, q, None, temperature=1.0, seed=3, step=1, fused=True)
    _same(ref, got)
    assert int(got["len"][3]) == -1
    # past the scratch limit: refused synchronously, nothing enqueued
    w = synth.WORKLOADS["filtered"]
    B, K, V = w["B"], w["K"], w["V"]
    big_p = torch.empty((B, K + 1, V), dtype=torch.float32, device="cuda")
    big_q = torch.empty((B, K, V), dtype=torch.float32, device="cuda")
    with pytest.raises(psi.PsiSpecError) as e:
        psi.verify_linear_noalloc(big_p, big_q, None, temperature=1.0, top_k=50, top_p=f32(0.95), fused=True)
    assert e.value.status == psi.ESCRATCH
