"""GPU parity of multi-round generation on the toy order-2 model: the model's
logits bit for bit against the synthetic generator, and whole generation runs
(first token, drafts, verification, commit, round after round) against the
oracle's loop, request by request and round by round."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import NEAR_TIE_ACCEPT, NEAR_TIE_CDF, THREADS, f32

pytestmark = pytest.mark.gpu


def _psi():
    import lossless_speculative_verification_amd as psi
    return psi


def _model(psi):
    m = synth.TOY_MODEL
    return psi.toy_model(m["seed"], m["sd"], m["n_heavy"], m["boost"], m["rho"], m["noise"])


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


@pytest.mark.parametrize("V,kind,dtype", [(32768, 0, "bf16"), (32768, 1, "bf16"), (1001, 0, "f32"),
                                          (1001, 1, "f32"), (7, 1, "bf16")])
def test_toy_logits_bit_exact(V, kind, dtype):
    psi = _psi()
    rows = 50
    ctx = synth.randint(3, 0, 2 * rows, 1 << 20).reshape(rows, 2)
    pos = synth.randint(4, 0, rows, 64)
    g = psi.toy_logits(torch.from_numpy(ctx).cuda(), V, pos=torch.from_numpy(pos).cuda() if kind else None,
                       kind=kind, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, model=_model(psi))
    torch.cuda.synchronize()
    ref = synth.toy_logits(ctx, pos if kind else None, V=V, kind=kind, dtype=dtype)
    assert np.array_equal(_bits(g), ref)


def compare_generation(g: dict, o: dict):
    """Round by round per request: identical until the oracle's round holds a
    near tie (accept band or inverse-CDF band), after which the request is not
    compared. Returns the number of requests cut short."""
    gs, gl, grt = g["seq"].cpu().numpy(), g["len"].cpu().numpy(), g["round_tokens"].cpu().numpy()
    os_, ol, ort = o["seq"], o["len"], o["round_tokens"]
    near = (o["margin_acc"] < NEAR_TIE_ACCEPT) | (o["margin_cdf"] < NEAR_TIE_CDF)
    cut = 0
    for b in range(len(ol)):
        off = 0
        for r in range(ort.shape[1]):
            n = ort[b, r]
            same = grt[b, r] == n and np.array_equal(gs[b, off:off + n], os_[b, off:off + n])
            if not same:
                assert near[b, r], (f"request {b} round {r}: gpu {gs[b, off:off + grt[b, r]].tolist()} vs oracle "
                                    f"{os_[b, off:off + n].tolist()} (margins {o['margin_acc'][b, r]:.3g}, "
                                    f"{o['margin_cdf'][b, r]:.3g})")
                cut += 1
                break
            off += n
        else:
            assert gl[b] == ol[b] and np.array_equal(gs[b], os_[b])
    return cut


def _run(B, block, V, T, rounds, dtype="bf16", seed=1, prompt_seed=0):
    psi = _psi()
    prompt = synth.randint(prompt_seed, 0, 2 * B, V).reshape(B, 2)
    g = psi.generate_toy(torch.from_numpy(prompt).cuda(), block, V, rounds, temperature=T, seed=seed,
                         dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, model=_model(psi))
    torch.cuda.synchronize()
    model = lambda kind, ctx, pos: synth.toy_logits(ctx, pos, V=V, kind=kind, dtype=dtype)
    o = oracle.generate(model, prompt, block, V, T, seed=seed, rounds=rounds, nthreads=THREADS)
    return g, o


@pytest.mark.parametrize("B,block,V,T,rounds,dtype", [
    (16, 8, 4096, 1.0, 6, "bf16"), (12, 4, 3001, 0.7, 8, "f32"), (8, 16, 2048, 1.0, 4, "bf16"),
    (4, 2, 500, 1.3, 10, "f32"), (64, 8, 32768, 1.0, 3, "bf16")])
def test_generate_parity(B, block, V, T, rounds, dtype):
    g, o = _run(B, block, V, f32(T), rounds, dtype)
    cut = compare_generation(g, o)
    assert cut <= max(1, B // 16)
    rt = g["round_tokens"].cpu().numpy()
    assert rt.min() >= 2 and rt.max() <= block + 1


def test_generate_greedy():
    g, o = _run(16, 6, 4096, 0.0, 5, "bf16")
    assert compare_generation(g, o) == 0
