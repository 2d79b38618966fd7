"""Benchmark of lossless Psi-Spec block verification on one MI355X.

Workload (high-concurrency linear verification): B=256 requests, K=8 draft
positions, V=151936 vocabulary, bfloat16 logits, temperature 1, draft/target
correlation rho swept over {0.5, 0.8, 0.95}; one psispec_verify_linear call per
decode step, step t using pre-drawn draft set t (drawn on the GPU with
psispec_draft_sample before the timed region). Inputs are synthetic (seeded,
see synth/) and resident in HBM before timing starts.

Prints ONE JSON line: verified (request, position) rows/s over the whole sweep
(value), emitted tokens/s, the HBM roofline fraction of the verify call, and the
CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak, AMD public specification
B, K, V = 256, 8, 151936
RHOS = (0.5, 0.8, 0.95)
T = 1.0


def bytes_alg(B, K, V, esz=2):
    """Algorithmic HBM bytes of one verify call: every target and draft logit
    read once, draft ids read, output tokens/lengths written."""
    return B * (2 * K + 1) * V * esz + 4 * B * K + 4 * B * (K + 2)


def cpu_baseline(p, q, drafts, seed, budget_s=10.0, threads=16):
    """Times the CPU oracle (test infrastructure, never tuned) on whole verify
    calls of the same workload until about budget_s seconds have passed."""
    import oracle

    steps = 0
    t0 = time.perf_counter()
    while True:
        s = steps % len(drafts)
        oracle.verify_linear(p, q, drafts[s], T, seed=seed, step=s, nthreads=threads)
        steps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    wall = time.perf_counter() - t0
    return {"value": B * K * steps / wall, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": f"{steps} full verify calls (B={B}, K={K}, V={V}, bf16, rho=0.8), {threads} threads, "
                      f"{wall:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}): verification shards by request "
              "with no exchange, so the single-GPU figure is the per-GPU figure.", file=sys.stderr)
        sys.exit(2)

    import torch

    import lossless_speculative_verification_amd as psi
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    steps, warm = args.steps, args.warmup
    ws = torch.empty(psi.workspace_bytes(B, 2 * K + 1, V, psi.DTYPE_BF16), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(psi.workspace_bytes(B, K, V, psi.DTYPE_BF16), dtype=torch.uint8, device=dev)
    out_tokens = torch.empty((steps + warm, B, K + 1), dtype=torch.int32, device=dev)
    out_len = torch.empty((steps + warm, B), dtype=torch.int32, device=dev)
    out_probs = torch.empty((B, K, 2), dtype=torch.float32, device=dev)
    out_resid = torch.empty((B,), dtype=torch.float64, device=dev)
    drafts = torch.empty((steps + warm, B, K), dtype=torch.int32, device=dev)

    per_rho = []
    total_rows = 0
    total_time = 0.0
    total_emitted = 0
    kernel_ms = []
    host_inputs = None
    p_np = np.empty((B, K + 1, V), dtype=np.uint16)
    q_np = np.empty((B, K, V), dtype=np.uint16)
    for rho in RHOS:
        synth.pair(B, K + 1, K, V, "bf16", seed=args.seed, out_p=p_np, out_q=q_np,
                   **{**synth.RECIPES["highconc"], "rho": rho})
        p = torch.from_numpy(p_np.view(np.int16)).view(torch.bfloat16).to(dev)
        q = torch.from_numpy(q_np.view(np.int16)).view(torch.bfloat16).to(dev)
        # pre-drawn draft sets (untimed): set t is used at step t
        for t in range(steps + warm):
            psi.draft_sample(q, temperature=T, seed=args.seed, step=t, out=drafts[t], workspace=ws_d)
        torch.cuda.synchronize()
        if rho == 0.8 and not args.no_cpu_baseline:
            host_inputs = (p_np.copy(), q_np.copy(), drafts[:64].cpu().numpy())
        stream = torch.cuda.current_stream()

        def call(t):
            psi.verify_linear(p, q, drafts[t], temperature=T, seed=args.seed, step=t,
                              out=dict(tokens=out_tokens[t], len=out_len[t], probs=out_probs, resid=out_resid),
                              workspace=ws, stream=stream)

        for t in range(warm):
            call(t)
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(stream)
        for t in range(warm, warm + steps):
            call(t)
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ev_ms = ev0.elapsed_time(ev1)
        lens = out_len[warm:warm + steps].cpu().numpy()
        assert (lens >= 0).all()
        emitted = int((lens + 1).sum())
        per_rho.append({"rho": rho, "ms_per_step": 1e3 * wall / steps, "event_ms_per_step": ev_ms / steps,
                        "rows_per_s": B * K * steps / wall, "emitted_tok_per_s": emitted / wall,
                        "mean_accepted": float(lens.mean()), "mean_emitted": float((lens + 1).mean())})
        kernel_ms.append(ev_ms / steps)
        total_rows += B * K * steps
        total_time += wall
        total_emitted += emitted
        del p, q
        torch.cuda.empty_cache()

    call_ms = float(np.mean(kernel_ms))
    achieved = bytes_alg(B, K, V) / (call_ms * 1e-3) / 1e9
    result = {
        "metric": "verified (req·pos) rows/s + emitted tok/s; % of HBM peak, B=256 K=8 V=151936",
        "value": total_rows / total_time,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": 1e3 * total_time / (steps * len(RHOS)),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "high-concurrency linear verify B=256 K=8 V=151936 bf16 T=1, rho sweep",
                   "B": B, "K": K, "V": V, "rho": list(RHOS), "temperature": T,
                   "steps_per_rho": steps, "parallelism": "none"},
        "emitted_tok_per_s": total_emitted / total_time,
        "hbm_frac": achieved / HBM_PEAK_GBS,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "psispec_verify_linear (whole call)",
                     "bytes_per_launch": bytes_alg(B, K, V), "avg_launch_ms": call_ms},
        "per_rho": per_rho,
    }
    if host_inputs is not None:
        result["cpu_baseline"] = cpu_baseline(host_inputs[0], host_inputs[1], host_inputs[2], args.seed,
                                              budget_s=args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
