"""Seeded synthetic logit generators for the verification workloads.

Holds no verification arithmetic: it only fills target logits p and draft
logits q with seeded normals (synth.c), heavy-token boosts and a draft/target
correlation, as described per workload below. The GPU tests, the benchmark and
the oracle all read the same arrays.

Workloads (shapes follow the pages' Qwen3-8B / Llama-3-vocabulary setting,
see the Uno explainer §5.1 for the throughput protocol and §6.3 for the
accept-length range the correlation knob is meant to cover):
  tiny       B=1,   K=4,  V=1024,   fp32, a ~ N(0, 2^2),                     d = a + N(0, 0.5^2)
  qwen       B=64,  K=8,  V=151936, bf16, a ~ N(0, 3^2) + 8 on 20 ids/row,   d = rho*a + sqrt(1-rho^2)*3*eps, rho=0.9
  highconc   B=256, K=8,  V=151936, bf16, same as qwen,                       rho in {0.5, 0.8, 0.95}
  filtered   B=128, K=16, V=128256, fp32, a ~ N(0, 2^2),                     d = a + N(0, 0.5^2)
  tree       B=4,   N=32, V=151936, bf16, same as qwen,                       rho = 0.85
  toy model  an order-2 synthetic language model (target and drafter logits from
             the last two tokens) for multi-round generation; see syn_toy_logits
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")


def build() -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-ffp-contract=off", "-fPIC", "-shared", "-o", _LIB, _SRC, "-lm",
           "-lpthread"]
    subprocess.run(cmd, check=True)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        L.syn_pair.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                               ctypes.c_float, ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_float,
                               ctypes.c_float, ctypes.c_int, P, P, ctypes.c_int]
        L.syn_pair.restype = ctypes.c_int
        L.syn_randint.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64, P]
        L.syn_randint.restype = ctypes.c_int
        L.syn_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, P]
        L.syn_normal.restype = ctypes.c_int
        L.syn_toy_logits.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, P, P, ctypes.c_int,
                                     ctypes.c_float, ctypes.c_int, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                     ctypes.c_int, P]
        L.syn_toy_logits.restype = ctypes.c_int
        _lib = L
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# Recipe per workload: value distribution of a (target) and d (draft).
RECIPES = {
    "tiny": dict(sd_a=2.0, n_heavy=0, boost=0.0, mode=0, rho=0.0, sd_noise=0.5),
    "qwen": dict(sd_a=3.0, n_heavy=20, boost=8.0, mode=1, rho=0.9, sd_noise=3.0),
    "highconc": dict(sd_a=3.0, n_heavy=20, boost=8.0, mode=1, rho=0.8, sd_noise=3.0),
    "filtered": dict(sd_a=2.0, n_heavy=0, boost=0.0, mode=0, rho=0.0, sd_noise=0.5),
    "tree": dict(sd_a=3.0, n_heavy=20, boost=8.0, mode=1, rho=0.85, sd_noise=3.0),
    "treesampler": dict(sd_a=3.0, n_heavy=20, boost=8.0, mode=1, rho=0.85, sd_noise=3.0),
    "tvloss": dict(sd_a=3.0, n_heavy=20, boost=8.0, mode=1, rho=0.85, sd_noise=3.0),
}

# Shapes and sampling parameters per workload.
WORKLOADS = {
    "tiny": dict(B=1, K=4, V=1024, dtype="f32", temperature=1.0, top_k=0, top_p=1.0, fused=True),
    "qwen": dict(B=64, K=8, V=151936, dtype="bf16", temperature=0.7, top_k=0, top_p=1.0, fused=True),
    "highconc": dict(B=256, K=8, V=151936, dtype="bf16", temperature=1.0, top_k=0, top_p=1.0, fused=False),
    "filtered": dict(B=128, K=16, V=128256, dtype="f32", temperature=1.0, top_k=50, top_p=0.95, fused=True),
    "greedy": dict(B=128, K=16, V=128256, dtype="f32", temperature=0.0, top_k=0, top_p=1.0, fused=True),
    "tree": dict(B=4, N=32, V=151936, dtype="bf16", temperature=1.0, top_k=0, top_p=1.0),
    # Tree Sampler: a block of 16 draft positions, 32 candidates per position,
    # 32 kept prefixes, verified against one target row per prefix plus the root
    "treesampler": dict(B=4, K=16, cands=32, nodes=32, V=151936, dtype="bf16", temperature=1.0),
    # TV distillation loss: 8 sequences x 256 noisy positions, teacher and
    # student logits per position, forward and backward
    "tvloss": dict(R=2048, V=151936, dtype="bf16", temperature=1.0),
}
WORKLOADS_RECIPE = {"greedy": "filtered"}


def pair(B, Rp, Rq, V, dtype, seed=0, sd_a=2.0, n_heavy=0, boost=0.0, mode=0, rho=0.0, sd_noise=0.5,
         nthreads=None, out_p=None, out_q=None):
    """Target logits [B, Rp, V] and draft logits [B, Rq, V].

    dtype "f32" gives float32 arrays; "bf16" gives uint16 arrays holding
    bfloat16 bits. out_p / out_q may be preallocated arrays to fill.
    """
    bf16 = dtype == "bf16"
    npdt = np.uint16 if bf16 else np.float32
    p = out_p if out_p is not None else np.empty((B, Rp, V), dtype=npdt)
    q = out_q if out_q is not None else np.empty((B, Rq, V), dtype=npdt)
    assert p.dtype == npdt and q.dtype == npdt and p.flags.c_contiguous and q.flags.c_contiguous
    assert p.shape == (B, Rp, V) and q.shape == (B, Rq, V)
    rc = lib().syn_pair(int(seed), B, Rp, Rq, V, float(sd_a), int(n_heavy), float(boost), int(mode), float(rho),
                        float(sd_noise), int(bf16), p.ctypes.data_as(ctypes.c_void_p),
                        q.ctypes.data_as(ctypes.c_void_p), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("syn_pair rejected its arguments")
    return p, q


def linear_inputs(workload, seed=0, B=None, K=None, V=None, rho=None, nthreads=None, **over):
    """(p [B, K+1, V], q [B, K, V]) for a named workload; shape/rho overrides allowed."""
    w = dict(WORKLOADS[workload])
    r = dict(RECIPES[WORKLOADS_RECIPE.get(workload, workload)])
    if rho is not None:
        r["rho"] = rho
    r.update(over)
    B = B or w["B"]
    K = K or w["K"]
    V = V or w["V"]
    return pair(B, K + 1, K, V, w["dtype"], seed=seed, nthreads=nthreads, **r)


def tree_inputs(workload="tree", seed=0, B=None, N=None, V=None, rho=None, nthreads=None, **over):
    """(p [B, N+1, V], q [B, N+1, V]) for the tree workload."""
    w = dict(WORKLOADS[workload])
    r = dict(RECIPES[workload])
    if rho is not None:
        r["rho"] = rho
    r.update(over)
    B = B or w["B"]
    N = N or w["N"]
    V = V or w["V"]
    return pair(B, N + 1, N + 1, V, w["dtype"], seed=seed, nthreads=nthreads, **r)


def treesampler_inputs(seed=0, B=None, K=None, nodes=None, V=None, nthreads=None):
    """(p [B, nodes+1, V], q [B, K, V]) for the Tree Sampler workload: draft
    rows per block position and target rows per kept prefix (plus the root),
    row i of p correlated with row i of q for i < K."""
    w = WORKLOADS["treesampler"]
    B = B or w["B"]
    K = K or w["K"]
    nodes = nodes or w["nodes"]
    V = V or w["V"]
    return pair(B, nodes + 1, K, V, w["dtype"], seed=seed, nthreads=nthreads, **RECIPES["treesampler"])


def tv_inputs(seed=0, R=None, V=None, nthreads=None):
    """(teacher p [R, V], student q [R, V]) for the TV-loss workload; row r of
    q is correlated with row r of p."""
    w = WORKLOADS["tvloss"]
    R = R or w["R"]
    V = V or w["V"]
    p, q = pair(R, 1, 1, V, w["dtype"], seed=seed, nthreads=nthreads, **RECIPES["tvloss"])
    return p.reshape(R, V), q.reshape(R, V)


def branch_chain_parent(branches=4, depth=8):
    """Topology of the tree workload: `branches` children of the root, each the
    head of a chain of `depth` nodes; node branches_k*depth + j has parent
    k*depth + j - 1 (j > 0) or -1 (j == 0)."""
    par = []
    for k in range(branches):
        for j in range(depth):
            par.append(-1 if j == 0 else k * depth + j - 1)
    return np.array(par, dtype=np.int32)


def randint(seed, stream, count, n):
    out = np.empty(count, dtype=np.int32)
    lib().syn_randint(int(seed), int(stream), int(count), int(n), out.ctypes.data_as(ctypes.c_void_p))
    return out


def normal(seed, stream, count):
    out = np.empty(count, dtype=np.float64)
    lib().syn_normal(int(seed), int(stream), int(count), out.ctypes.data_as(ctypes.c_void_p))
    return out


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    return (h.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even narrowing of float32 to bfloat16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


# Toy order-2 model of the multi-round generation workload: target logits
# sd * z + boost on about n_heavy / 1024 of the tokens per context; the drafter
# rho * a + noise * z' per block position.
TOY_MODEL = dict(seed=1234, sd=2.0, n_heavy=1, boost=6.0, rho=0.8, noise=1.5)


def toy_logits(ctx, pos=None, V=32768, kind=0, dtype="bf16", model=None):
    """Toy-model logits [rows, V]: ctx [rows, 2] int32 (last two tokens), pos
    [rows] int32 block positions (draft kind only). kind 0 = target, 1 = draft.
    float32, or uint16 bfloat16 bits."""
    m = dict(TOY_MODEL)
    m.update(model or {})
    ctx = np.ascontiguousarray(ctx, dtype=np.int32).reshape(-1, 2)
    rows = ctx.shape[0]
    pp = None if pos is None else np.ascontiguousarray(pos, dtype=np.int32).reshape(rows)
    bf16 = dtype == "bf16"
    out = np.empty((rows, V), dtype=np.uint16 if bf16 else np.float32)
    rc = lib().syn_toy_logits(int(m["seed"]), rows, int(V), ctx.ctypes.data_as(ctypes.c_void_p),
                              None if pp is None else pp.ctypes.data_as(ctypes.c_void_p), int(kind), float(m["sd"]),
                              int(m["n_heavy"]), float(m["boost"]), float(m["rho"]), float(m["noise"]), int(bf16),
                              out.ctypes.data_as(ctypes.c_void_p))
    if rc != 0:
        raise ValueError("syn_toy_logits rejected its arguments")
    return out
