"""GPU parity of tree verification (and its node drafts) against the CPU oracle:
the branch-and-chain tree workload at full size, wide, deep and random
topologies, greedy and filtered modes, request errors, a chain tree against the
linear verifier, and the first emitted token's law over many replicas."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import THREADS, Tally, compare_drafts, compare_tree, f32, to_dev
from oracle_helpers import chi2_pvalue

pytestmark = pytest.mark.gpu


def _psi():
    import lossless_speculative_verification_amd as psi
    return psi


def _case(p, q, parent, T=1.0, top_k=0, top_p=1.0, seed=0, step=0, nodes=None, tally=None):
    """Runs GPU and oracle; node drafts fused on the GPU (and drawn by the
    oracle, compared draw by draw) when nodes is None, the oracle then
    verifying the GPU's drafts. Returns (gpu dict, oracle dict); the draft
    comparison is added to `tally` when one is given."""
    psi = _psi()
    T, top_p = f32(T), f32(top_p)
    pd, qd = to_dev(p), to_dev(q)
    if nodes is None:
        g = psi.verify_tree(pd, qd, parent, None, temperature=T, top_k=top_k, top_p=top_p, seed=seed, step=step,
                            fused=True)
        torch.cuda.synchronize()
        on, om = oracle.tree_draft(q, parent, T, top_k=top_k, top_p=top_p, seed=seed, step=step, nthreads=THREADS,
                                   margins=True)
        gn = g["nodes"].cpu().numpy()
        td = compare_drafts(gn, on, om, name="tree drafts")
        if tally is not None:
            tally += td
        else:
            td.check()
        # the oracle verifies the GPU's drafts (equal to its own except excused draws)
        on = gn
    else:
        on = np.ascontiguousarray(nodes, dtype=np.int32)
        g = psi.verify_tree(pd, qd, parent, torch.from_numpy(on).cuda(), temperature=T, top_k=top_k, top_p=top_p,
                            seed=seed, step=step)
        torch.cuda.synchronize()
    o = oracle.verify_tree(p, q, parent, on, T, top_k=top_k, top_p=top_p, seed=seed, step=step, nthreads=THREADS)
    return g, o


def wide_parent(root_children=12, grand=2):
    par = [-1] * root_children
    for i in range(root_children):
        par += [i] * grand
    return np.array(par, dtype=np.int32)


def random_parent(N, seed):
    rng = np.random.default_rng(seed)
    return np.array([rng.integers(-1, n) if n else -1 for n in range(N)], dtype=np.int32)


def test_tree_workload_full_size():
    """Four branches of eight-node chains, p and q [4, 33, 151936] bf16, T=1,
    node drafts fused; 256 random-number seeds over four input sets."""
    parent = synth.branch_chain_parent(4, 8)
    inputs = [synth.tree_inputs("tree", seed=s) for s in range(4)]
    tally = Tally("tree workload x256 seeds")
    lens = []
    for seed in range(256):
        p, q = inputs[seed % 4]
        g, o = _case(p, q, parent, seed=seed, step=seed // 4, tally=tally)
        tally += compare_tree(g, o)
        lens += list(o["len"])
    tally.check()
    assert max(lens) >= 2


@pytest.mark.parametrize("topo,dtype,V,T,noise", [
    ("branch", "bf16", 5000, 1.0, 1.5), ("wide", "f32", 3000, 0.8, 2.0), ("wide", "bf16", 1001, 1.0, 2.5),
    ("random", "f32", 2048, 1.0, 1.0), ("random", "bf16", 777, 1.3, 2.0), ("chain64", "f32", 1500, 1.0, 0.7),
    ("single", "bf16", 4096, 1.0, 1.0)])
def test_tree_topologies(topo, dtype, V, T, noise):
    parent = {"branch": synth.branch_chain_parent(4, 8), "wide": wide_parent(), "random": random_parent(40, V),
              "chain64": np.arange(-1, 63, dtype=np.int32), "single": np.array([-1], dtype=np.int32)}[topo]
    N = len(parent)
    B = 6
    p, q = synth.pair(B, N + 1, N + 1, V, dtype, seed=V + N, sd_a=2.0, mode=0, sd_noise=noise)
    rejected = 0
    for step in range(4):
        g, o = _case(p, q, parent, T=T, seed=3, step=step)
        compare_tree(g, o, name="tree").check()
        rejected += int(np.sum(o["len"] < oracle.tree_depth(parent)))
    assert rejected > 0


def test_tree_given_nodes():
    """Node tokens supplied by the caller (not fused), including tokens the draft
    rows make unlikely."""
    parent = wide_parent(5, 3)
    N, V, B = len(parent), 2000, 8
    p, q = synth.pair(B, N + 1, N + 1, V, "f32", seed=17, sd_a=2.0, mode=0, sd_noise=1.0)
    for step in range(3):
        nodes = synth.randint(40 + step, 0, B * N, V).reshape(B, N)
        g, o = _case(p, q, parent, seed=8, step=step, nodes=nodes)
        compare_tree(g, o, name="tree").check()


def test_chain_tree_matches_linear_gpu():
    """A chain tree reproduces the GPU linear verifier bit for bit."""
    psi = _psi()
    p, ql = synth.linear_inputs("qwen", seed=2, B=16, K=6)
    K = ql.shape[1]
    qt = np.concatenate([ql, ql[:, -1:]], axis=1)
    parent = np.arange(-1, K - 1, dtype=np.int32)
    pd, qld, qtd = to_dev(p), to_dev(ql), to_dev(qt)
    T = f32(0.7)
    for step in range(4):
        lin = psi.verify_linear(pd, qld, None, temperature=T, seed=1, step=step, fused=True)
        tr = psi.verify_tree(pd, qtd, parent, None, temperature=T, seed=1, step=step, fused=True)
        torch.cuda.synchronize()
        assert torch.equal(tr["nodes"], lin["draft"])
        assert torch.equal(tr["len"], lin["len"])
        assert torch.equal(tr["tokens"], lin["tokens"])


@pytest.mark.parametrize("fused", [True, False])
def test_tree_greedy(fused):
    parent = random_parent(30, 1)
    N, V, B = len(parent), 3000, 8
    p, q = synth.pair(B, N + 1, N + 1, V, "bf16", seed=4, sd_a=2.0, mode=0, sd_noise=0.3)
    nodes = None if fused else oracle.tree_draft(q, parent, 0.0)
    if not fused:
        nodes[::3, 1] = (nodes[::3, 1] + 1) % V
    g, o = _case(p, q, parent, T=0.0, nodes=nodes)
    t = compare_tree(g, o)
    assert t.excused == 0


@pytest.mark.parametrize("top_k,top_p", [(20, 0.9), (256, 1.0), (5, 0.5)])
def test_tree_filtered(top_k, top_p):
    parent = wide_parent(6, 2)
    N, V, B = len(parent), 4000, 8
    p, q = synth.pair(B, N + 1, N + 1, V, "f32", seed=top_k, sd_a=2.0, mode=0, sd_noise=0.8)
    for step in range(3):
        g, o = _case(p, q, parent, T=1.0, top_k=top_k, top_p=top_p, seed=2, step=step)
        compare_tree(g, o, name="tree").check()


@pytest.mark.parametrize("topo,dtype,V,top_k,top_p,noise", [
    ("wide", "f32", 4000, 0, 0.9, 0.8), ("wide", "bf16", 3001, 300, 1.0, 2.0), ("wide", "f32", 5000, 500, 0.7, 2.5),
    ("branch", "bf16", 6000, 0, 0.5, 1.5), ("random", "f32", 2048, 2048, 0.95, 1.0)])
def test_tree_filtered_wide(topo, dtype, V, top_k, top_p, noise):
    """Filters without a small bound on the kept set (top-p alone, top_k above
    256, top_k >= V with a top-p); high draft noise makes several rejections
    at a node, each a residual pass over the filtered row pair."""
    parent = {"wide": wide_parent(12, 2), "branch": synth.branch_chain_parent(4, 8),
              "random": random_parent(40, 7)}[topo]
    N, B = len(parent), 6
    p, q = synth.pair(B, N + 1, N + 1, V, dtype, seed=V + top_k, sd_a=2.0, mode=0, sd_noise=noise)
    tally = Tally(f"tree wide {topo} k={top_k} p={top_p}")
    for step in range(3):
        print(f"[tree wide] {topo} {dtype} V={V} k={top_k} p={top_p} step {step}", flush=True)
        g, o = _case(p, q, parent, T=1.0, top_k=top_k, top_p=top_p, seed=4, step=step, tally=tally)
        tally += compare_tree(g, o)
    tally.check()


def test_tree_workload_top_p_alone():
    """The tree workload at full size ([4, 33, 151936] bf16) with top_k = 0 and
    top_p = 0.95, node drafts fused, 16 random-number seeds."""
    parent = synth.branch_chain_parent(4, 8)
    p, q = synth.tree_inputs("tree", seed=0)
    tally = Tally("tree workload top-p alone x16")
    for seed in range(16):
        print(f"[tree wide] full size seed {seed}", flush=True)
        g, o = _case(p, q, parent, top_k=0, top_p=0.95, seed=seed, step=seed, tally=tally)
        tally += compare_tree(g, o)
    tally.check()


def test_tree_errors():
    parent = synth.branch_chain_parent(2, 3)
    N, V, B = len(parent), 1000, 6
    p, q = synth.pair(B, N + 1, N + 1, V, "f32", seed=6, sd_a=2.0, mode=0, sd_noise=0.5)
    p[1, 6, 3] = np.nan        # a leaf row
    q[2, 2, :] = -np.inf       # an inner draft row
    p[3, 0, 9] = np.inf
    nodes = oracle.tree_draft(q, parent, 1.0)
    nodes[4, 2] = V            # token out of range
    g, o = _case(p, q, parent, nodes=nodes)
    gl = g["len"].cpu().numpy()
    assert list(gl[[1, 2, 3, 4]]) == [-1] * 4 and gl[0] >= 0 and gl[5] >= 0
    compare_tree(g, o, name="tree").check()
    g, o = _case(p, q, parent)  # fused: request 2 has no valid drafts
    assert np.all(g["nodes"].cpu().numpy()[2] == -1)
    compare_tree(g, o, name="tree").check()
    for top_k, top_p in ((0, 0.9), (400, 1.0)):  # the same through the cut search
        g, o = _case(p, q, parent, nodes=nodes, top_k=top_k, top_p=top_p)
        assert list(g["len"].cpu().numpy()[[1, 2, 3, 4]]) == [-1] * 4
        compare_tree(g, o, name="tree wide errors").check()


def test_tree_first_token_law():
    """Over 40000 replicas of one small request (root with 3 i.i.d. children,
    each heading a 2-chain), the first emitted token follows P_root."""
    psi = _psi()
    V, reps = 12, 40000
    parent = np.array([-1, -1, -1, 0, 1, 2, 3, 4, 5], dtype=np.int32)
    N = len(parent)
    rng = np.random.default_rng(5)
    a = rng.normal(0, 1.5, (1, N + 1, V)).astype(np.float32)
    d = (a + rng.normal(0, 1.2, (1, N + 1, V))).astype(np.float32)
    p = np.ascontiguousarray(np.broadcast_to(a, (reps, N + 1, V)))
    q = np.ascontiguousarray(np.broadcast_to(d, (reps, N + 1, V)))
    g = psi.verify_tree(to_dev(p), to_dev(q), parent, None, temperature=1.0, seed=77, step=0, fused=True)
    torch.cuda.synchronize()
    first = g["tokens"].cpu().numpy()[:, 0]
    P = np.exp(a[0, 0].astype(np.float64) - np.logaddexp.reduce(a[0, 0].astype(np.float64)))
    counts = np.bincount(first, minlength=V)
    assert chi2_pvalue(counts, P * reps) > 1e-4
