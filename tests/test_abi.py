"""The C-ABI library loads on a host without a GPU, exports every entry point
declared in include/psispec.h, and rejects bad arguments synchronously (host
validation only; no kernel is launched by these tests)."""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "psispec.h")


@pytest.fixture(scope="module")
def psi():
    import lossless_speculative_verification_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(psispec_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(psi):
    names = declared_functions()
    assert {"psispec_draft_sample", "psispec_verify_linear", "psispec_verify_tree",
            "psispec_workspace_bytes", "psispec_strerror", "psispec_version", "psispec_tree_depth"} <= set(names)
    lib = ctypes.CDLL(psi.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_params_layout_matches_header(psi):
    assert ctypes.sizeof(psi.Params) == 32
    assert psi.Params.seed.offset == 16 and psi.Params.step.offset == 24


def test_strerror_and_version(psi):
    assert psi.strerror(0) == "success"
    for code in (-1, -2, -3, -4):
        assert psi.strerror(code) and psi.strerror(code) != "unknown status"
    assert psi.version() >= 100


def test_workspace_bytes(psi):
    a = psi.workspace_bytes(256, 17, 151936, psi.DTYPE_BF16)
    assert a > 0 and a % 256 == 0
    assert psi.workspace_bytes(512, 17, 151936, psi.DTYPE_BF16) > a
    assert psi.workspace_bytes(0, 17, 151936, 1) == 0
    assert psi.workspace_bytes(1, 0, 10, 1) == 0
    assert psi.workspace_bytes(1, 3, 10, 7) == 0


def test_tree_depth(psi):
    import synth
    assert psi.tree_depth(synth.branch_chain_parent(4, 8)) == 8
    assert psi.tree_depth([-1, 0, 0, 1]) == 3
    assert psi.tree_depth([-1, 2]) == psi.EINVAL
    assert psi.tree_depth(np.arange(-1, 99)) == psi.EUNSUPPORTED  # depth 100 > 64


def _call_linear(psi, B=2, K=3, V=64, dtype=1, prm=None, ws_bytes=1 << 20, null=None, ws_addr=1 << 20):
    prm = prm if prm is not None else psi.make_params()
    fake = {k: ctypes.c_void_p(0x10000000 + 0x1000 * i) for i, k in
            enumerate(["p", "q", "d", "tok", "len", "probs", "resid"])}
    if null:
        fake[null] = None
    return psi.lib.psispec_verify_linear(fake["p"], fake["q"], dtype, B, K, V, fake["d"], ctypes.byref(prm),
                                         fake["tok"], fake["len"], fake["probs"], fake["resid"],
                                         ctypes.c_void_p(ws_addr), ws_bytes, None)


def test_linear_argument_errors(psi):
    for k in ("p", "q", "d", "tok", "len"):
        assert _call_linear(psi, null=k) == psi.EINVAL
    assert _call_linear(psi, B=0) == psi.EINVAL
    assert _call_linear(psi, K=0) == psi.EINVAL
    assert _call_linear(psi, V=0) == psi.EINVAL
    assert _call_linear(psi, K=65) == psi.EUNSUPPORTED
    assert _call_linear(psi, dtype=5) == psi.EUNSUPPORTED
    assert _call_linear(psi, prm=psi.make_params(temperature=-1.0)) == psi.EINVAL
    assert _call_linear(psi, prm=psi.make_params(temperature=float("nan"))) == psi.EINVAL
    assert _call_linear(psi, prm=psi.make_params(top_p=0.0)) == psi.EINVAL
    assert _call_linear(psi, prm=psi.make_params(top_p=1.5)) == psi.EINVAL
    assert _call_linear(psi, prm=psi.make_params(top_k=-2)) == psi.EINVAL
    assert _call_linear(psi, ws_bytes=16) == psi.EWORKSPACE
    assert _call_linear(psi, ws_addr=(1 << 20) + 8) == psi.EINVAL


def test_noalloc_argument_errors(psi):
    """The entry point without a workspace validates like psispec_verify_linear
    and refuses, before touching the GPU, a call whose scratch need exceeds
    the library's fixed array (the filtered workload at full size)."""
    f = ctypes.c_void_p(1 << 20)
    L = psi.lib

    def call(B=4, K=3, V=512, dtype=1, prm=None, null=None):
        prm = prm or psi.make_params()
        args = dict(p=f, q=f, d=f, tok=f, len=f)
        if null:
            args[null] = None
        return L.psispec_verify_linear_noalloc(args["p"], args["q"], dtype, B, K, V, args["d"], ctypes.byref(prm),
                                               args["tok"], args["len"], None, None, None)

    for k in ("p", "q", "d", "tok", "len"):
        assert call(null=k) == psi.EINVAL
    assert call(B=0) == psi.EINVAL
    assert call(K=65) == psi.EUNSUPPORTED
    assert call(dtype=5) == psi.EUNSUPPORTED
    assert call(prm=psi.make_params(top_p=0.0)) == psi.EINVAL
    big = psi.make_params(temperature=1.0, top_k=50, top_p=0.95)
    assert call(B=128, K=16, V=128256, dtype=0, prm=big) == psi.ESCRATCH
    assert psi.strerror(psi.ESCRATCH) != psi.strerror(-99)


def test_draft_argument_errors(psi):
    prm = psi.make_params()
    f = ctypes.c_void_p(0x20000000)
    ws = ctypes.c_void_p(1 << 20)
    assert psi.lib.psispec_draft_sample(None, 1, 2, 3, 64, ctypes.byref(prm), f, ws, 1 << 20, None) == psi.EINVAL
    assert psi.lib.psispec_draft_sample(f, 1, 2, 3, 64, None, f, ws, 1 << 20, None) == psi.EINVAL
    assert psi.lib.psispec_draft_sample(f, 1, 2, 3, 64, ctypes.byref(prm), f, ws, 8, None) == psi.EWORKSPACE
    assert psi.lib.psispec_draft_sample(f, 1, 2, 99, 64, ctypes.byref(prm), f, ws, 1 << 20, None) == psi.EUNSUPPORTED


def test_binding_has_no_fallback(psi):
    """The binding is marshalling only: it calls the library for every step."""
    src = open(os.path.join(ROOT, "lossless_speculative_verification_amd", "__init__.py")).read()
    assert "oracle" not in src
    assert "softmax" not in src and "torch.exp" not in src


def test_filter_limits(psi):
    # every admissible filter is accepted (the workspace check is the first to
    # fail here, before any launch): top-p without a top-k, top-k above 256,
    # top_k >= V with a top-p, and the bounded kept-set path
    for V, k, p in ((1000, 0, 0.9), (4096, 257, 1.0), (4096, 5000, 0.5), (4096, 256, 0.9), (4096, 4096, 0.3)):
        assert _call_linear(psi, V=V, prm=psi.make_params(top_k=k, top_p=p), ws_bytes=16) == psi.EWORKSPACE


def _call_cands(psi, B=2, K=15, V=1000, dtype=1, prm=None, cands=32, nodes=32, ws_bytes=1 << 30, ws_addr=1 << 20,
                null=None):
    prm = prm if prm is not None else psi.make_params()
    fake = {k: ctypes.c_void_p(0x10000000 + 0x1000 * i) for i, k in enumerate(["q", "par", "tok"])}
    if null:
        fake[null] = None
    return psi.lib.psispec_tree_candidates(fake["q"], dtype, B, K, V, ctypes.byref(prm), cands, nodes, fake["par"],
                                           fake["tok"], ctypes.c_void_p(ws_addr), ws_bytes, None)


def test_tree_candidates_argument_errors(psi):
    for k in ("q", "par", "tok"):
        assert _call_cands(psi, null=k) == psi.EINVAL
    assert _call_cands(psi, B=0) == psi.EINVAL
    assert _call_cands(psi, cands=0) == psi.EINVAL
    assert _call_cands(psi, nodes=0) == psi.EINVAL
    assert _call_cands(psi, prm=psi.make_params(temperature=0.0)) == psi.EINVAL  # no greedy candidates
    assert _call_cands(psi, prm=psi.make_params(top_k=8)) == psi.EUNSUPPORTED
    assert _call_cands(psi, prm=psi.make_params(top_p=0.5)) == psi.EUNSUPPORTED
    assert _call_cands(psi, V=20, cands=21) == psi.EUNSUPPORTED
    assert _call_cands(psi, V=4096, cands=257) == psi.EUNSUPPORTED
    assert _call_cands(psi, K=64, cands=65) == psi.EUNSUPPORTED  # K * cands > 4096
    assert _call_cands(psi, K=65, cands=8) == psi.EUNSUPPORTED
    assert _call_cands(psi, nodes=257) == psi.EUNSUPPORTED
    assert _call_cands(psi, ws_bytes=16) == psi.EWORKSPACE
    assert _call_cands(psi, ws_addr=(1 << 20) + 8) == psi.EINVAL


def _call_det(psi, B=2, N=31, V=1000, dtype=1, prm=None, ws_bytes=1 << 30, ws_addr=1 << 20, null=None):
    prm = prm if prm is not None else psi.make_params()
    fake = {k: ctypes.c_void_p(0x10000000 + 0x1000 * i) for i, k in
            enumerate(["p", "par", "ntok", "tok", "path", "len"])}
    if null:
        fake[null] = None
    return psi.lib.psispec_verify_tree_det(fake["p"], dtype, B, N, V, fake["par"], fake["ntok"], ctypes.byref(prm),
                                           fake["tok"], fake["path"], fake["len"], ctypes.c_void_p(ws_addr),
                                           ws_bytes, None)


def test_verify_tree_det_argument_errors(psi):
    for k in ("p", "par", "ntok", "tok", "path", "len"):
        assert _call_det(psi, null=k) == psi.EINVAL
    assert _call_det(psi, N=0) == psi.EINVAL
    assert _call_det(psi, V=0) == psi.EINVAL
    assert _call_det(psi, N=257) == psi.EUNSUPPORTED
    assert _call_det(psi, dtype=3) == psi.EUNSUPPORTED
    assert _call_det(psi, prm=psi.make_params(temperature=-0.5)) == psi.EINVAL
    assert _call_det(psi, prm=psi.make_params(top_k=4)) == psi.EUNSUPPORTED
    assert _call_det(psi, prm=psi.make_params(top_p=0.9)) == psi.EUNSUPPORTED
    assert _call_det(psi, ws_bytes=16) == psi.EWORKSPACE
    assert _call_det(psi, ws_addr=(1 << 20) + 4) == psi.EINVAL


def test_tv_loss_argument_errors(psi):
    f = {k: ctypes.c_void_p(0x10000000 + 0x1000 * i) for i, k in enumerate(["p", "q", "loss", "grad"])}

    def call(R=4, V=100, dtype=1, T=1.0, ws_bytes=1 << 30, ws_addr=1 << 20, null=None):
        a = dict(f)
        if null:
            a[null] = None
        return psi.lib.psispec_tv_loss(a["p"], a["q"], dtype, R, V, T, None, a["loss"], a["grad"],
                                       ctypes.c_void_p(ws_addr), ws_bytes, None)

    for k in ("p", "q", "loss"):
        assert call(null=k) == psi.EINVAL
    assert call(R=0) == psi.EINVAL
    assert call(V=0) == psi.EINVAL
    assert call(T=0.0) == psi.EINVAL
    assert call(T=float("inf")) == psi.EINVAL
    assert call(dtype=2) == psi.EUNSUPPORTED
    assert call(ws_bytes=8) == psi.EWORKSPACE
    assert call(ws_addr=(1 << 20) + 16) == psi.EINVAL
    # the generic workspace lacks the sign words of the gradient pass
    for R, V, dtype in ((4, 100, 1), (2048, 151936, 1), (3, 3001, 0)):
        need = psi.tv_workspace_bytes(R, V, dtype)
        assert need >= psi.workspace_bytes(R, 2, V, dtype) + R * -(-V // (8 if dtype == 1 else 4)) * 2
        assert call(R=R, V=V, dtype=dtype, ws_bytes=need - 1) == psi.EWORKSPACE
    assert psi.tv_workspace_bytes(0, 100, 1) == 0 and psi.tv_workspace_bytes(4, 100, 2) == 0


def test_generate_argument_errors(psi):
    m = psi.toy_model()
    prm = psi.make_params()
    f = ctypes.c_void_p(0x10000000)

    def call(B=4, block=8, V=100, dtype=1, rounds=3, prm_=prm, ws_bytes=1 << 30, ws_addr=1 << 20, model=m, prompt=f):
        return psi.lib.psispec_generate_toy(B, block, V, dtype, ctypes.byref(model) if model else None,
                                            ctypes.byref(prm_), prompt, rounds, f, f, f, ctypes.c_void_p(ws_addr),
                                            ws_bytes, None)

    assert call(model=None) == psi.EINVAL
    assert call(prompt=None) == psi.EINVAL
    assert call(B=0) == psi.EINVAL
    assert call(rounds=0) == psi.EINVAL
    assert call(block=1) == psi.EINVAL
    assert call(block=66) == psi.EUNSUPPORTED
    assert call(dtype=4) == psi.EUNSUPPORTED
    assert call(prm_=psi.make_params(top_k=5)) == psi.EUNSUPPORTED
    assert call(ws_bytes=64) == psi.EWORKSPACE
    assert call(ws_addr=(1 << 20) + 64) == psi.EINVAL
    assert psi.lib.psispec_generate_workspace_bytes(4, 1, 100, 1) == 0
    assert psi.lib.psispec_toy_logits(4, 100, None, None, 0, ctypes.byref(m), 1, f, None) == psi.EINVAL
    assert psi.lib.psispec_toy_logits(4, 100, f, None, 1, ctypes.byref(m), 1, f, None) == psi.EINVAL  # drafter needs pos


def test_lmhead_argument_errors(psi):
    prm = psi.make_params()
    f = ctypes.c_void_p(0x10000000)
    u = ctypes.c_void_p(0x10000008)  # not 16-byte aligned

    def call(B=2, K=3, H=128, V=1000, prm_=prm, ws_bytes=1 << 30, ws_addr=1 << 20, ht=f, hd=f, w=f):
        return psi.lib.psispec_verify_lmhead(ht, hd, w, B, K, H, V, f, ctypes.byref(prm_), f, f,
                                             ctypes.c_void_p(ws_addr), ws_bytes, None)

    assert call(ht=None) == psi.EINVAL
    assert call(B=0) == psi.EINVAL
    assert call(H=0) == psi.EINVAL
    assert call(H=96) == psi.EUNSUPPORTED          # not a multiple of 128
    assert call(H=192) == psi.EUNSUPPORTED
    assert call(K=65) == psi.EUNSUPPORTED
    assert call(prm_=psi.make_params(temperature=0.0)) == psi.EUNSUPPORTED
    assert call(prm_=psi.make_params(top_k=10)) == psi.EUNSUPPORTED
    assert call(w=u) == psi.EINVAL
    assert call(ws_bytes=1024) == psi.EWORKSPACE
    assert psi.lib.psispec_lmhead_workspace_bytes(2, 3, 1000) > 0
