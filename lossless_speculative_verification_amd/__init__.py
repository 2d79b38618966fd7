"""Python binding of libpsispec (lossless Psi-Spec block verification on MI355X).

Argument marshalling only: every step of the method runs in the HIP kernels of
libpsispec.so (built in-tree by build.py). torch provides device memory and the
current stream; there is no CPU or torch fallback — if the library is missing
the import fails.

Function names mirror the C ABI in include/psispec.h:
  draft_sample   psispec_draft_sample
  verify_linear  psispec_verify_linear
  verify_tree    psispec_verify_tree
  tree_candidates  psispec_tree_candidates
  verify_tree_det  psispec_verify_tree_det
  tv_loss          psispec_tv_loss
  verify_lmhead    psispec_verify_lmhead
  toy_logits       psispec_toy_logits (synthetic stand-in model)
  generate_toy     psispec_generate_toy
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpsispec.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP, ESCRATCH = 0, -1, -2, -3, -4, -5
DTYPE_F32, DTYPE_BF16 = 0, 1
FUSED_DRAFT = 1
MAX_K = 64


class PsiSpecError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {strerror(status)} ({status})")
        self.status = status


class Params(ctypes.Structure):
    """psispec_params (include/psispec.h)."""

    _fields_ = [("temperature", ctypes.c_float), ("top_k", ctypes.c_int32), ("top_p", ctypes.c_float),
                ("flags", ctypes.c_uint32), ("seed", ctypes.c_uint64), ("step", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32)]


class ToyModel(ctypes.Structure):
    """psispec_toy_model (include/psispec.h)."""

    _fields_ = [("seed", ctypes.c_uint64), ("sd", ctypes.c_float), ("n_heavy", ctypes.c_int32),
                ("boost", ctypes.c_float), ("rho", ctypes.c_float), ("noise", ctypes.c_float),
                ("reserved", ctypes.c_uint32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libpsispec.so is not built ({LIB_PATH}); run "
                          "`python lossless_speculative_verification_amd/build.py`")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.psispec_workspace_bytes.argtypes = [i64, i32, i32, ctypes.c_int]
    L.psispec_workspace_bytes.restype = sz
    L.psispec_tv_workspace_bytes.argtypes = [i64, i32, ctypes.c_int]
    L.psispec_tv_workspace_bytes.restype = sz
    L.psispec_draft_sample.argtypes = [P, ctypes.c_int, i64, i32, i32, ctypes.POINTER(Params), P, P, sz, P]
    L.psispec_draft_sample.restype = ctypes.c_int
    L.psispec_verify_linear.argtypes = [P, P, ctypes.c_int, i64, i32, i32, P, ctypes.POINTER(Params), P, P, P, P,
                                        P, sz, P]
    L.psispec_verify_linear.restype = ctypes.c_int
    L.psispec_verify_linear_noalloc.argtypes = [P, P, ctypes.c_int, i64, i32, i32, P, ctypes.POINTER(Params), P, P,
                                                P, P, P]
    L.psispec_verify_linear_noalloc.restype = ctypes.c_int
    L.psispec_tree_depth.argtypes = [P, i32]
    L.psispec_tree_depth.restype = i32
    L.psispec_verify_tree.argtypes = [P, P, ctypes.c_int, i64, i32, i32, P, P, ctypes.POINTER(Params), P, P, P, P,
                                      sz, P]
    L.psispec_verify_tree.restype = ctypes.c_int
    L.psispec_tree_candidates.argtypes = [P, ctypes.c_int, i64, i32, i32, ctypes.POINTER(Params), i32, i32, P, P,
                                          P, sz, P]
    L.psispec_tree_candidates.restype = ctypes.c_int
    L.psispec_verify_tree_det.argtypes = [P, ctypes.c_int, i64, i32, i32, P, P, ctypes.POINTER(Params), P, P, P,
                                          P, sz, P]
    L.psispec_verify_tree_det.restype = ctypes.c_int
    L.psispec_tv_loss.argtypes = [P, P, ctypes.c_int, i64, i32, ctypes.c_float, P, P, P, P, sz, P]
    L.psispec_tv_loss.restype = ctypes.c_int
    L.psispec_toy_logits.argtypes = [i64, i32, P, P, ctypes.c_int, ctypes.POINTER(ToyModel), ctypes.c_int, P, P]
    L.psispec_toy_logits.restype = ctypes.c_int
    L.psispec_generate_workspace_bytes.argtypes = [i64, i32, i32, ctypes.c_int]
    L.psispec_generate_workspace_bytes.restype = sz
    L.psispec_generate_toy.argtypes = [i64, i32, i32, ctypes.c_int, ctypes.POINTER(ToyModel),
                                       ctypes.POINTER(Params), P, i32, P, P, P, P, sz, P]
    L.psispec_generate_toy.restype = ctypes.c_int
    L.psispec_lmhead_workspace_bytes.argtypes = [i64, i32, i32]
    L.psispec_lmhead_workspace_bytes.restype = sz
    L.psispec_verify_lmhead.argtypes = [P, P, P, i64, i32, i32, i32, P, ctypes.POINTER(Params), P, P, P, sz, P]
    L.psispec_verify_lmhead.restype = ctypes.c_int
    L.psispec_strerror.argtypes = [ctypes.c_int]
    L.psispec_strerror.restype = ctypes.c_char_p
    L.psispec_version.argtypes = []
    L.psispec_version.restype = ctypes.c_int
    L.psispec_set_timing_events.argtypes = [P, ctypes.c_int]
    L.psispec_set_timing_events.restype = ctypes.c_int
    L.psispec_timing_count.argtypes = []
    L.psispec_timing_count.restype = ctypes.c_int
    return L


lib = _load()


class KernelTimer:
    """Per-kernel durations of library calls, measured with HIP events that the
    library's kernel launches record at their start and end
    (psispec_set_timing_events).

    Holds `calls` rows of 2 * `kernels` events; `arm(i)` points the library at
    row i, `disarm()` stops recording, `durations()` returns [calls, kernels]
    ms (kernel j of call i is column j) after the stream has been synchronised.
    """

    def __init__(self, calls: int, kernels: int):
        slots = 2 * kernels
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [ctypes.c_void_p]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.calls, self.slots = calls, slots
        self._ev = (ctypes.c_void_p * (calls * slots))()
        for i in range(calls * slots):
            rc = self._hip.hipEventCreate(ctypes.byref(self._ev, i * ctypes.sizeof(ctypes.c_void_p)))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
        self.recorded = [0] * calls

    def arm(self, i: int):
        self._row = i
        lib.psispec_set_timing_events(ctypes.byref(self._ev, i * self.slots * ctypes.sizeof(ctypes.c_void_p)),
                                      self.slots)

    def note(self):
        """Records how many events the last armed call wrote (call after it)."""
        self.recorded[self._row] = lib.psispec_timing_count()

    @staticmethod
    def disarm():
        lib.psispec_set_timing_events(None, 0)

    def durations(self):
        import numpy as np

        out = np.full((self.calls, self.slots // 2), np.nan)
        ms = ctypes.c_float()
        for i in range(self.calls):
            for j in range(self.recorded[i] // 2):
                a, b = self._ev[i * self.slots + 2 * j], self._ev[i * self.slots + 2 * j + 1]
                if self._hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0:
                    out[i, j] = ms.value
        return out

    def __del__(self):
        try:
            self.disarm()
            for i in range(self.calls * self.slots):
                self._hip.hipEventDestroy(self._ev[i])
        except Exception:
            pass


def strerror(status: int) -> str:
    return lib.psispec_strerror(int(status)).decode()


def version() -> int:
    return lib.psispec_version()


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


def workspace_bytes(B: int, rows_per_req: int, V: int, dtype: int) -> int:
    return int(lib.psispec_workspace_bytes(int(B), int(rows_per_req), int(V), int(dtype)))


def tv_workspace_bytes(R: int, V: int, dtype: int) -> int:
    return int(lib.psispec_tv_workspace_bytes(int(R), int(V), int(dtype)))


def make_params(temperature=1.0, top_k=0, top_p=1.0, seed=0, step=0, fused=False) -> Params:
    return Params(float(temperature), int(top_k), float(top_p), FUSED_DRAFT if fused else 0, int(seed) & (2**64 - 1),
                  int(step) & 0xFFFFFFFF, 0)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, rc):
    if rc != OK:
        raise PsiSpecError(fn, rc)


def _workspace(ws, nbytes, device):
    if ws is None:
        return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < nbytes:
        raise PsiSpecError("workspace", EWORKSPACE)
    return ws


def draft_sample(q: torch.Tensor, temperature=1.0, top_k=0, top_p=1.0, seed=0, step=0, out=None, workspace=None,
                 stream=None) -> torch.Tensor:
    """Draft tokens [B, K] int32 drawn from q [B, K, V] (psispec_draft_sample)."""
    assert q.is_cuda and q.is_contiguous() and q.dim() == 3
    B, K, V = q.shape
    dt = dtype_code(q)
    out = out if out is not None else torch.empty((B, K), dtype=torch.int32, device=q.device)
    ws = _workspace(workspace, workspace_bytes(B, K, V, dt), q.device)
    prm = make_params(temperature, top_k, top_p, seed, step)
    rc = lib.psispec_draft_sample(_ptr(q), dt, B, K, V, ctypes.byref(prm), _ptr(out), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream))
    _check("psispec_draft_sample", rc)
    return out


def verify_linear(p: torch.Tensor, q: torch.Tensor, draft_tokens: torch.Tensor | None, temperature=1.0, top_k=0,
                  top_p=1.0, seed=0, step=0, fused=False, out=None, want_probs=True, want_resid=True,
                  workspace=None, stream=None) -> dict:
    """psispec_verify_linear. p [B, K+1, V], q [B, K, V]; draft_tokens [B, K] int32
    (written when fused). Returns dict(tokens [B, K+1], len [B], probs [B, K, 2]
    or None, resid [B] or None, draft [B, K])."""
    assert p.is_cuda and q.is_cuda and p.is_contiguous() and q.is_contiguous()
    B, K1, V = p.shape
    K = K1 - 1
    assert q.shape == (B, K, V) and p.dtype == q.dtype
    dt = dtype_code(p)
    dev = p.device
    if draft_tokens is None:
        if not fused:
            raise ValueError("draft_tokens required unless fused=True")
        draft_tokens = torch.empty((B, K), dtype=torch.int32, device=dev)
    assert draft_tokens.dtype == torch.int32 and draft_tokens.is_contiguous()
    if out is None:
        out = dict(tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev),
                   len=torch.empty((B,), dtype=torch.int32, device=dev),
                   probs=torch.empty((B, K, 2), dtype=torch.float32, device=dev) if want_probs else None,
                   resid=torch.empty((B,), dtype=torch.float64, device=dev) if want_resid else None)
    ws = _workspace(workspace, workspace_bytes(B, 2 * K + 1, V, dt), dev)
    prm = make_params(temperature, top_k, top_p, seed, step, fused)
    rc = lib.psispec_verify_linear(_ptr(p), _ptr(q), dt, B, K, V, _ptr(draft_tokens), ctypes.byref(prm),
                                   _ptr(out["tokens"]), _ptr(out["len"]), _ptr(out.get("probs")),
                                   _ptr(out.get("resid")), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check("psispec_verify_linear", rc)
    out["draft"] = draft_tokens
    return out


def verify_linear_noalloc(p: torch.Tensor, q: torch.Tensor, draft_tokens: torch.Tensor | None, temperature=1.0,
                          top_k=0, top_p=1.0, seed=0, step=0, fused=False, out=None, want_probs=True,
                          want_resid=True, stream=None) -> dict:
    """psispec_verify_linear_noalloc: psispec_verify_linear with the library's
    fixed device scratch as its workspace. Same arguments and outputs as
    verify_linear (outputs are allocated here only when `out` is None)."""
    assert p.is_cuda and q.is_cuda and p.is_contiguous() and q.is_contiguous()
    B, K1, V = p.shape
    K = K1 - 1
    assert q.shape == (B, K, V) and p.dtype == q.dtype
    dt = dtype_code(p)
    dev = p.device
    if draft_tokens is None:
        if not fused:
            raise ValueError("draft_tokens required unless fused=True")
        draft_tokens = torch.empty((B, K), dtype=torch.int32, device=dev)
    assert draft_tokens.dtype == torch.int32 and draft_tokens.is_contiguous()
    if out is None:
        out = dict(tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev),
                   len=torch.empty((B,), dtype=torch.int32, device=dev),
                   probs=torch.empty((B, K, 2), dtype=torch.float32, device=dev) if want_probs else None,
                   resid=torch.empty((B,), dtype=torch.float64, device=dev) if want_resid else None)
    prm = make_params(temperature, top_k, top_p, seed, step, fused)
    rc = lib.psispec_verify_linear_noalloc(_ptr(p), _ptr(q), dt, B, K, V, _ptr(draft_tokens), ctypes.byref(prm),
                                           _ptr(out["tokens"]), _ptr(out["len"]), _ptr(out.get("probs")),
                                           _ptr(out.get("resid")), _stream(stream))
    _check("psispec_verify_linear_noalloc", rc)
    out["draft"] = draft_tokens
    return out


def tree_depth(parent) -> int:
    import numpy as np

    par = np.ascontiguousarray(parent, dtype=np.int32)
    return int(lib.psispec_tree_depth(par.ctypes.data_as(ctypes.c_void_p), par.size))


def verify_tree(p: torch.Tensor, q: torch.Tensor, parent, node_tokens, temperature=1.0, top_k=0, top_p=1.0,
                seed=0, step=0, fused=False, out=None, workspace=None, stream=None) -> dict:
    """psispec_verify_tree. p, q [B, N+1, V]; parent: host int sequence [N];
    node_tokens [B, N] int32 (input; output when fused, allocated if None).
    Returns dict(tokens [B, D+1], path [B, D], len [B], nodes [B, N])."""
    import numpy as np

    assert p.is_cuda and q.is_cuda and p.is_contiguous() and q.is_contiguous()
    B, R, V = p.shape
    N = R - 1
    assert q.shape == p.shape and p.dtype == q.dtype
    par = np.ascontiguousarray(parent, dtype=np.int32)
    assert par.size == N
    D = int(lib.psispec_tree_depth(par.ctypes.data_as(ctypes.c_void_p), N))
    if D < 0:
        raise PsiSpecError("psispec_tree_depth", D)
    dt = dtype_code(p)
    dev = p.device
    if node_tokens is None:
        assert fused, "node_tokens are required unless fused"
        node_tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
    assert node_tokens.is_cuda and node_tokens.dtype == torch.int32 and node_tokens.shape == (B, N)
    if out is None:
        out = dict(tokens=torch.empty((B, D + 1), dtype=torch.int32, device=dev),
                   path=torch.empty((B, D), dtype=torch.int32, device=dev),
                   len=torch.empty((B,), dtype=torch.int32, device=dev))
    ws = _workspace(workspace, workspace_bytes(B, 2 * R, V, dt), dev)
    prm = make_params(temperature, top_k, top_p, seed, step, fused)
    rc = lib.psispec_verify_tree(_ptr(p), _ptr(q), dt, B, N, V, par.ctypes.data_as(ctypes.c_void_p),
                                 _ptr(node_tokens), ctypes.byref(prm), _ptr(out["tokens"]), _ptr(out["path"]),
                                 _ptr(out["len"]), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check("psispec_verify_tree", rc)
    out["nodes"] = node_tokens
    return out


def tree_candidates(q: torch.Tensor, cands: int, nodes: int, temperature=1.0, out=None, workspace=None,
                    stream=None) -> dict:
    """psispec_tree_candidates. q [B, K, V] draft logits. Returns dict(parent
    [B, nodes], tokens [B, nodes]) int32: the `nodes` most probable prefixes over
    the top-`cands` tokens of every position, best first."""
    assert q.is_cuda and q.is_contiguous() and q.dim() == 3
    B, K, V = q.shape
    dt = dtype_code(q)
    if out is None:
        out = dict(parent=torch.empty((B, nodes), dtype=torch.int32, device=q.device),
                   tokens=torch.empty((B, nodes), dtype=torch.int32, device=q.device))
    ws = _workspace(workspace, workspace_bytes(B, K, V, dt), q.device)
    prm = make_params(temperature)
    rc = lib.psispec_tree_candidates(_ptr(q), dt, B, K, V, ctypes.byref(prm), int(cands), int(nodes),
                                     _ptr(out["parent"]), _ptr(out["tokens"]), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream))
    _check("psispec_tree_candidates", rc)
    return out


def verify_tree_det(p: torch.Tensor, parent: torch.Tensor, node_tokens: torch.Tensor, temperature=1.0, seed=0,
                    step=0, out=None, workspace=None, stream=None) -> dict:
    """psispec_verify_tree_det. p [B, N+1, V]; parent and node_tokens [B, N]
    int32 device tensors (one tree per request). Returns dict(tokens [B, N+1],
    path [B, N], len [B])."""
    assert p.is_cuda and p.is_contiguous() and p.dim() == 3
    B, R, V = p.shape
    N = R - 1
    for t in (parent, node_tokens):
        assert t.is_cuda and t.dtype == torch.int32 and t.is_contiguous() and t.shape == (B, N)
    dt = dtype_code(p)
    dev = p.device
    if out is None:
        out = dict(tokens=torch.empty((B, N + 1), dtype=torch.int32, device=dev),
                   path=torch.empty((B, N), dtype=torch.int32, device=dev),
                   len=torch.empty((B,), dtype=torch.int32, device=dev))
    ws = _workspace(workspace, workspace_bytes(B, R, V, dt), dev)
    prm = make_params(temperature, seed=seed, step=step)
    rc = lib.psispec_verify_tree_det(_ptr(p), dt, B, N, V, _ptr(parent), _ptr(node_tokens), ctypes.byref(prm),
                                     _ptr(out["tokens"]), _ptr(out["path"]), _ptr(out["len"]), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream))
    _check("psispec_verify_tree_det", rc)
    return out


def tv_loss(p: torch.Tensor, q: torch.Tensor, temperature=1.0, row_weights: torch.Tensor | None = None, grad=True,
            out=None, workspace=None, stream=None) -> dict:
    """psispec_tv_loss. Teacher logits p and student logits q [..., V] (same
    shape and dtype). Returns dict(loss [R] float64, grad [R, V] in the logits'
    dtype or None), R = the product of the leading dimensions."""
    assert p.is_cuda and q.is_cuda and p.is_contiguous() and q.is_contiguous()
    assert p.shape == q.shape and p.dtype == q.dtype
    V = p.shape[-1]
    R = p.numel() // V
    dt = dtype_code(p)
    dev = p.device
    if row_weights is not None:
        assert row_weights.is_cuda and row_weights.dtype == torch.float32 and row_weights.numel() == R
    if out is None:
        out = dict(loss=torch.empty((R,), dtype=torch.float64, device=dev),
                   grad=torch.empty((R, V), dtype=p.dtype, device=dev) if grad else None)
    ws = _workspace(workspace, tv_workspace_bytes(R, V, dt), dev)
    rc = lib.psispec_tv_loss(_ptr(p), _ptr(q), dt, R, V, float(temperature), _ptr(row_weights), _ptr(out["loss"]),
                             _ptr(out.get("grad")), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check("psispec_tv_loss", rc)
    return out


def toy_model(seed=1234, sd=2.0, n_heavy=1, boost=6.0, rho=0.8, noise=1.5) -> ToyModel:
    return ToyModel(int(seed) & (2**64 - 1), float(sd), int(n_heavy), float(boost), float(rho), float(noise), 0)


def toy_logits(ctx: torch.Tensor, V: int, pos: torch.Tensor | None = None, kind=0, dtype=torch.bfloat16,
               model: ToyModel | None = None, out=None, stream=None) -> torch.Tensor:
    """psispec_toy_logits: ctx [rows, 2] int32 (and pos [rows] for kind 1) ->
    logits [rows, V] of the synthetic toy model."""
    assert ctx.is_cuda and ctx.dtype == torch.int32 and ctx.is_contiguous()
    rows = ctx.numel() // 2
    m = model if model is not None else toy_model()
    out = out if out is not None else torch.empty((rows, V), dtype=dtype, device=ctx.device)
    rc = lib.psispec_toy_logits(rows, int(V), _ptr(ctx), _ptr(pos), int(kind), ctypes.byref(m), dtype_code(out),
                                _ptr(out), _stream(stream))
    _check("psispec_toy_logits", rc)
    return out


def generate_toy(prompt: torch.Tensor, block: int, V: int, rounds: int, temperature=1.0, seed=0, step=0,
                 dtype=torch.bfloat16, model: ToyModel | None = None, out=None, workspace=None, stream=None) -> dict:
    """psispec_generate_toy: prompt [B, 2] int32 -> dict(seq [B, rounds*(block+1)],
    len [B], round_tokens [B, rounds])."""
    assert prompt.is_cuda and prompt.dtype == torch.int32 and prompt.is_contiguous()
    B = prompt.numel() // 2
    dev = prompt.device
    m = model if model is not None else toy_model()
    dt = DTYPE_BF16 if dtype == torch.bfloat16 else DTYPE_F32
    if out is None:
        out = dict(seq=torch.empty((B, rounds * (block + 1)), dtype=torch.int32, device=dev),
                   len=torch.empty((B,), dtype=torch.int32, device=dev),
                   round_tokens=torch.empty((B, rounds), dtype=torch.int32, device=dev))
    nbytes = int(lib.psispec_generate_workspace_bytes(B, int(block), int(V), dt))
    ws = _workspace(workspace, nbytes, dev)
    prm = make_params(temperature, seed=seed, step=step)
    rc = lib.psispec_generate_toy(B, int(block), int(V), dt, ctypes.byref(m), ctypes.byref(prm), _ptr(prompt),
                                  int(rounds), _ptr(out["seq"]), _ptr(out["len"]), _ptr(out["round_tokens"]),
                                  _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check("psispec_generate_toy", rc)
    return out


def verify_lmhead(h_target: torch.Tensor, h_draft: torch.Tensor, w_vocab: torch.Tensor, draft_tokens: torch.Tensor,
                  temperature=1.0, seed=0, step=0, out=None, workspace=None, stream=None) -> dict:
    """psispec_verify_lmhead. h_target [B, K+1, H], h_draft [B, K, H], w_vocab
    [V, H] (bf16), draft_tokens [B, K] int32. Returns dict(tokens [B, K+1], len [B])."""
    for t in (h_target, h_draft, w_vocab):
        assert t.is_cuda and t.is_contiguous() and t.dtype == torch.bfloat16
    B, K1, H = h_target.shape
    K = K1 - 1
    V = w_vocab.shape[0]
    assert h_draft.shape == (B, K, H) and w_vocab.shape == (V, H)
    assert draft_tokens.is_cuda and draft_tokens.dtype == torch.int32 and draft_tokens.shape == (B, K)
    dev = h_target.device
    if out is None:
        out = dict(tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev),
                   len=torch.empty((B,), dtype=torch.int32, device=dev))
    ws = _workspace(workspace, int(lib.psispec_lmhead_workspace_bytes(B, K, V)), dev)
    prm = make_params(temperature, seed=seed, step=step)
    rc = lib.psispec_verify_lmhead(_ptr(h_target), _ptr(h_draft), _ptr(w_vocab), B, K, H, V, _ptr(draft_tokens),
                                   ctypes.byref(prm), _ptr(out["tokens"]), _ptr(out["len"]), _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(stream))
    _check("psispec_verify_lmhead", rc)
    return out
