"""Python binding of the low-rank draft LM head (argument marshalling only).

Every step of the head runs in liblrhead.so's HIP kernels; this module checks
tensor dtypes, devices and shapes, hands raw device pointers and torch's
current HIP stream to the C ABI, and allocates outputs and the workspace with
torch. See include/lrhead.h for the operations and their contracts.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib

_DTYPES = {torch.bfloat16: _lib.BF16, torch.float32: _lib.FP32}


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


class Head:
    """A low-rank head (Q: r x d, P: V x r) with its full-rank head W (V x d).

    The tensors must live on one ROCm device, share dtype (bfloat16 or
    float32) and be contiguous; they are borrowed, not copied.
    """

    def __init__(self, Q: torch.Tensor, P: torch.Tensor, W: torch.Tensor, *,
                 B_max: int, k_max: int, workspace: torch.Tensor | None = None):
        _need(Q.dtype in _DTYPES, f"unsupported dtype {Q.dtype}")
        _need(P.dtype == Q.dtype and W.dtype == Q.dtype, "Q, P, W must share a dtype")
        _need(Q.dim() == 2 and P.dim() == 2 and W.dim() == 2, "Q, P, W must be matrices")
        r, d = Q.shape
        V = P.shape[0]
        _need(tuple(P.shape) == (V, r), f"P is {tuple(P.shape)}, expected ({V}, {r})")
        _need(tuple(W.shape) == (V, d), f"W is {tuple(W.shape)}, expected ({V}, {d})")
        for name, t in (("Q", Q), ("P", P), ("W", W)):
            _need(t.is_cuda and t.device == Q.device, f"{name} must be on {Q.device}")
            _need(t.is_contiguous(), f"{name} must be contiguous")
        self.lib = _lib.load()
        self.dtype = Q.dtype
        self.code = _DTYPES[Q.dtype]
        self.device = Q.device
        self.V, self.d, self.r = int(V), int(d), int(r)
        self.B_max, self.k_max = int(B_max), int(k_max)
        nbytes = self.lib.lrhead_workspace_bytes(self.code, V, d, r, B_max, k_max)
        if nbytes == 0:
            _lib.check(self.lib.lrhead_create(ctypes.byref(ctypes.c_void_p()), self.code, V, d, r,
                                              None, None, None, B_max, k_max, None, 0),
                       "lrhead_workspace_bytes")
        if workspace is None:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        _need(workspace.dtype == torch.uint8 and workspace.is_cuda and workspace.numel() >= nbytes,
              f"workspace must be a uint8 device tensor of >= {nbytes} bytes")
        self.workspace = workspace
        self._tensors = (Q, P, W)
        self._h = ctypes.c_void_p()
        rc = self.lib.lrhead_create(ctypes.byref(self._h), self.code, V, d, r, _ptr(Q), _ptr(P), _ptr(W),
                                    B_max, k_max, _ptr(workspace), workspace.numel())
        _lib.check(rc, "lrhead_create")

    # ------------------------------------------------------------ helpers
    def _stream(self):
        return ctypes.c_void_p(torch.cuda.current_stream(self.device).cuda_stream)

    def _rows(self, H: torch.Tensor) -> int:
        _need(H.dtype == self.dtype, f"H must be {self.dtype}")
        _need(H.dim() == 2 and H.shape[1] == self.d, f"H must be (B, {self.d})")
        _need(H.is_cuda and H.device == self.device and H.is_contiguous(), "H must be contiguous on the device")
        return int(H.shape[0])

    def _out(self, shape, dtype):
        return torch.empty(shape, dtype=dtype, device=self.device)

    # -------------------------------------------------------------- calls
    def candidates(self, H: torch.Tensor, k: int, *, want_score: bool = True):
        """Low-rank retrieval: (idx int32 [B, k], score fp32 [B, k] or None)."""
        B = self._rows(H)
        idx = self._out((B, k), torch.int32)
        score = self._out((B, k), torch.float32) if want_score else None
        _lib.check(self.lib.lrhead_candidates(self._h, _ptr(H), B, k, _ptr(idx), _ptr(score), self._stream()),
                   "lrhead_candidates")
        return idx, score

    def logits(self, H: torch.Tensor, idx: torch.Tensor) -> torch.Tensor:
        """Exact full-rank logits of the given ids (fp32 [B, k])."""
        B = self._rows(H)
        _need(idx.dtype == torch.int32 and idx.dim() == 2 and idx.shape[0] == B, "idx must be int32 (B, k)")
        _need(idx.is_cuda and idx.is_contiguous(), "idx must be contiguous on the device")
        k = int(idx.shape[1])
        out = self._out((B, k), torch.float32)
        _lib.check(self.lib.fullhead_logits(self._h, _ptr(H), B, _ptr(idx), k, _ptr(out), self._stream()),
                   "fullhead_logits")
        return out

    def dense_logits(self, H: torch.Tensor) -> torch.Tensor:
        """All V full-head logits (fp32 [B, V]); a test aid."""
        B = self._rows(H)
        out = self._out((B, self.V), torch.float32)
        _lib.check(self.lib.fullhead_logits(self._h, _ptr(H), B, None, 0, _ptr(out), self._stream()),
                   "fullhead_logits(dense)")
        return out

    def full_topk(self, H: torch.Tensor, k: int, *, out=None):
        """Full-head baseline: (idx int32 [B, k], logits fp32 [B, k])."""
        B = self._rows(H)
        if out is None:
            idx = self._out((B, k), torch.int32)
            logits = self._out((B, k), torch.float32)
        else:
            idx, logits = out
        _lib.check(self.lib.fullhead_topk(self._h, _ptr(H), B, k, _ptr(idx), _ptr(logits), self._stream()),
                   "fullhead_topk")
        return idx, logits

    def draft(self, H: torch.Tensor, k: int, *, want_score: bool = True, out=None):
        """One draft-head call: (idx, score or None, logits), all [B, k]."""
        B = self._rows(H)
        if out is None:
            idx = self._out((B, k), torch.int32)
            score = self._out((B, k), torch.float32) if want_score else None
            logits = self._out((B, k), torch.float32)
        else:
            idx, score, logits = out
        _lib.check(self.lib.lrhead_draft(self._h, _ptr(H), B, k, _ptr(idx), _ptr(score), _ptr(logits),
                                         self._stream()), "lrhead_draft")
        return idx, score, logits

    def set_stage_events(self, before, after) -> None:
        """Attach two hipEvent_t handles (ints or None) to the score pass's dispatch: its start and end."""
        _lib.check(self.lib.lrhead_set_stage_events(self._h, before, after), "lrhead_set_stage_events")

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            self.lib.lrhead_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def draft_static(Q: torch.Tensor, P: torch.Tensor, W: torch.Tensor, H: torch.Tensor, k: int, *,
                 want_score: bool = True, out=None):
    """One draft-head call through lrhead_draft_static: no handle and no
    workspace (the library's own device scratch); returns (idx, score or
    None, logits), all [B, k]. Outputs are allocated here unless `out`
    gives them."""
    _need(Q.dtype in _DTYPES and P.dtype == Q.dtype and W.dtype == Q.dtype and H.dtype == Q.dtype,
          "Q, P, W and H must share a supported dtype")
    for name, t in (("Q", Q), ("P", P), ("W", W), ("H", H)):
        _need(t.is_cuda and t.device == Q.device and t.is_contiguous() and t.dim() == 2,
              f"{name} must be a contiguous matrix on {Q.device}")
    r, d = Q.shape
    V = P.shape[0]
    B = H.shape[0]
    _need(tuple(P.shape) == (V, r) and tuple(W.shape) == (V, d) and H.shape[1] == d, "shapes of Q, P, W, H disagree")
    if out is None:
        idx = torch.empty((B, k), dtype=torch.int32, device=Q.device)
        score = torch.empty((B, k), dtype=torch.float32, device=Q.device) if want_score else None
        logits = torch.empty((B, k), dtype=torch.float32, device=Q.device)
    else:
        idx, score, logits = out
    lib = _lib.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream(Q.device).cuda_stream)
    _lib.check(lib.lrhead_draft_static(_DTYPES[Q.dtype], V, d, r, _ptr(Q), _ptr(P), _ptr(W), _ptr(H), B, k,
                                       _ptr(idx), _ptr(score), _ptr(logits), stream), "lrhead_draft_static")
    return idx, score, logits


def branch(logits: torch.Tensor, idx: torch.Tensor, nb: int, parent: torch.Tensor | None = None):
    """Draft distribution over each row's candidates and its nb branches.

    logits: [B, k] float32, idx: [B, k] int32 (as returned by Head.draft),
    parent: optional [B] float32 path probabilities. Returns (probs [B, k],
    branch ids [B, nb], branch probabilities [B, nb], branch path
    probabilities [B, nb]); see lrhead_branch in include/lrhead.h.
    """
    _need(logits.is_cuda and idx.is_cuda, "logits and idx must be device tensors")
    _need(logits.dtype == torch.float32 and idx.dtype == torch.int32, "logits float32, idx int32")
    _need(logits.dim() == 2 and idx.shape == logits.shape, "logits and idx must be [B, k] alike")
    _need(logits.is_contiguous() and idx.is_contiguous(), "logits and idx must be contiguous")
    B, k = logits.shape
    if parent is not None:
        _need(parent.is_cuda and parent.dtype == torch.float32 and parent.shape == (B,) and parent.is_contiguous(),
              "parent must be a contiguous float32 device tensor of shape [B]")
    lib = _lib.load()
    dev = logits.device
    probs = torch.empty((B, k), dtype=torch.float32, device=dev)
    br_idx = torch.empty((B, nb), dtype=torch.int32, device=dev)
    br_prob = torch.empty((B, nb), dtype=torch.float32, device=dev)
    br_path = torch.empty((B, nb), dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    _lib.check(lib.lrhead_branch(_ptr(logits), _ptr(idx), _ptr(parent), B, k, nb, _ptr(probs), _ptr(br_idx),
                                 _ptr(br_prob), _ptr(br_path), stream), "lrhead_branch")
    return probs, br_idx, br_prob, br_path


def factor(W: torch.Tensor, r: int, omega: torch.Tensor, q: int = 1):
    """A low-rank head (P: [V, r], Q: [r, d], bf16) built from W ([V, d], bf16)
    with the Gaussian test matrix omega ([d, r], float32); q subspace
    iterations. See lrhead_factor in include/lrhead.h."""
    _need(W.is_cuda and W.dtype == torch.bfloat16 and W.dim() == 2 and W.is_contiguous(),
          "W must be a contiguous bfloat16 device matrix")
    V, d = W.shape
    _need(omega.is_cuda and omega.dtype == torch.float32 and tuple(omega.shape) == (d, r) and omega.is_contiguous(),
          f"omega must be a contiguous float32 device tensor of shape ({d}, {r})")
    lib = _lib.load()
    nbytes = lib.lrhead_factor_workspace_bytes(V, d, r)
    _need(nbytes > 0, f"r = {r} outside [1, min(512, d, V)]")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=W.device)
    P = torch.empty((V, r), dtype=torch.bfloat16, device=W.device)
    Q = torch.empty((r, d), dtype=torch.bfloat16, device=W.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream(W.device).cuda_stream)
    _lib.check(lib.lrhead_factor(_ptr(W), V, d, r, q, _ptr(omega), _ptr(P), _ptr(Q), _ptr(ws), nbytes, stream),
               "lrhead_factor")
    return P, Q
