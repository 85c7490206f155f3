"""The allocation-free entry point (lrhead_draft_static, the library's own
device scratch) against lrhead_draft on a handle with its own workspace:
the same kernels, so the outputs must agree bit for bit. Two calls in a row,
the second on a smaller input, so that the second call runs over whatever
the first left in the shared scratch."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import gen
import rank_lm_head_amd as lr
from parity_util import check_lowrank, dev

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _draft_static_raw(t, k):
    """lrhead_draft_static through the C ABI (ctypes), outputs from torch."""
    lib = lr.load()
    B = t["H"].shape[0]
    V, r = t["P"].shape
    d = t["Q"].shape[1]
    code = lr.BF16 if t["Q"].dtype == torch.bfloat16 else lr.FP32
    idx = torch.empty((B, k), dtype=torch.int32, device=DEV)
    score = torch.empty((B, k), dtype=torch.float32, device=DEV)
    logits = torch.empty((B, k), dtype=torch.float32, device=DEV)
    p = lambda x: ctypes.c_void_p(x.data_ptr())
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib.lrhead_draft_static(code, V, d, r, p(t["Q"]), p(t["P"]), p(t["W"]), p(t["H"]), B, k, p(idx), p(score),
                                 p(logits), s)
    assert rc == 0, lr._lib.LrheadError(rc, "lrhead_draft_static")
    return idx, score, logits


@pytest.mark.parametrize("shapes", [
    [(20000, 512, 128, 8, "bf16", 64), (5000, 256, 64, 1, "bf16", 16)],     # eight-row path, then the one-row pass
    [(60000, 2048, 128, 1, "bf16", 32), (4096, 256, 32, 1, "fp32", 8)],      # one-row pass with many slices, then fp32
])
def test_static_scratch_matches_the_workspace_call(shapes):
    for V, d, r, B, dt, k in shapes:
        print(f"[run] static scratch V={V} d={d} r={r} B={B} {dt} k={k}", flush=True)
        inp = gen.make_custom(V, d, r, B, dt, seed=V + B)
        t = {x: dev(inp[x], DEV) for x in ("Q", "P", "W", "H")}
        head = lr.Head(t["Q"], t["P"], t["W"], B_max=B, k_max=k)
        ref = [x.cpu().numpy() for x in head.draft(t["H"], k)]
        got = [x.cpu().numpy() for x in _draft_static_raw(t, k)]
        torch.cuda.synchronize()
        for a, b in zip(ref, got):
            assert np.array_equal(a, b)
        if V <= 60000:
            errs, _ = check_lowrank(inp, k, *got)
            assert not errs, errs[:5]
        head.close()


def test_static_scratch_rejects_calls_beyond_it():
    """A call whose workspace exceeds the static scratch fails on the host
    with LRHEAD_EWORKSPACE and enqueues nothing."""
    lib = lr.load()
    need = lib.lrhead_workspace_bytes(lr.BF16, 151936, 5120, 256, 2048, 64)
    assert need > lr._lib.STATIC_SCRATCH_BYTES
    x = torch.empty(16, dtype=torch.uint8, device=DEV)
    p = ctypes.c_void_p(x.data_ptr())
    rc = lib.lrhead_draft_static(lr.BF16, 151936, 5120, 256, p, p, p, p, 2048, 64, p, None, p, None)
    assert rc == lr._lib.EWORKSPACE
    assert b"static scratch" in lib.lrhead_last_error()
