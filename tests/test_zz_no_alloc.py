"""sms_forward_noalloc (the forward that allocates nothing: its split rows'
partials live in the library's per-GPU scratch) against sms_forward_ws with a
workspace from torch, through the C ABI: bit-identical outputs on two calls
in a row, the second with a smaller input; short rows (no split); a forced
split too large for the scratch is rejected before any launch."""

import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
from attention_softmax_amd import _lib, sms_workspace_bytes
from attention_softmax_amd.workloads import TORCH_DTYPE, draw_mask, draw_x
from tests.parity import DTYPE_OF, compare, decoded, mask_4d, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def strides(t):
    return _lib.strides4(t.stride())


def call_noalloc(x, mask, y, mode, scale, causal):
    L = _lib.lib()
    code = _lib.DTYPE_CODES[DTYPE_OF[x.dtype]]
    B, H, Sq, Sk = x.shape
    return L.sms_forward_noalloc(x.data_ptr(), strides(x),
                                 None if mask is None else mask.data_ptr(),
                                 _lib.MASK_MODES[mode], y.data_ptr(), strides(y), code,
                                 B, H, Sq, Sk, float(scale), causal,
                                 torch.cuda.current_stream().cuda_stream)


def call_ws(x, mask, y, mode, scale, causal, ws):
    L = _lib.lib()
    code = _lib.DTYPE_CODES[DTYPE_OF[x.dtype]]
    B, H, Sq, Sk = x.shape
    wptr, wbytes = (ws.data_ptr(), ws.numel()) if ws is not None else (None, 0)
    return L.sms_forward_ws(x.data_ptr(), strides(x),
                            None if mask is None else mask.data_ptr(),
                            _lib.MASK_MODES[mode], y.data_ptr(), strides(y), code,
                            B, H, Sq, Sk, float(scale), causal, wptr, wbytes,
                            torch.cuda.current_stream().cuda_stream)


CASES = [
    # (dtype, shape, mask mode, causal): a split-row shape, then a smaller one
    ("f16", (1, 2, 3, 200000), "sq_sk", 0),
    ("f32", (1, 1, 2, 70000), "b_sq_sk", 2),
]


def _inputs(dtype, shape, mode, seed):
    x = draw_x(shape, dtype, ("normal", 2.0), seed, DEV)
    mask = draw_mask(shape, mode, dtype, ("bernoulli_neginf", 0.2), seed + 1, DEV)
    return x, mask


def test_noalloc_matches_workspace_call_twice():
    for i, (dtype, shape, mode, causal) in enumerate(CASES):
        say(f"no-alloc call {i + 1}: {dtype} {shape} mask {mode} causal {causal}")
        need = sms_workspace_bytes(TORCH_DTYPE[dtype], shape)
        assert 0 < need <= _lib.lib().sms_noalloc_scratch_bytes(), need  # rows are split
        x, mask = _inputs(dtype, shape, mode, 7 + i)
        y1 = torch.full_like(x, 3.0)
        assert call_noalloc(x, mask, y1, mode, 0.25, causal) == 0
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        y2 = torch.full_like(x, 5.0)
        assert call_ws(x, mask, y2, mode, 0.25, causal, ws) == 0
        torch.cuda.synchronize()
        assert torch.equal(y1, y2), f"call {i + 1}: no-alloc output differs"
        # and both against the oracle on the first and last rows
        B, H, Sq, Sk = shape
        rows = [0, B * H * Sq - 1]
        ref = oracle.forward_rows(to_np(x), dtype, rows, mask_4d(mask, mode), 0.25,
                                  {0: False, 1: True, 2: "bottom_right"}[causal])
        got = decoded(y1).reshape(-1, Sk)[rows]
        compare(got, ref, dtype, f"no-alloc call {i + 1}", rowsum=True)


def test_noalloc_short_rows_and_errors():
    say("no-alloc short rows and a forced split beyond the scratch")
    x, mask = _inputs("bf16", (2, 3, 5, 1000), "b_sq_sk", 3)
    y1, y2 = torch.empty_like(x), torch.empty_like(x)
    assert call_noalloc(x, mask, y1, "b_sq_sk", 0.5, 1) == 0
    assert call_ws(x, mask, y2, "b_sq_sk", 0.5, 1, None) == 0
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_noalloc_rejects_a_split_beyond_its_scratch(monkeypatch):
    # 300 rows forced into 64 chunks need 300 * 64 * 8 = 153600 bytes
    monkeypatch.setenv("SMS_FORCE_SPLIT", "64")
    x, mask = _inputs("f32", (1, 3, 100, 4096), "sq_sk", 5)
    need = sms_workspace_bytes(torch.float32, tuple(x.shape))
    assert need == 300 * 64 * 8 > _lib.lib().sms_noalloc_scratch_bytes()
    y = torch.full_like(x, 9.0)
    assert call_noalloc(x, mask, y, "sq_sk", 1.0, 0) == 9  # SMS_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert (y == 9.0).all()  # nothing launched
