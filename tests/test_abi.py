"""The C ABI loads and exports what include/sms.h declares; host-side argument
checks. CPU only: every call here fails validation (or is a zero-size no-op)
before the library would launch anything."""

import ctypes
import os
import re

import pytest
import torch

from attention_softmax_amd import _lib, causal_code, mask_kind_of, mask_mode_of
from attention_softmax_amd.workloads import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sms.h")

# A non-NULL, 16-byte aligned address that is never dereferenced: every call
# that receives it is rejected by the host-side checks first. The tests that
# pass it run only where no GPU is visible, so that no mistake in a check can
# ever turn one of them into a launch on a real device.
FAKE = 0x10000
FAKE_ODD = 0x10001
no_device = pytest.mark.skipif(torch.cuda.is_available(),
                               reason="passes fake device pointers; host-only test")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sms_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n


def test_noalloc_scratch_size(L):
    # a host-only query: the per-GPU scratch of sms_forward_noalloc holds the
    # largest automatic split (2048 + 255 (row, chunk) pairs of 8 bytes)
    assert L.sms_noalloc_scratch_bytes() == 65536
    assert L.sms_noalloc_scratch_bytes() >= (2048 + 255) * 8


def test_abi_version_and_status_text(L):
    assert L.sms_abi_version() == _lib.ABI_VERSION
    for code, name in _lib.STATUS_NAMES.items():
        text = L.sms_status_str(code).decode()
        assert text and text != "unknown status", (code, name)
    assert L.sms_status_str(99).decode() == "unknown status"


def _fwd(L, x=FAKE, xs=(64, 64, 64, 1), mask=None, mode=0, y=FAKE, ys=(64, 64, 64, 1),
         dtype=0, B=1, H=1, Sq=1, Sk=64, scale=1.0, causal=0):
    return L.sms_forward(x, _lib.strides4(xs) if xs is not None else None, mask, mode, y,
                         _lib.strides4(ys) if ys is not None else None, dtype, B, H, Sq, Sk,
                         scale, causal, None)


def _bwd(L, y=FAKE, dy=FAKE, dx=FAKE, st=(64, 64, 64, 1), dtype=0, B=1, H=1, Sq=1, Sk=64):
    s = _lib.strides4(st)
    return L.sms_backward(y, s, dy, s, dx, s, dtype, B, H, Sq, Sk, 1.0, 0, None)


@no_device
def test_forward_argument_checks(L):
    assert _fwd(L, dtype=7) == 4                                  # dtype
    assert _fwd(L, mode=9) == 5                                   # mask mode
    assert _fwd(L, B=-1) == 2 and _fwd(L, Sk=-3) == 2             # negative dims
    assert _fwd(L, x=None) == 1 and _fwd(L, y=None) == 1          # NULL tensors
    assert _fwd(L, mode=1, mask=None) == 1                        # mask required by mode
    assert _fwd(L, xs=None) == 1                                  # NULL strides
    assert _fwd(L, xs=(64, 64, 64, 2)) == 3                       # key axis not contiguous
    assert _fwd(L, ys=(64, -64, 64, 1)) == 3                      # negative stride
    assert _fwd(L, x=FAKE_ODD) == 6                               # misaligned fp32 pointer
    assert _fwd(L, dtype=1, y=FAKE_ODD) == 6                      # misaligned fp16 pointer
    assert _fwd(L, mode=2, mask=FAKE_ODD) == 6                    # misaligned mask
    assert _fwd(L, Sk=L.sms_max_sk(0) + 1) == 2                   # too long a row
    assert _fwd(L, B=1 << 20, H=1 << 10, Sq=1 << 3) == 2          # 2^33 rows
    assert _fwd(L, Sq=1 << 23, Sk=1 << 20) == 2                   # 2^23 streamed rows: > 2^32 lanes
    assert _fwd(L, Sk=1 << 31) == 2
    assert _fwd(L, mode=0x10) == 5                                # boolean flag without a shape
    assert _fwd(L, mode=0x15, mask=FAKE) == 5                     # boolean key lengths
    assert _fwd(L, mode=6, mask=FAKE) == 5
    assert _fwd(L, causal=3) == 8 and _fwd(L, causal=-1) == 8     # unknown causal mode
    assert _fwd(L, mode=5, mask=FAKE_ODD) == 6                    # int32 lengths misaligned


@no_device
def test_zero_sizes_are_noops(L):
    # NULL pointers are fine when there is nothing to do.
    for dims in ((0, 1, 1, 8), (1, 0, 1, 8), (1, 1, 0, 8), (1, 1, 1, 0)):
        B, H, Sq, Sk = dims
        assert _fwd(L, x=None, y=None, B=B, H=H, Sq=Sq, Sk=Sk) == 0
        assert _bwd(L, y=None, dy=None, dx=None, B=B, H=H, Sq=Sq, Sk=Sk) == 0


@no_device
def test_backward_argument_checks(L):
    assert _bwd(L, dtype=9) == 4
    assert _bwd(L, dy=None) == 1 and _bwd(L, dx=None) == 1
    assert _bwd(L, st=(64, 64, 64, 0)) == 3
    assert _bwd(L, dx=FAKE_ODD) == 6
    assert _bwd(L, Sk=L.sms_max_sk(2) + 1, dtype=2) == 2
    s = _lib.strides4((64, 64, 64, 1))
    assert L.sms_backward(FAKE, s, FAKE, s, FAKE, s, 0, 1, 1, 1, 64, 1.0, 4, None) == 8


@no_device
def test_copy_reference_argument_checks(L):
    assert L.sms_copy_reference(None, None, 0, None) == 0          # nothing to copy
    assert L.sms_copy_reference(FAKE, FAKE + 4096, -16, None) == 2  # negative size
    assert L.sms_copy_reference(None, FAKE, 16, None) == 1
    assert L.sms_copy_reference(FAKE, None, 16, None) == 1
    assert L.sms_copy_reference(FAKE + 8, FAKE + 4096, 16, None) == 6   # src not 16-byte aligned
    assert L.sms_copy_reference(FAKE, FAKE + 4104, 16, None) == 6       # dst not 16-byte aligned
    assert L.sms_copy_reference(FAKE, FAKE + 4096, 24, None) == 6       # size not a multiple of 16
    assert L.sms_copy_reference(FAKE, FAKE + 4096, (1 << 36), None) == 2  # 2^26 KiB: 2^32 lanes


def test_f64_queries(L):
    assert L.sms_max_sk(3) == 1 << 30
    assert L.sms_path(3, 1000, 0) == 4 and L.sms_path(3, 1 << 20, 1) == 4
    assert L.sms_workspace_bytes(3, 1, 1, 8, 1 << 20, 0) == 0   # fp64 rows never split


@no_device
def test_f64_alignment(L):
    assert _fwd(L, dtype=3, x=FAKE + 4) == 6                   # fp64 needs 8-byte alignment
    assert _bwd(L, dtype=3, dy=FAKE + 4) == 6


def test_workspace_sizes(L, monkeypatch):
    """8 bytes per (row, chunk); chunks = min(ceil(2048 / rows), vectors // 1024)
    for fewer than 256 rows of at least 16384 vectors, else no split (0); -1 for
    invalid arguments."""
    monkeypatch.delenv("SMS_FORCE_SPLIT", raising=False)
    monkeypatch.delenv("SMS_SPLIT", raising=False)
    ws = L.sms_workspace_bytes
    # fp16, 8 rows of 2^20 keys: unaligned rows span (2^20 + 14) // 8 = 131073
    # vectors -> min(256, 128) = 128 chunks
    assert ws(1, 1, 1, 8, 1 << 20, 0) == 8 * 128 * 8
    assert ws(1, 1, 1, 8, 1 << 20, 1) == 8 * 128 * 8
    assert ws(0, 1, 2, 1, 1 << 16, 0) == 2 * 16 * 8       # fp32: 16385 vectors -> 16 chunks
    assert ws(0, 1, 1, 255, 1 << 16, 0) == 255 * 9 * 8     # 255 rows -> 9 chunks
    assert ws(0, 1, 1, 256, 1 << 16, 0) == 0               # 256 rows: one workgroup each
    assert ws(1, 1, 1, 4, 1024, 0) == 0                    # 129 vectors: short rows
    assert ws(1, 1, 1, 1, 16383 * 8 - 14, 0) == 0          # 16382 vectors: short rows
    assert ws(1, 1, 1, 1, 16384 * 8 - 14, 0) == 16 * 8     # 16384 vectors: 16 chunks
    assert ws(1, 0, 1, 1, 1 << 20, 0) == 0                 # empty
    assert ws(7, 1, 1, 1, 64, 0) == -1 and ws(0, -1, 1, 1, 64, 0) == -1
    assert ws(0, 1, 1, 1, (1 << 30) + 1, 0) == -1
    monkeypatch.setenv("SMS_FORCE_SPLIT", "3")
    assert ws(0, 2, 3, 4, 100, 0) == 24 * 3 * 8            # forced: any shape
    monkeypatch.setenv("SMS_FORCE_SPLIT", "0")
    monkeypatch.setenv("SMS_SPLIT", "0")
    assert ws(1, 1, 1, 8, 1 << 20, 0) == 0


@no_device
def test_workspace_argument_checks(L):
    s = _lib.strides4((1 << 20, 1 << 20, 1 << 20, 1))
    need = L.sms_workspace_bytes(1, 1, 1, 8, 1 << 20, 0)
    args = (FAKE, s, None, 0, FAKE, s, 1, 1, 1, 8, 1 << 20, 1.0, 0)
    assert L.sms_forward_ws(*args, FAKE, need - 1, None) == 9     # too small
    assert L.sms_forward_ws(*args, FAKE + 4, need, None) == 9     # not 8-byte aligned
    bargs = (FAKE, s, FAKE, s, FAKE, s, 1, 1, 1, 8, 1 << 20, 1.0, 0)
    assert L.sms_backward_ws(*bargs, FAKE, 8, None) == 9
    # argument errors are still reported first
    assert L.sms_forward_ws(FAKE, s, None, 0, None, s, 1, 1, 1, 8, 1 << 20, 1.0, 0, FAKE, 8,
                            None) == 1


def test_max_sk_and_paths(L):
    assert L.sms_max_sk(0) == L.sms_max_sk(1) == L.sms_max_sk(2) == 1 << 30
    assert L.sms_max_sk(5) == 0
    # the benchmark workloads: rows-per-wave, wave-per-row and multi-wave families
    expect = {1: 0, 2: 2, 3: 2, 4: 2, 5: 2}
    code = {"f32": 0, "f16": 1, "bf16": 2}
    for i, c in CONFIGS.items():
        assert L.sms_path(code[c["dtype"]], c["shape"][3], 0) == expect[i], i
    # rows beyond 4096 16-byte vectors stream; beyond 2^30 keys: unsupported
    assert L.sms_path(0, 4096 * 4, 0) == 2 and L.sms_path(0, 4096 * 4 + 1, 0) == 3
    assert L.sms_path(1, 4096 * 8, 1) == 2 and L.sms_path(1, 4096 * 8 + 1, 1) == 3
    # the backward keeps whole-vector rows of up to 8192 vectors in one pass
    assert L.sms_path(1, 4096 * 8 + 8, 1) == 2 and L.sms_path(1, 4096 * 8 + 8, 0) == 3
    assert L.sms_path(0, 8192 * 4, 1) == 2 and L.sms_path(0, 8192 * 4 + 4, 1) == 3
    assert L.sms_path(2, 1 << 30, 0) == 3 and L.sms_path(2, (1 << 30) + 1, 0) == -1


def test_mask_mode_inference():
    shape = (2, 3, 5, 7)
    z = lambda *s: torch.empty(s)  # noqa: E731
    assert mask_mode_of(None, shape) == "none"
    assert mask_mode_of(z(5, 7), shape) == "sq_sk"
    assert mask_mode_of(z(1, 1, 5, 7), shape) == "sq_sk"
    assert mask_mode_of(z(2, 5, 7), shape) == "b_sq_sk"
    assert mask_mode_of(z(2, 1, 5, 7), shape) == "b_sq_sk"
    assert mask_mode_of(z(2, 1, 7), shape) == "b_1_sk"
    assert mask_mode_of(z(2, 1, 1, 7), shape) == "b_1_sk"
    assert mask_mode_of(z(2, 3, 5, 7), shape) == "full"
    for bad in ((3, 5, 7), (5, 6), (2, 3, 1, 7), (7,)):
        with pytest.raises(ValueError):
            mask_mode_of(z(*bad), shape)
    assert mask_mode_of(torch.zeros(2, dtype=torch.int32), shape) == "key_lengths"
    with pytest.raises(ValueError):
        mask_mode_of(torch.zeros(3, dtype=torch.int32), shape)
    assert mask_kind_of(torch.zeros(5, 7, dtype=torch.bool)) == "bool"
    assert mask_kind_of(torch.zeros(5, 7, dtype=torch.uint8)) == "bool"
    assert mask_kind_of(torch.zeros(2, dtype=torch.int64)) == "lengths"
    assert mask_kind_of(torch.zeros(5, 7, dtype=torch.bfloat16)) == "additive"
    assert [causal_code(c) for c in (False, True, "top_left", "bottom_right", None, 2)] == \
        [0, 1, 1, 2, 0, 2]
    with pytest.raises(ValueError):
        causal_code("diagonal")


def test_binding_refuses_cpu_tensors():
    from attention_softmax_amd import sms_forward, sms_backward, scaled_mask_softmax
    x = torch.zeros(1, 1, 2, 8)
    with pytest.raises(ValueError, match="GPU"):
        sms_forward(x, None, torch.empty_like(x))
    with pytest.raises(ValueError, match="GPU"):
        sms_backward(x, x, torch.empty_like(x))
    with pytest.raises(ValueError, match="GPU"):
        scaled_mask_softmax(x)
