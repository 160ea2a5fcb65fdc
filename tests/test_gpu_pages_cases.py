"""The pages' own verification cases, through the C ABI, against the float64
oracle (element by element, every row, with the tolerances of
tests/tolerance.py).

* lmnt.cn "Custom fused Softmax operator in CUDA, wrapped into PyTorch",
  sec. 5.1: the test matrix {scale only (no mask, no causal flag); an additive
  mask holding both 0 and -inf; the causal flag only; the causal flag and the
  mask together} x {fp32, fp16} x sequence length {128, 512, 1024}, on
  x [2, 4, S, S] ~ N(0, 1) with scale 1/sqrt(64) and a full-shape
  [2, 4, S, S] mask that is 0 on keys below S/2 and -inf from S/2 on. The
  page compares the forward; the backward (dy ~ N(0, 1)) is checked on the
  same inputs too, as the page's autograd wrapper needs it (sec. 4.3).
* pnsm.cn ScaledMaskSoftmax article, sec. 3.4: logits [2, 8, 128, 128]
  ~ N(0, 1), a full-shape additive mask with -1e9 on key columns 60 and up,
  scale 0.5; in fp32 and in fp16. In fp16, -1e9 has no finite value and the
  mask holds -inf there (the article's sec. 2.3 discusses that very case).

The inputs are drawn by this repository's seeded generator (not torch's
global one the pages seed), so the values differ from the pages' while the
shapes and distributions are theirs.
"""

import sys

import pytest
import torch

import oracle
from attention_softmax_amd import sms_backward, sms_forward
from attention_softmax_amd.workloads import TORCH_DTYPE, draw_x
from tests.parity import compare, decoded, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _run(x, mask, scale, causal, dtype, what, dy_seed):
    y = torch.empty_like(x)
    sms_forward(x, mask, y, scale, causal)
    dy = draw_x(tuple(x.shape), dtype, ("normal", 1.0), dy_seed, DEV)
    dx = torch.empty_like(x)
    sms_backward(y, dy, dx, scale, causal)
    torch.cuda.synchronize()
    ref = oracle.forward(to_np(x), dtype, None if mask is None else to_np(mask), scale, causal)
    s1 = compare(decoded(y), ref, dtype, what, rowsum=True)
    refb = oracle.backward(to_np(y), to_np(dy), dtype, scale)
    s2 = compare(decoded(dx), refb, dtype, what + " backward")
    return ref, s1, s2


LMNT_CASES = ["scale_only", "mask_0_and_neginf", "causal_only", "causal_and_mask"]


@pytest.mark.parametrize("S", [128, 512, 1024])
@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("case", LMNT_CASES)
def test_lmnt_sec_5_1_matrix(case, dtype, S):
    B, H, D = 2, 4, 64
    what = f"lmnt.cn sec. 5.1 {case} {dtype} S={S}"
    say(what)
    seed = 4200 + 10 * LMNT_CASES.index(case) + S // 128
    x = draw_x((B, H, S, S), dtype, ("normal", 1.0), seed, DEV)
    mask = None
    if case in ("mask_0_and_neginf", "causal_and_mask"):
        mask = torch.zeros((B, H, S, S), dtype=TORCH_DTYPE[dtype], device=DEV)
        mask[:, :, :, S // 2:] = -float("inf")
    causal = case in ("causal_only", "causal_and_mask")
    ref, s1, s2 = _run(x, mask, 1.0 / D ** 0.5, causal, dtype, what, seed + 5)
    # the page's own check is against an unfused softmax of x*scale + mask:
    # the masked keys get exactly 0, and with the causal flag every key past
    # the query does
    if mask is not None:
        assert (ref[..., S // 2:] == 0).all()
    say(f"  forward {s1} backward {s2}")


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_pnsm_sec_3_4_padding_mask(dtype):
    B, H, Sq, Sk = 2, 8, 128, 128
    what = f"pnsm.cn sec. 3.4 {dtype}"
    say(what)
    x = draw_x((B, H, Sq, Sk), dtype, ("normal", 1.0), 42, DEV)
    mask = torch.zeros((B, H, Sq, Sk), dtype=TORCH_DTYPE[dtype], device=DEV)
    mask[:, :, :, 60:] = -1e9
    if dtype == "f16":
        assert torch.isinf(mask[0, 0, 0, 60]) and mask[0, 0, 0, 60] < 0
    ref, s1, s2 = _run(x, mask, 0.5, False, dtype, what, 43)
    y = torch.empty_like(x)
    sms_forward(x, mask, y, 0.5, False)
    torch.cuda.synchronize()
    # exp(-1e9 * ...) underflows to exactly 0 in every precision: padded keys
    # get probability 0 and the first 60 keys carry the whole row
    assert (y[..., 60:] == 0).all()
    assert (ref[..., 60:] == 0).all()
    say(f"  forward {s1} backward {s2}")
