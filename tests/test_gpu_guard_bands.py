"""Guard bands: every output is written inside a buffer whose bytes before
and after (and, for padded rows, between rows) hold a seeded random pattern;
after the call those bytes must be unchanged, and the outputs must still
match the float64 oracle. Shapes are the tails of every tile size: softmax
rows of odd lengths and lengths one past a vector or a workgroup, long rows
on the split path; attention with 129 / 300 queries (128-query and 32-query
tiles) over 65 / 100 keys (64-key and 128-key tiles)."""

import sys

import numpy as np
import pytest
import torch

import oracle
from attention_softmax_amd import (sms_attention_backward, sms_attention_forward, sms_backward,
                                   sms_forward)
from attention_softmax_amd.workloads import TORCH_DTYPE, draw_mask, draw_x
from tests.parity import compare, decoded, mask_4d, to_np
from tests.tolerance import attention_forward_bounds, compare_attention

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
PRE = 4096   # guard bytes before an output (keeps its start on a 256-byte line)
POST = 4099  # guard bytes after it


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class Guarded:
    """An output tensor inside a byte buffer filled with a seeded pattern;
    ``pitch`` > the last dim pads each row."""

    def __init__(self, shape, dtype, seed, pitch=None):
        self.shape = tuple(shape)
        last = self.shape[-1]
        self.pitch = last if pitch is None else pitch
        esz = torch.empty((), dtype=dtype).element_size()
        rows = int(np.prod(self.shape[:-1])) if len(self.shape) > 1 else 1
        self.nbytes = rows * self.pitch * esz
        g = torch.Generator(device=DEV)
        g.manual_seed(seed)
        self.raw = torch.randint(0, 256, (PRE + self.nbytes + POST,), dtype=torch.uint8,
                                 generator=g, device=DEV)
        self.before = self.raw.clone()
        body = self.raw[PRE:PRE + self.nbytes].view(dtype)
        self.t = body.view(self.shape[:-1] + (self.pitch,))[..., :last]
        self.dtype = dtype

    def check(self, what):
        torch.cuda.synchronize()
        after = self.raw.clone()
        # put the output elements back to their old bytes: then every byte must match
        ab = after[PRE:PRE + self.nbytes].view(self.dtype).view(self.shape[:-1] + (self.pitch,))
        bb = self.before[PRE:PRE + self.nbytes].view(self.dtype).view(
            self.shape[:-1] + (self.pitch,))
        ab[..., :self.shape[-1]] = bb[..., :self.shape[-1]]
        diff = (after != self.before).nonzero().flatten()
        assert diff.numel() == 0, (f"{what}: {diff.numel()} guard bytes changed, first at byte "
                                   f"{int(diff[0]) - PRE} from the output's start")


SOFTMAX_SHAPES = [(2, 3, 5, 1000), (1, 2, 3, 65), (2, 2, 4, 4097), (1, 2, 129, 129),
                  (2, 1, 3, 8), (1, 1, 2, 140000)]


@pytest.mark.parametrize("pad", [0, 24])
@pytest.mark.parametrize("shape", SOFTMAX_SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_softmax_guard_bands(dtype, shape, pad):
    say(f"guard bands softmax {dtype} {shape} pad={pad}")
    td = TORCH_DTYPE[dtype]
    B, H, Sq, Sk = shape
    seed = 7 + sum(shape) + pad
    x = draw_x(shape, dtype, ("normal", 2.0), seed, DEV)
    mask = draw_mask(shape, "b_sq_sk", dtype, ("bernoulli_neginf", 0.2), seed + 1, DEV)
    for causal in (False, True):
        y = Guarded(shape, td, seed + 2, Sk + pad)
        sms_forward(x, mask, y.t, 0.75, causal)
        y.check(f"y {dtype} {shape} causal={causal}")
        ref = oracle.forward(to_np(x), dtype, mask_4d(mask, "b_sq_sk"), 0.75, causal)
        compare(decoded(y.t), ref, dtype, "guarded forward", rowsum=True)
        dy = draw_x(shape, dtype, ("normal", 1.0), seed + 3, DEV)
        dx = Guarded(shape, td, seed + 4, Sk + pad)
        sms_backward(y.t, dy, dx.t, 0.75, causal)
        dx.check(f"dx {dtype} {shape} causal={causal}")
        compare(decoded(dx.t), oracle.backward(to_np(y.t), to_np(dy), dtype, 0.75), dtype,
                "guarded backward")


ATTN_SHAPES = [(129, 65), (300, 100), (129, 100), (300, 65)]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Sq,Sk", ATTN_SHAPES)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_attention_guard_bands(dtype, Sq, Sk, D):
    say(f"guard bands attention {dtype} {Sq}x{Sk} D={D}")
    td = TORCH_DTYPE[dtype]
    B, H, Hk = 2, 4, 2
    seed = 100 + Sq + Sk + D
    q = draw_x((B, H, Sq, D), dtype, ("normal", 1.0), seed, DEV)
    k = draw_x((B, Hk, Sk, D), dtype, ("normal", 1.0), seed + 1, DEV)
    v = draw_x((B, Hk, Sk, D), dtype, ("normal", 1.0), seed + 2, DEV)
    do = draw_x((B, H, Sq, D), dtype, ("normal", 1.0), seed + 3, DEV)
    sc = D ** -0.5
    for causal in (False, True, "bottom_right"):
        tag = f"{dtype} {Sq}x{Sk} D={D} causal={causal}"
        o = Guarded((B, H, Sq, D), td, seed + 4)
        lse = Guarded((B, H, Sq), torch.float32, seed + 5)
        sms_attention_forward(q, k, v, None, sc, causal, o=o.t, lse=lse.t)
        o.check("O " + tag)
        lse.check("LSE " + tag)
        qn, kn, vn, don = (to_np(t) for t in (q, k, v, do))
        o_ref, lse_ref = oracle.attention.forward(qn, kn, vn, dtype, scale=sc, is_causal=causal)
        P, _ = oracle.attention.probabilities(qn, kn, dtype, scale=sc, is_causal=causal)
        bounds = attention_forward_bounds(P, lse_ref, *(oracle.decode(a, dtype)
                                                        for a in (qn, kn, vn)),
                                          o_ref, float(np.float32(sc)), dtype)
        compare_attention(oracle.decode(to_np(o.t), dtype), o_ref, bounds, dtype,
                          "guarded O " + tag, to_np(lse.t), lse_ref)
        dq = Guarded((B, H, Sq, D), td, seed + 6)
        dk = Guarded((B, Hk, Sk, D), td, seed + 7)
        dv = Guarded((B, Hk, Sk, D), td, seed + 8)
        sms_attention_backward(q, k, v, o.t, lse.t, do, None, sc, causal, dq=dq.t, dk=dk.t,
                               dv=dv.t)
        for g, n in ((dq, "dQ"), (dk, "dK"), (dv, "dV")):
            g.check(f"{n} {tag}")
        # the guarded gradients equal those written into plain tensors
        rq, rk, rv = sms_attention_backward(q, k, v, o.t.contiguous(), lse.t.contiguous(), do,
                                            None, sc, causal)
        torch.cuda.synchronize()
        for g, r, n in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
            assert torch.equal(g.t, r), f"guarded {n} differs ({tag})"
