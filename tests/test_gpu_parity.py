"""HIP path against the float64 oracle, through the C ABI (via the binding).

Small shapes are checked element by element on every row; the benchmark
workloads at full size are checked here on sampled rows (oracle one row at a
time) plus properties over every row: exact zeros where keys are masked or
causal-future, and row sums. tests/test_gpu_every_row.py checks every row of
them against the oracle.
"""

import math
import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
from attention_softmax_amd import (SmsError, scaled_mask_softmax, sms_backward, sms_forward,
                                   sms_max_sk, sms_workspace_bytes)
from attention_softmax_amd.workloads import (CONFIGS, TORCH_DTYPE, draw_dy, draw_lengths,
                                             draw_mask, draw_x, make_config)
from tests.parity import (DTYPE_OF, compare, decoded, gather_mask_rows, gather_rows, mask_4d,
                          sample_rows, to_np)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def fwd(x, mask=None, scale=1.0, causal=False, y=None):
    y = torch.empty_like(x) if y is None else y
    sms_forward(x, mask, y, scale, causal)
    torch.cuda.synchronize()
    return y


def bwd(y, dy, scale=1.0, causal=False, dx=None):
    dx = torch.empty_like(y) if dx is None else dx
    sms_backward(y, dy, dx, scale, causal)
    torch.cuda.synchronize()
    return dx


def oracle_fwd(x, mask, mode, scale, causal, kind="additive"):
    dt = DTYPE_OF[x.dtype]
    if mask is not None and kind == "lengths":
        return oracle.forward(to_np(x), dt, None, scale, causal, "lengths", to_np(mask))
    return oracle.forward(to_np(x), dt, mask_4d(mask, mode), scale, causal, kind)


def dtname(t):
    return DTYPE_OF[t.dtype]


# ------------------------------------------------------------ shape sweep

SK_SWEEP = [1, 3, 7, 8, 63, 64, 65, 77, 127, 128, 1000, 1001, 1024, 2047, 2048, 2049, 4095,
            4096, 4097, 8192]
MODES = ["none", "sq_sk", "b_sq_sk", "b_1_sk", "full"]


def _mask_kind(mode):
    return ("normal", 2.0) if mode in ("b_1_sk",) else ("bernoulli_neginf", 0.25)


# (shape mode, kind): every additive and boolean shape, key lengths, none
MASK_CASES = ([("none", "none")] + [(m, "additive") for m in MODES[1:]] +
              [(m, "bool") for m in MODES[1:]] + [("key_lengths", "lengths")])
CAUSALS = (False, True, "bottom_right")


def make_mask(shape, mode, kind, dtype, seed):
    """A mask of the given shape mode and kind for x of ``shape``."""
    if kind == "none":
        return None
    if kind == "lengths":
        return draw_lengths(shape[0], 0, shape[3] + 2, seed, DEV)  # 0 .. beyond Sk
    if kind == "bool":
        return draw_mask(shape, mode, dtype, ("bool", 0.3), seed, DEV)
    return draw_mask(shape, mode, dtype, _mask_kind(mode), seed, DEV)


def check_fwd_bwd(x, mask, mode, kind, scale, causal, what, dy_seed=None):
    dtype = dtname(x)
    y = fwd(x, mask, scale, causal)
    compare(decoded(y), oracle_fwd(x, mask, mode, scale, causal, kind), dtype, what, rowsum=True)
    if dy_seed is not None:
        dy = draw_x(tuple(x.shape), dtype, ("normal", 1.0), dy_seed, DEV)
        dx = bwd(y, dy, scale, causal)
        compare(decoded(dx), oracle.backward(to_np(y), to_np(dy), dtype, scale), dtype,
                what + " bwd")
    return y


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "f64"])
@pytest.mark.parametrize("Sk", SK_SWEEP)
def test_sweep_all_modes(dtype, Sk):
    """Every mask shape and kind (additive, boolean, key lengths), no causal rule
    and both causal alignments (Sq = 3 < Sk), on a few rows of each length;
    forward, and backward with the same causal promise."""
    say(f"sweep dtype={dtype} Sk={Sk}")
    shape = (2, 2, 3, Sk)
    for mode, kind in MASK_CASES:
        for causal in CAUSALS:
            seed = zlib.crc32(f"{dtype}/{Sk}/{mode}/{kind}/{causal}".encode()) % 10000
            x = draw_x(shape, dtype, ("normal", 3.0), seed, DEV)
            mask = make_mask(shape, mode, kind, dtype, seed + 1)
            check_fwd_bwd(x, mask, mode, kind, 0.3, causal,
                          f"{dtype} Sk={Sk} {mode}/{kind} causal={causal}",
                          dy_seed=seed + 2 if causal else None)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("Sk", [1, 8, 77, 1000, 2048])
def test_bottom_right_causal_more_queries_than_keys(dtype, Sk, monkeypatch):
    """Sq > Sk with the bottom-right rule: the first Sq - Sk rows have no key and
    are all zeros; through both the general and the aligned-row kernels."""
    say(f"bottom-right Sq>Sk dtype={dtype} Sk={Sk}")
    shape = (1, 2, Sk + 5, Sk)
    for fast in ("1", "0"):
        monkeypatch.setenv("SMS_FAST", fast)
        for mode, kind in (("none", "none"), ("sq_sk", "bool"), ("key_lengths", "lengths"),
                           ("b_sq_sk", "additive")):
            seed = zlib.crc32(f"br/{dtype}/{Sk}/{mode}/{kind}".encode()) % 10000
            x = draw_x(shape, dtype, ("normal", 3.0), seed, DEV)
            mask = make_mask(shape, mode, kind, dtype, seed + 1)
            y = check_fwd_bwd(x, mask, mode, kind, 0.5, "bottom_right",
                              f"BR {dtype} Sk={Sk} {mode}/{kind} fast={fast}", dy_seed=seed + 2)
            assert (y[:, :, :5] == 0).all()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("Sk", [5, 64, 200, 1000, 1030, 4096])
def test_causal_square(dtype, Sk):
    """Sq = Sk causal: every query position, sampled rows against the oracle and
    exact zeros after the diagonal on every row."""
    say(f"causal square dtype={dtype} Sk={Sk}")
    shape = (1, 2, Sk, Sk)
    x = draw_x(shape, dtype, ("normal", 8.0), Sk, DEV)
    mask = draw_mask(shape, "sq_sk", dtype, ("bernoulli_neginf", 0.1), Sk + 7, DEV)
    y = fwd(x, mask, 1 / math.sqrt(128), True)
    fut = torch.triu(torch.ones(Sk, Sk, dtype=torch.bool, device=DEV), diagonal=1)
    assert (y[:, :, fut] == 0).all()
    rows = sample_rows(2 * Sk, Sk, k=min(2 * Sk, 160), seed=Sk)
    xr, mr = gather_rows(x, rows), gather_mask_rows(mask, "sq_sk", shape, rows)
    yr = oracle.decode(gather_rows(y, rows), dtype)
    for i, r in enumerate(rows):
        q = r % Sk
        ref = oracle.forward_row(xr[i], dtype, mr[i], 1 / math.sqrt(128), True, q)
        compare(yr[i], ref, dtype, f"row {r}")


# ------------------------------------------------ workloads, reduced sizes

SMALL = {1: (1, 2, 64, 64), 2: (2, 4, 64, 1024), 3: (1, 2, 2048, 2048),
         4: (1, 2, 4096, 4096), 5: (2, 2, 1000, 1000)}


@pytest.mark.parametrize("fast", ["1", "0"])
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_workload_recipe_small(cfg, fast, monkeypatch):
    """Each workload's recipe (dtype, distributions, mask mode, causal, scale) at
    a size the oracle covers on every row; forward and backward; through the
    aligned-row persistent kernels (fast=1) and the general kernels (fast=0)."""
    monkeypatch.setenv("SMS_FAST", fast)
    say(f"workload {cfg} small shape {SMALL[cfg]} fast={fast}")
    w = make_config(cfg, DEV, shape=SMALL[cfg], with_dy=True)
    x, mask, mode, dt = w["x"], w["mask"], w["mode"], w["dtype"]
    y = fwd(x, mask, w["scale"], w["causal"])
    ref = oracle_fwd(x, mask, mode, w["scale"], w["causal"])
    compare(decoded(y), ref, dt, f"cfg{cfg} fwd", rowsum=True)
    dx = bwd(y, w["dy"], w["scale"], w["causal"])
    refb = oracle.backward(to_np(y), to_np(w["dy"]), dt, w["scale"])
    compare(decoded(dx), refb, dt, f"cfg{cfg} bwd")
    # the causal promise changes nothing when it holds
    if w["causal"]:
        dx0 = bwd(y, w["dy"], w["scale"], False)
        compare(decoded(dx0), refb, dt, f"cfg{cfg} bwd without the causal promise")


# -------------------------------------------------- workloads, full sizes

def _full_forward_check(cfg):
    c = CONFIGS[cfg]
    say(f"workload {cfg} full {c['shape']}")
    w = make_config(cfg, DEV)
    x, mask, mode, dt = w["x"], w["mask"], w["mode"], w["dtype"]
    B, H, Sq, Sk = x.shape
    y = fwd(x, mask, w["scale"], w["causal"])
    rows = sample_rows(B * H * Sq, Sq, k=256, seed=cfg)
    xr = gather_rows(x, rows)
    mr = gather_mask_rows(mask, mode, x.shape, rows)
    yr = oracle.decode(gather_rows(y, rows), dt)
    for i, r in enumerate(rows):
        ref = oracle.forward_row(xr[i], dt, None if mr is None else mr[i], w["scale"],
                                 w["causal"], r % Sq)
        compare(yr[i], ref, dt, f"cfg{cfg} row {r}", rowsum=True)
    # every row: masked / causal-future keys exactly 0, row sums near 1. For
    # fp16/bf16 the bound follows from 2 ulp per element: sum_k 2 ulp(y_k) <=
    # 2^-(p-2) * sum_k y_k plus 2 subnormal ulps per element.
    p, emin = {"f32": (24, -126), "f16": (11, -14), "bf16": (8, -126)}[dt]
    tol = 1e-5 if dt == "f32" else 2.0 ** -(p - 2) + Sk * 2.0 ** (emin - p + 2)
    for b in range(B):
        yb = y[b]
        if w["causal"]:
            fut = torch.triu(torch.ones(Sq, Sk, dtype=torch.bool, device=DEV), diagonal=1)
            assert not ((yb != 0) & fut).any(), f"cfg{cfg} b={b}: causal-future key not 0"
        if mask is not None:
            mb = {"sq_sk": mask, "b_sq_sk": mask[b], "b_1_sk": mask[b], "full": mask[b]}[mode]
            assert not ((yb != 0) & torch.isinf(mb)).any(), f"cfg{cfg} b={b}: masked key not 0"
        s = yb.double().sum(-1)
        assert (s - 1).abs().max().item() <= tol, f"cfg{cfg} b={b} row sum"
    return w, y, rows


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_workload_full_size(cfg):
    w, y, rows = _full_forward_check(cfg)
    if CONFIGS[cfg]["backward"]:
        dt = w["dtype"]
        say(f"workload {cfg} full backward")
        dx = bwd(y, w["dy"], w["scale"], w["causal"])
        yr, dyr = gather_rows(y, rows), gather_rows(w["dy"], rows)
        dxr = oracle.decode(gather_rows(dx, rows), dt)
        for i, r in enumerate(rows):
            ref = oracle.backward_row(yr[i], dyr[i], dt, w["scale"])
            compare(dxr[i], ref, dt, f"cfg{cfg} bwd row {r}")
        # sum_k dx_k ~ 0 on every row (sum_k y_k ~ 1)
        s = dx.double().sum(-1).abs().max().item()
        assert s < 1e-2, s
        del dx
    del w, y
    torch.cuda.empty_cache()


# ------------------------------------------- strides, alignment, in place

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "f64"])
@pytest.mark.parametrize("Sk,pad,xoff,yoff,moff", [
    (1000, 0, 1, 1, 0),    # rows start mid-line, x and y alike
    (1000, 0, 1, 0, 0),    # x and y with different offsets -> element stores
    (1001, 0, 0, 0, 0),    # odd length: rows alternate alignment
    (1001, 7, 0, 0, 3),    # padded strides with a scalar tail; mask offset
    (256, 8, 0, 0, 1),     # aligned rows, misaligned mask rows
    (77, 3, 2, 5, 1),
])
def test_strided_and_misaligned(dtype, Sk, pad, xoff, yoff, moff):
    say(f"strided dtype={dtype} Sk={Sk} pad={pad} xoff={xoff} yoff={yoff} moff={moff}")
    B, H, Sq = 2, 3, 4
    td = TORCH_DTYPE[dtype]
    n = B * H * Sq * (Sk + pad)
    xs = draw_x((xoff + n,), dtype, ("normal", 3.0), Sk + pad, DEV)
    x = xs[xoff:].view(B, H, Sq, Sk + pad)[..., :Sk]
    ys = torch.full((yoff + n,), 7.0, dtype=td, device=DEV)
    y = ys[yoff:].view(B, H, Sq, Sk + pad)[..., :Sk]
    ms = draw_mask((1, 1, 1, moff + B * Sq * Sk), "full", dtype, ("bernoulli_neginf", 0.2), 5,
                   DEV).reshape(-1)
    mask = ms[moff:].view(B, Sq, Sk)
    fwd(x, mask, 0.5, True, y=y)
    ref = oracle_fwd(x.contiguous(), mask, "b_sq_sk", 0.5, True)
    compare(decoded(y), ref, dtype, "strided fwd", rowsum=True)
    if pad:  # the padding between rows is untouched
        gaps = ys[yoff:].view(B, H, Sq, Sk + pad)[..., Sk:]
        assert (gaps == 7.0).all()
    # backward with the same strided layout
    dys = draw_x((xoff + n,), dtype, ("normal", 1.0), 99, DEV)
    dy = dys[xoff:].view(B, H, Sq, Sk + pad)[..., :Sk]
    dxs = torch.zeros((yoff + n,), dtype=td, device=DEV)
    dx = dxs[yoff:].view(B, H, Sq, Sk + pad)[..., :Sk]
    bwd(y, dy, 0.5, True, dx=dx)
    refb = oracle.backward(to_np(y), to_np(dy), dtype, 0.5)
    compare(decoded(dx), refb, dtype, "strided bwd")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "f64"])
@pytest.mark.parametrize("Sk,pad,xoff,yoff,moff", [
    (1000, 0, 1, 1, 0),    # contiguous rows mid-line: NaN before the first, after the last
    (1000, 0, 1, 0, 0),    # y at another offset
    (1001, 7, 0, 0, 3),    # NaN in every row's padding, mask at an odd offset
    (77, 3, 2, 5, 1),
    (5, 11, 3, 1, 2),      # rows shorter than one vector
])
def test_nan_around_rows_is_not_read_into_results(dtype, Sk, pad, xoff, yoff, moff):
    """Partial 16-byte vectors at a row's ends are loaded as whole aligned
    lines; the elements of those lines outside the row (other tensors'
    bytes, padding) must not reach any result even when they are NaN."""
    say(f"nan-around dtype={dtype} Sk={Sk} pad={pad} xoff={xoff} yoff={yoff} moff={moff}")
    B, H, Sq = 2, 3, 4
    td = TORCH_DTYPE[dtype]
    nan = float("nan")
    n, tail = B * H * Sq * (Sk + pad), 16

    def framed(off, body):  # body (B,H,Sq,Sk) at element off of a NaN buffer, NaN padding
        buf = torch.full((off + n + tail,), nan, dtype=td, device=DEV)
        rows = buf[off:off + n].view(B, H, Sq, Sk + pad)
        if body is not None:
            rows[..., :Sk] = body
        return buf, rows[..., :Sk]

    _, x = framed(xoff, draw_x((B, H, Sq, Sk), dtype, ("normal", 3.0), Sk + 11, DEV))
    ms = torch.full((moff + B * Sq * Sk + tail,), nan, dtype=td, device=DEV)
    ms[moff:moff + B * Sq * Sk] = draw_mask((B, 1, Sq, Sk), "b_sq_sk", dtype,
                                            ("bernoulli_neginf", 0.2), 5, DEV).reshape(-1)
    mask = ms[moff:moff + B * Sq * Sk].view(B, Sq, Sk)
    ys, y = framed(yoff, None)
    fwd(x, mask, 0.5, True, y=y)
    ref = oracle_fwd(x.contiguous(), mask, "b_sq_sk", 0.5, True)
    compare(decoded(y), ref, dtype, "nan-around fwd", rowsum=True)
    _, dy = framed(xoff, draw_x((B, H, Sq, Sk), dtype, ("normal", 1.0), Sk + 12, DEV))
    dxs, dx = framed(yoff, None)
    bwd(y, dy, 0.5, True, dx=dx)
    refb = oracle.backward(to_np(y), to_np(dy), dtype, 0.5)
    compare(decoded(dx), refb, dtype, "nan-around bwd")
    # Nothing outside the rows was written: every byte there is still NaN.
    for buf, rows in ((ys, y), (dxs, dx)):
        inside = torch.zeros(buf.shape, dtype=torch.bool, device=DEV)
        off = rows.storage_offset()
        inside[off:off + n].view(B, H, Sq, Sk + pad)[..., :Sk] = True
        assert torch.isnan(buf[~inside]).all()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_permuted_strides_and_in_place(dtype):
    say(f"permuted/in-place dtype={dtype}")
    base = draw_x((2, 5, 3, 512), dtype, ("normal", 2.0), 3, DEV)  # [B, Sq, H, Sk] storage
    x = base.permute(0, 2, 1, 3)                                   # [B, H, Sq, Sk] view
    ref = oracle_fwd(x.contiguous(), None, "none", 0.7, False)
    y = fwd(x, None, 0.7, False)
    compare(decoded(y), ref, dtype, "permuted")
    xi = x.clone()
    fwd(xi, None, 0.7, False, y=xi)                                # in place
    assert torch.equal(xi, y)
    dy = draw_x(tuple(y.shape), dtype, ("normal", 1.0), 4, DEV)
    refb = oracle.backward(to_np(y), to_np(dy), dtype, 0.7)
    g = dy.clone()
    bwd(y, g, 0.7, False, dx=g)                                    # dx == dy in place
    compare(decoded(g), refb, dtype, "in-place bwd")


# ------------------------------------------------------ forced kernel shapes

@pytest.mark.parametrize("aligned", [False, True])
@pytest.mark.parametrize("tpr", [4, 8, 16, 32, 64, 128, 256, 512, 1024])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_every_lanes_per_row(tpr, dtype, aligned, monkeypatch):
    """Each row width (rows per wave, one wave, 2..16 waves per row) on a row
    length it can hold, against the oracle: an odd length (general kernels) and
    a whole number of 16-byte vectors (persistent aligned-row kernels)."""
    E = 4 if dtype == "f32" else 8
    Sk = min(4 * tpr * E - E + 1, 3 * tpr * E + 5)
    if aligned:
        Sk = 3 * tpr * E + E
    say(f"forced TPR={tpr} dtype={dtype} Sk={Sk}")
    monkeypatch.setenv("SMS_FORCE_TPR", str(tpr))
    shape = (1, 3, 5, Sk)
    x = draw_x(shape, dtype, ("normal", 4.0), tpr, DEV)
    mask = draw_mask(shape, "b_sq_sk", dtype, ("bernoulli_neginf", 0.3), tpr + 1, DEV)
    for causal in (False, True):
        y = fwd(x, mask, 0.25, causal)
        compare(decoded(y), oracle_fwd(x, mask, "b_sq_sk", 0.25, causal), dtype,
                f"TPR={tpr} causal={causal}", rowsum=True)
    dy = draw_x(shape, dtype, ("normal", 1.0), tpr + 2, DEV)
    dx = bwd(y, dy, 0.25, True)
    compare(decoded(dx), oracle.backward(to_np(y), to_np(dy), dtype, 0.25), dtype,
            f"TPR={tpr} bwd")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("tpr,nv", [(128, 1), (256, 1), (512, 1), (128, 2), (256, 2)])
def test_head_groups(dtype, tpr, nv, monkeypatch):
    """The forward over head groups (one workgroup takes query q of G heads
    that share a mask row) against the oracle and bit for bit against one row
    per workgroup: every mask shape and kind, both causal rules, H = 4 (groups
    of 2 and 4) and H = 3 (no group divides it). Mask shapes that vary by
    head, and widths the groups are not built for, fall back to one row."""
    E = 4 if dtype == "f32" else 8
    Sk = (tpr * (nv - 1) + tpr // 2 + 3) * E  # nv vectors per lane at tpr lanes
    say(f"head groups dtype={dtype} TPR={tpr} NV={nv} Sk={Sk}")
    monkeypatch.setenv("SMS_FORCE_TPR", str(tpr))
    for H in (4, 3):
        shape = (2, H, 3, Sk)
        for mode, kind in MASK_CASES:
            for causal in CAUSALS:
                seed = zlib.crc32(f"hg/{dtype}/{tpr}/{nv}/{H}/{mode}/{kind}/{causal}".encode()) % 10000
                x = draw_x(shape, dtype, ("normal", 3.0), seed, DEV)
                mask = make_mask(shape, mode, kind, dtype, seed + 1)
                monkeypatch.setenv("SMS_HEADS", "1")
                y1 = fwd(x, mask, 0.3, causal)
                compare(decoded(y1), oracle_fwd(x, mask, mode, 0.3, causal, kind), dtype,
                        f"H={H} {mode}/{kind} causal={causal}", rowsum=True)
                for g in ("2", "4", "0"):
                    monkeypatch.setenv("SMS_HEADS", g)
                    assert torch.equal(fwd(x, mask, 0.3, causal), y1), \
                        f"G={g} H={H} {mode}/{kind} causal={causal}"


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("tpr,nv", [(128, 1), (256, 1), (512, 1), (1024, 1), (256, 2), (128, 4)])
def test_early_exit_of_future_wavefronts(dtype, tpr, nv, monkeypatch):
    """Aligned rows whose causal bound (both alignments, more queries than
    keys so that some rows see no key) or key length leaves whole wavefronts
    of a row with no key to read: those wavefronts end early, forward and
    backward, and the results are the oracle's and bit for bit those of the
    kernels without the early exit."""
    E = 4 if dtype == "f32" else 8
    Sk = (tpr * (nv - 1) + tpr // 2 + 5) * E  # nv vectors per lane at tpr lanes
    say(f"early exit dtype={dtype} TPR={tpr} NV={nv} Sk={Sk}")
    monkeypatch.setenv("SMS_FORCE_TPR", str(tpr))
    for Sq, causal, kind in ((Sk // 8 + 3, True, "none"), (Sk // 8 + 3, "bottom_right", "none"),
                             (Sk + 40, "bottom_right", "none"), (5, False, "lengths"),
                             (5, True, "lengths")):
        shape = (1, 1, Sq, Sk) if Sq > Sk else (2, 2, Sq, Sk)
        seed = zlib.crc32(f"ee/{dtype}/{tpr}/{nv}/{Sq}/{causal}/{kind}".encode()) % 10000
        x = draw_x(shape, dtype, ("normal", 3.0), seed, DEV)
        mask = (draw_lengths(shape[0], 0, Sk, seed + 1, DEV) if kind == "lengths" else None)
        dy = draw_x(shape, dtype, ("normal", 1.0), seed + 2, DEV)
        outs = {}
        for early in ("0", "1"):
            monkeypatch.setenv("SMS_EARLY", early)
            y = fwd(x, mask, 0.3, causal)
            outs[early] = (y, bwd(y, dy, 0.3, causal))
        what = f"Sq={Sq} causal={causal} {kind}"
        assert torch.equal(outs["0"][0], outs["1"][0]), what + " forward"
        assert torch.equal(outs["0"][1], outs["1"][1]), what + " backward"
        y, dx = outs["1"]
        compare(decoded(y), oracle_fwd(x, mask, "key_lengths" if kind == "lengths" else "none",
                                       0.3, causal, "lengths" if kind == "lengths" else "additive"),
                dtype, what, rowsum=True)
        compare(decoded(dx), oracle.backward(to_np(y), to_np(dy), dtype, 0.3), dtype,
                what + " bwd")


def test_forced_width_too_small_is_an_error(monkeypatch):
    monkeypatch.setenv("SMS_FORCE_TPR", "4")
    x = torch.zeros(1, 1, 2, 4096, device=DEV)
    with pytest.raises(SmsError, match="SHAPE"):
        sms_forward(x, None, torch.empty_like(x))


@pytest.mark.parametrize("shape", [(2, 3, 5, 1024), (3, 1, 1, 2048), (1, 4, 1, 512),
                                   (2, 1, 7, 256), (1, 1, 1, 4096)])
def test_padded_and_permuted_rows_agree(shape):
    """Contiguous, padded-row and [H,B]-ordered operands give identical bits,
    including shapes with size-1 axes (row coordinates from the fast divisions)."""
    B, H, Sq, Sk = shape
    x = draw_x(shape, "f16", ("normal", 4.0), 7, DEV)
    dy = draw_dy(shape, "f16", 8, DEV)
    y0 = fwd(x, None, 0.25, True)
    dx0 = bwd(y0, dy, 0.25, True)
    # padded rows (row stride Sk + 8, still 16-byte aligned) and a [H,B] storage order
    for make in (lambda t: torch.zeros(B, H, Sq, Sk + 8, dtype=t.dtype, device=DEV)[..., :Sk],
                 lambda t: torch.zeros(H, B, Sq, Sk, dtype=t.dtype, device=DEV).transpose(0, 1)):
        xs, dys = make(x), make(dy)
        xs.copy_(x)
        dys.copy_(dy)
        ys, dxs = make(x), make(x)
        sms_forward(xs, None, ys, 0.25, True)
        sms_backward(ys, dys, dxs, 0.25, True)
        assert torch.equal(ys, y0) and torch.equal(dxs, dx0)
    compare(decoded(y0), oracle_fwd(x, None, "none", 0.25, True), "f16", f"flat {shape}")


# ------------------------------------------------------------------ edges

def test_edge_rows():
    say("edge rows")
    # fully masked rows (by mask, and by causal + mask at key 0 for q = 0) -> zeros
    x = draw_x((1, 2, 4, 300), "f16", ("normal", 1.0), 0, DEV)
    mask = torch.zeros(4, 300, dtype=torch.float16, device=DEV)
    mask[1] = -math.inf
    mask[0, 0] = -math.inf
    y = fwd(x, mask, 1.0, True)
    assert (y[:, :, 0] == 0).all() and (y[:, :, 1] == 0).all()
    assert not torch.isnan(y).any()
    compare(decoded(y), oracle_fwd(x, mask, "sq_sk", 1.0, True), "f16", "fully masked")
    dy = torch.randn_like(y)
    dx = bwd(y, dy, 1.0, True)
    assert (dx[:, :, :2] == 0).all()
    # Sk = 1: probability exactly 1 (or 0 when masked)
    x1 = torch.randn(2, 2, 3, 1, device=DEV)
    assert (fwd(x1) == 1).all()
    # large equal-ish scores; an fp16 probability that is a subnormal
    xs = torch.tensor([[[[1000.0, 1001.0]]]], device=DEV)
    compare(decoded(fwd(xs)), [[[[1 / (1 + math.e), math.e / (1 + math.e)]]]], "f32", "[1000,1001]")
    xh = torch.tensor([[[[0.0, -12.0]]]], device=DEV, dtype=torch.float16)
    yh = fwd(xh)
    assert yh[0, 0, 0, 1].item() == 103 * 2.0 ** -24  # RNE of 6.1442e-06, kept subnormal
    # scale 0 -> uniform over unmasked keys; negative scale flips the order
    xu = draw_x((1, 1, 2, 100), "f32", ("normal", 5.0), 3, DEV)
    yu = fwd(xu, None, 0.0)
    assert torch.allclose(yu, torch.full_like(yu, 0.01), atol=1e-9, rtol=0)
    compare(decoded(fwd(xu, None, -0.5)), oracle_fwd(xu, None, "none", -0.5, False), "f32",
            "negative scale")


def test_zero_size_and_errors():
    x = torch.empty(2, 0, 3, 8, device=DEV)
    fwd(x)
    bwd(x, x)
    x = torch.randn(1, 1, 2, 8, device=DEV)
    with pytest.raises(TypeError):
        sms_forward(x, torch.zeros(2, 8, dtype=torch.float16, device=DEV), torch.empty_like(x))
    with pytest.raises(ValueError):
        sms_forward(x, None, torch.empty(1, 1, 2, 9, device=DEV))
    with pytest.raises(SmsError, match="SHAPE"):
        big = torch.empty(1, 1, 1, sms_max_sk(torch.float32) + 1, device=DEV)
        sms_forward(big, None, big)


def test_deterministic():
    w = make_config(5, DEV, shape=(2, 4, 1000, 1000), with_dy=True)
    y1 = fwd(w["x"], w["mask"], w["scale"], False)
    y2 = fwd(w["x"], w["mask"], w["scale"], False)
    assert torch.equal(y1, y2)
    d1 = bwd(y1, w["dy"], w["scale"])
    d2 = bwd(y1, w["dy"], w["scale"])
    assert torch.equal(d1, d2)


# --------------------------------------------------------------- autograd

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "f64"])
def test_autograd_and_streams(dtype):
    say(f"autograd dtype={dtype}")
    shape = (2, 3, 17, 130)
    x = draw_x(shape, dtype, ("normal", 3.0), 1, DEV).requires_grad_(True)
    mask = draw_mask(shape, "b_sq_sk", dtype, ("bernoulli_neginf", 0.2), 2, DEV)
    dy = draw_x(shape, dtype, ("normal", 1.0), 3, DEV)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        y = scaled_mask_softmax(x, mask, 0.35, True)
        (y * dy).sum().backward() if dtype in ("f32", "f64") else y.backward(dy)
    torch.cuda.synchronize()
    compare(decoded(y.detach()), oracle_fwd(x.detach(), mask, "b_sq_sk", 0.35, True), dtype,
            "autograd fwd")
    refb = oracle.backward(to_np(y.detach()), to_np(dy), dtype, 0.35)
    compare(decoded(x.grad), refb, dtype, "autograd bwd")
    # non-contiguous upstream gradient
    x.grad = None
    y = scaled_mask_softmax(x, mask, 0.35, True)
    g = torch.cat([dy, dy], dim=-1)[..., ::2]
    y.backward(g)
    torch.cuda.synchronize()
    compare(decoded(x.grad), oracle.backward(to_np(y.detach()), to_np(g.contiguous()), dtype,
                                             0.35), dtype, "autograd strided dy")


# ------------------------------------------------------------ HIP graphs

@pytest.mark.parametrize("dtype,shape,mode,causal", [
    ("f16", (2, 4, 64, 2048), "b_sq_sk", True),   # aligned-row kernels, 128 lanes
    ("f32", (3, 2, 40, 1001), "sq_sk", False),    # general kernels (unaligned rows)
    ("bf16", (1, 2, 2, 40000), "none", True),     # streaming kernels
])
def test_hip_graph_capture_and_replay(dtype, shape, mode, causal):
    """Forward + backward captured once into a HIP graph (torch.cuda.CUDAGraph)
    and replayed on new inputs copied into the static buffers, with eager work
    and synchronisation between replays: every replay equals the eager call bit
    for bit, and the oracle."""
    say(f"graph dtype={dtype} shape={shape} mode={mode} causal={causal}")
    kind = ("bernoulli_neginf", 0.2)
    x = draw_x(shape, dtype, ("normal", 3.0), 11, DEV)
    mask = draw_mask(shape, mode, dtype, kind, 12, DEV) if mode != "none" else None
    dy = draw_dy(shape, dtype, 13, DEV)
    y, dx = torch.empty_like(x), torch.empty_like(x)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream
        sms_forward(x, mask, y, 0.3, causal)
        sms_backward(y, dy, dx, 0.3, causal)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sms_forward(x, mask, y, 0.3, causal)
        sms_backward(y, dy, dx, 0.3, causal)
    for rep in range(3):
        xn = draw_x(shape, dtype, ("normal", 3.0), 100 + rep, DEV)
        dyn = draw_dy(shape, dtype, 200 + rep, DEV)
        x.copy_(xn)
        dy.copy_(dyn)
        g.replay()
        torch.cuda.synchronize()
        ye = fwd(xn, mask, 0.3, causal)  # eager, on fresh buffers
        dxe = bwd(ye, dyn, 0.3, causal)
        assert torch.equal(y, ye), f"replay {rep}: y differs from the eager call"
        assert torch.equal(dx, dxe), f"replay {rep}: dx differs from the eager call"
        compare(decoded(y), oracle_fwd(xn, mask, mode, 0.3, causal), dtype, f"graph fwd {rep}",
                rowsum=True)
        compare(decoded(dx), oracle.backward(to_np(y), to_np(dyn), dtype, 0.3), dtype,
                f"graph bwd {rep}")
    del g


# ------------------------------------------------- long rows (streaming)

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("Sk", [1, 7, 64, 77, 1000, 1001, 4096, 5000])
def test_streaming_kernels_on_short_rows(dtype, Sk, monkeypatch):
    """The two-pass streaming kernels, forced onto short rows: every mask mode,
    causal or not, aligned or not, forward and backward, against the oracle."""
    monkeypatch.setenv("SMS_FORCE_STREAM", "1")
    say(f"stream forced dtype={dtype} Sk={Sk}")
    for mode, kind in MASK_CASES:
        for causal in CAUSALS:
            shape = (2, 2, 3, Sk)
            seed = zlib.crc32(f"s/{dtype}/{Sk}/{mode}/{kind}/{causal}".encode()) % 10000
            x = draw_x(shape, dtype, ("normal", 3.0), seed, DEV)
            mask = make_mask(shape, mode, kind, dtype, seed + 1)
            check_fwd_bwd(x, mask, mode, kind, 0.3, causal,
                          f"stream {dtype} Sk={Sk} {mode}/{kind} causal={causal}",
                          dy_seed=seed + 2)


@pytest.mark.parametrize("dtype,Sk,mode,kind", [
    ("f32", 16385, "b_1_sk", "additive"),   # one past the register-resident fp32 reach
    ("f32", 262144, "none", "none"),        # 1 MB rows
    ("f32", 20000, "sq_sk", "bool"),
    ("f16", 32769, "sq_sk", "additive"),    # one past the fp16 reach
    ("f16", 40000, "b_sq_sk", "additive"),
    ("bf16", 100003, "full", "additive"),   # odd length: unaligned rows, element head/tail
    ("bf16", 50001, "key_lengths", "lengths"),
    ("f16", 140001, "b_sq_sk", "bool"),       # rows of >= 16384 vectors: split when auto
    ("bf16", 262147, "key_lengths", "lengths"),
    ("f16", 32776, "b_sq_sk", "additive"),   # 4097 vectors: the one-pass long-row backward
    ("f16", 65536, "sq_sk", "bool"),         # 8192 vectors: its longest row
    ("f32", 32768, "b_1_sk", "additive"),   # 8192 vectors of fp32
    ("f32", 65537, "full", "additive"),
    ("f64", 70001, "sq_sk", "additive"),     # fp64: two-pass kernels at every length
    ("f64", 40000, "b_1_sk", "bool"),
])
@pytest.mark.parametrize("split", ["auto", "off"])
def test_long_rows(dtype, Sk, mode, kind, split, monkeypatch):
    """Rows beyond one workgroup's registers: eight of them are split across
    workgroups (through a workspace) or, with splitting off, take the streaming
    kernels; every row against the oracle, every causal rule, both alignments."""
    if split == "off":
        monkeypatch.setenv("SMS_SPLIT", "0")
    say(f"long rows dtype={dtype} Sk={Sk} mode={mode} kind={kind} split={split}")
    shape = (1, 2, 4, Sk)
    x = draw_x(shape, dtype, ("normal", 4.0), Sk, DEV)
    if kind == "lengths":
        mask = torch.tensor([Sk // 3], dtype=torch.int32, device=DEV)
    else:
        mask = make_mask(shape, mode, kind, dtype, Sk + 1)
    for causal in CAUSALS:
        check_fwd_bwd(x, mask, mode, kind, 0.25, causal, f"long causal={causal}",
                      dy_seed=Sk + 2)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("Sk", [7, 77, 1001, 4097])
@pytest.mark.parametrize("chunks", [2, 7])
def test_split_forced_on_short_rows(dtype, Sk, chunks, monkeypatch):
    """The split kernels forced onto short rows with chunk boundaries at odd
    vectors (including chunks wholly past a causal bound or beyond the row):
    every mask shape and kind, every causal rule, against the oracle."""
    monkeypatch.setenv("SMS_FORCE_SPLIT", str(chunks))
    say(f"split forced dtype={dtype} Sk={Sk} chunks={chunks}")
    for mode, kind in MASK_CASES:
        for causal in CAUSALS:
            shape = (2, 2, 3, Sk)
            seed = zlib.crc32(f"p/{dtype}/{Sk}/{chunks}/{mode}/{kind}/{causal}".encode()) % 10000
            x = draw_x(shape, dtype, ("normal", 3.0), seed, DEV)
            mask = make_mask(shape, mode, kind, dtype, seed + 1)
            check_fwd_bwd(x, mask, mode, kind, 0.3, causal,
                          f"split {dtype} Sk={Sk} C={chunks} {mode}/{kind} causal={causal}",
                          dy_seed=seed + 2)


@pytest.mark.parametrize("dtype,Sk", [("f16", 200003), ("f32", 65536)])
def test_split_rows_in_place_deterministic_workspace(dtype, Sk):
    """Split rows: in place (y = x, dx = dy) equals out of place, two runs are
    bitwise equal, a caller workspace equals the default one, a short workspace
    is an error, and the result matches the streaming kernels within tolerance."""
    say(f"split properties dtype={dtype} Sk={Sk}")
    shape = (1, 1, 3, Sk)
    td = TORCH_DTYPE[dtype]
    assert sms_workspace_bytes(td, shape) > 0
    x = draw_x(shape, dtype, ("normal", 4.0), 21, DEV)
    dy = draw_dy(shape, dtype, 22, DEV)
    y = fwd(x, None, 0.5, "bottom_right")
    dx = bwd(y, dy, 0.5, "bottom_right")
    assert torch.equal(fwd(x, None, 0.5, "bottom_right"), y)
    assert torch.equal(bwd(y, dy, 0.5, "bottom_right"), dx)
    xi = x.clone()
    sms_forward(xi, None, xi, 0.5, "bottom_right")
    dyi = dy.clone()
    sms_backward(y, dyi, dyi, 0.5, "bottom_right")
    torch.cuda.synchronize()
    assert torch.equal(xi, y) and torch.equal(dyi, dx)
    ws = torch.empty(sms_workspace_bytes(td, shape), dtype=torch.uint8, device=DEV)
    yw = torch.empty_like(x)
    sms_forward(x, None, yw, 0.5, "bottom_right", workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(yw, y)
    with pytest.raises(SmsError, match="WORKSPACE"):
        sms_forward(x, None, yw, 0.5, "bottom_right", workspace=ws[:8])
    compare(decoded(y), oracle_fwd(x, None, "none", 0.5, "bottom_right"), dtype, "split fwd",
            rowsum=True)
    compare(decoded(dx), oracle.backward(to_np(y), to_np(dy), dtype, 0.5), dtype, "split bwd")


@pytest.mark.parametrize("moff", [1, 3, 5])
@pytest.mark.parametrize("dtype,Sk", [("f16", 1000), ("f32", 256), ("bf16", 77)])
def test_bool_mask_at_odd_offsets(dtype, Sk, moff):
    """Boolean mask rows that do not sit on a vector boundary: byte-wise mask
    loads in the general kernels, against the oracle."""
    say(f"bool mask offset dtype={dtype} Sk={Sk} moff={moff}")
    B, H, Sq = 2, 2, 5
    shape = (B, H, Sq, Sk)
    x = draw_x(shape, dtype, ("normal", 3.0), moff, DEV)
    full = draw_mask((1, 1, 1, moff + B * Sq * Sk), "full", dtype, ("bool", 0.3), moff + 1,
                     DEV).reshape(-1)
    mask = full[moff:].view(B, Sq, Sk)
    for causal in CAUSALS:
        check_fwd_bwd(x, mask, "b_sq_sk", "bool", 0.7, causal, f"bool moff={moff} {causal}")


def test_long_causal_square():
    """Causal with Sq = Sk = 40000 (fp16): query positions across the whole
    streamed row; sampled rows against the oracle, zeros after the diagonal."""
    Sk = 40000
    say(f"long causal square Sk={Sk}")
    shape = (1, 1, Sk, Sk)
    x = draw_x(shape, "f16", ("normal", 8.0), 5, DEV)
    y = fwd(x, None, 1 / math.sqrt(128), True)
    rows = sample_rows(Sk, Sk, k=48, seed=5) + [Sk - 1, 32767, 32768]
    xr = gather_rows(x, rows)
    yr = oracle.decode(gather_rows(y, rows), "f16")
    for i, r in enumerate(rows):
        ref = oracle.forward_row(xr[i], "f16", None, 1 / math.sqrt(128), True, r % Sk)
        compare(yr[i], ref, "f16", f"row {r}")
    for q0 in range(0, Sk, 8192):
        blk = y[0, 0, q0:q0 + 8192]
        k = torch.arange(Sk, device=DEV)
        fut = k.view(1, -1) > torch.arange(q0, q0 + blk.shape[0], device=DEV).view(-1, 1)
        assert not ((blk != 0) & fut).any()
    del x, y
    torch.cuda.empty_cache()
