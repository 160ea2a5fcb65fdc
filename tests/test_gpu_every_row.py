"""Every row of every workload at full size against the float64 oracle.

The GPU runs the forward (and the backward on the GPU's own y with the
workload's dy) once; the typed inputs and outputs are copied to the host and
split into blocks of whole (b, h) planes, which worker processes check with the
oracle element by element (tests/every_row.py). Up to 16 worker processes,
started fresh ("spawn"): they import numpy and the oracle only and never touch
the GPU.
"""

import concurrent.futures as cf
import multiprocessing as mp
import os
import sys

import pytest
import torch

from attention_softmax_amd import sms_backward, sms_forward
from attention_softmax_amd.workloads import CONFIGS, make_config
from tests import every_row
from tests.parity import mask_4d, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BLOCK_ELEMS = 1 << 22  # elements per task (whole planes, at least one)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _run_tasks(pool, limit, tasks, label):
    """Submit (fn, args) tasks, at most ``limit`` in flight; merge the stats."""
    stats, pending, done, n = {}, set(), 0, len(tasks)
    it = iter(tasks)
    step = max(1, n // 4)
    while True:
        while len(pending) < limit:
            t = next(it, None)
            if t is None:
                break
            pending.add(pool.submit(*t))
        if not pending:
            break
        fin, pending = cf.wait(pending, return_when=cf.FIRST_COMPLETED)
        for f in fin:
            every_row._merge(stats, f.result())  # re-raises a worker's AssertionError
            done += 1
            if done % step == 0 or done == n:
                say(f"  {label}: {done}/{n} blocks, worst so far {stats}")
    return stats


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_every_row_of_workload(cfg):
    c = CONFIGS[cfg]
    say(f"workload {cfg} every row: {c['name']}")
    w = make_config(cfg, DEV, with_dy=True)
    x, mask, mode, dt = w["x"], w["mask"], w["mode"], w["dtype"]
    B, H, Sq, Sk = x.shape
    y = torch.empty_like(x)
    sms_forward(x, mask, y, w["scale"], w["causal"])
    dx = torch.empty_like(x)
    sms_backward(y, w["dy"], dx, w["scale"], w["causal"])
    torch.cuda.synchronize()
    P = B * H
    x_np = to_np(x).reshape(P, 1, Sq, Sk)
    del x
    y_np = to_np(y).reshape(P, 1, Sq, Sk)
    del y
    dy_np = to_np(w["dy"]).reshape(P, 1, Sq, Sk)
    dx_np = to_np(dx).reshape(P, 1, Sq, Sk)
    del dx
    m4 = mask_4d(mask, mode)
    del w, mask
    torch.cuda.empty_cache()

    k = max(1, BLOCK_ELEMS // (Sq * Sk))
    blocks = [(p0, min(P, p0 + k)) for p0 in range(0, P, k)]
    fwd_tasks = [(every_row.forward_block, dt, x_np[p0:p1],
                  every_row.mask_planes(m4, range(p0, p1), H), y_np[p0:p1], c["scale"],
                  c["causal"], "additive", f"cfg{cfg} fwd planes {p0}..{p1 - 1}")
                 for p0, p1 in blocks]
    bwd_tasks = [(every_row.backward_block, dt, y_np[p0:p1], dy_np[p0:p1], dx_np[p0:p1],
                  c["scale"], f"cfg{cfg} bwd planes {p0}..{p1 - 1}") for p0, p1 in blocks]
    workers = max(1, min(16, os.cpu_count() or 1, len(blocks)))
    with cf.ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn")) as pool:
        sf = _run_tasks(pool, 2 * workers, fwd_tasks, f"cfg{cfg} forward")
        sb = _run_tasks(pool, 2 * workers, bwd_tasks, f"cfg{cfg} backward")
    say(f"workload {cfg}: {B * H * Sq} rows; forward {sf}; backward {sb}")
