"""Throughput of the fused scaled-masked softmax, forward + backward, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4]

A step is one forward (y = softmax(x*scale + mask), causal rule if the workload
has it) and one backward (dx = scale*y*(dy - sum dy*y)) over the whole synthetic
batch, through the C ABI, with every input already in HBM. The default workload
is the largest: fp16 x[4,32,4096,4096] = 8*N(0,1), scale 1/sqrt(128), additive
mask [4,4096,4096] with -inf at 10 % of the positions (the diagonal kept), the
causal rule; dy ~ N(0,1) fp16.

Before the W warm-up steps, the step runs untimed for a fixed wall time
(``--settle-seconds``) so that the GPU's clocks have left their idle state; the
JSON line states that time and the number of steps it took. The timed region is
exactly K steps.

value = algorithmic bytes of a step / time of a step (GB/s), where algorithmic
bytes count x and the mask once where the result depends on them, y and dy
where y can be nonzero, and every y and dx written. The same line carries the
per-kernel rate of the other workloads (fp32 [1,2,64,64], fp32 [8,32,1024,1024]
with key padding, fp16 [4,32,2048,2048] causal, bf16 [16,16,1000,1000] with a
[1000,1000] mask), each timed after its own settle phase, the float64
oracle timed on the host's cores over a sample of the headline workload's rows,
and two plain device copies of the forward's byte count: torch's and the
library's 16-byte copy kernel (copy_ceiling: what a kernel that reads and
writes those bytes once reaches with no arithmetic, and each kernel's rate as a
fraction of it).
One JSON line on stdout; diagnostics on stderr.

    python bench.py --op attention [--steps K] [--warmup W]

times the fused attention instead (O = softmax(Q K^T * scale) V and its
gradients, fp16 [4,32,4096,128] queries, keys, values and dO, causal): value =
the algorithmic flops of the forward's two products and the backward's five
(halved by the causal rule) / time of a forward + backward, in TFLOP/s against
the MI355X dense fp16 matrix peak. It is a diagnostic line for those kernels;
the default (softmax) line is the headline metric.
"""

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 / bf16 matrix, published
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
COPY_KERNEL = "__amd_rocclr_copyBuffer"  # torch's device copy, timed as the copy reference


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kept_keys(Sq, Sk, causal):
    """Keys per (b, h) plane the result depends on: all, or q+1 per row if causal."""
    if not causal:
        return Sq * Sk
    return sum(min(q + 1, Sk) for q in range(Sq)) if Sq <= 1 << 16 else None


def min_bytes(shape, dtype_bytes, mode, causal):
    """Algorithmic bytes of one forward and one backward launch."""
    B, H, Sq, Sk = shape
    full = B * H * Sq * Sk
    plane = kept_keys(Sq, Sk, causal)
    x_read = B * H * plane
    if mode == "none":
        m_read = 0
    elif mode == "b_1_sk":
        m_read = B * (min(Sk, Sq) if causal else Sk)
    elif mode == "sq_sk":
        m_read = plane
    elif mode == "b_sq_sk":
        m_read = B * plane
    else:
        m_read = B * H * plane
    fwd = (x_read + m_read + full) * dtype_bytes
    bwd = (2 * B * H * plane + full) * dtype_bytes
    return fwd, bwd


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    # From idle, MI355X runs the first launches of this size up to 15 % slow
    # while its clocks ramp: the settle phase runs the step past that, for a
    # fixed wall time, before the warm-up steps.
    ap.add_argument("--settle-seconds", type=float, default=2.0,
                    help="untimed wall time the step runs before --warmup (0 = none)")
    ap.add_argument("--workload", type=int, default=4, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--others", default="1,2,3,5",
                    help="workloads whose per-kernel rate the line also reports ('' = none)")
    ap.add_argument("--other-launches", type=int, default=20,
                    help="timed launches of each kernel of the other workloads")
    ap.add_argument("--op", default="softmax", choices=["softmax", "attention"],
                    help="softmax (the headline line) or the fused attention forward")
    ap.add_argument("--cpu-seconds", type=float, default=16.0,
                    help="CPU work (summed over workers) of the oracle CPU baseline sample "
                         "(0 = skip)")
    ap.add_argument("--cpu-workers", type=int, default=16,
                    help="most worker processes of the CPU baseline (one per core, at most "
                         "the host's CPU count)")
    ap.add_argument("--no-copy", action="store_true", help="skip the plain-copy reference")
    ap.add_argument("--no-torch", action="store_true",
                    help="skip the unfused PyTorch reference (context only)")
    ap.add_argument("--traffic", default=TRAFFIC_JSON,
                    help="HBM bytes per launch from rocprofv3 counters (see --ingest)")
    ap.add_argument("--ingest", default=None, metavar="DIR",
                    help="read rocprofv3 output under DIR (kt/, fetch/, write/) of a run of "
                         "this script, update --traffic and print a summary; no GPU work")
    return ap.parse_args()


def csrc_sha():
    """Hash of the sources the softmax kernels and their launches are built
    from (every file under csrc/ but the fused attention's own and the copy
    reference): counters taken on other sources are stale."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "attention_softmax_amd", "csrc")
    files = sorted(f for f in glob.glob(os.path.join(csrc, "*"))
                   if not os.path.basename(f).startswith(("attention", "copy_ref")))
    for f in files:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def _kernel_role(name):
    if "sms_fwd" in name:
        return "forward"
    if "sms_bwd" in name:
        return "backward"
    if COPY_KERNEL in name:
        return "copy"
    return None


def ingest(args):
    """Counters of one bench run -> HBM bytes per launch of each kernel.

    Reads rocprofv3 output under DIR: kt/ (kernel trace and stats), and one
    --pmc pass per subdirectory: dram/ (TCC_EA0_RDREQ_DRAM_32B_sum and
    TCC_EA0_WRREQ_WRITE_DRAM_32B_sum: requests from L2 to the memory
    controller in 32-byte units, a 64-byte request counted twice and a
    128-byte one four times), and, as cross-checks, fetch/ (FETCH_SIZE, KiB),
    write/ (WRITE_SIZE, KiB) and rdsize/ (TCC_EA0_RDREQ_{32B,64B,128B}_sum).
    The traffic of a launch is 32 * (RDREQ_DRAM_32B + WRREQ_WRITE_DRAM_32B); the
    plain copy kernel of known size in the same run shows what each counter
    reads for known bytes.
    """
    d = args.ingest
    stats = glob.glob(os.path.join(d, "kt", "*kernel_stats.csv"))
    trace_json = glob.glob(os.path.join(d, "kt_bench.json"))
    run = json.load(open(trace_json[0])) if trace_json else None
    avg = {}
    for row in csv.DictReader(open(stats[0])):
        role = _kernel_role(row["Name"])
        if role:
            avg[role] = (row["Name"], int(row["Calls"]), float(row["AverageNs"]) / 1e3)
    # The timed launches are the last `steps` of each kernel in the trace.
    timed = {}
    traces = glob.glob(os.path.join(d, "kt", "*kernel_trace.csv"))
    if traces and run:
        durs = {}
        for row in csv.DictReader(open(traces[0])):
            role = _kernel_role(row["Kernel_Name"])
            if role in ("forward", "backward"):
                durs.setdefault(role, []).append(
                    (int(row["Start_Timestamp"]), int(row["End_Timestamp"]) - int(row["Start_Timestamp"])))
        for role, v in durs.items():
            v.sort()
            last = [dt for _, dt in v[-run["steps"]:]]
            timed[role] = sum(last) / len(last) / 1e3

    def counter(sub, name, unit):
        """Median per dispatch of counter `name` (times `unit` bytes) by kernel role."""
        vals = {}
        for f in glob.glob(os.path.join(d, sub, "*counter_collection.csv")):
            for row in csv.DictReader(open(f)):
                if row["Counter_Name"] != name:
                    continue
                role = _kernel_role(row["Kernel_Name"])
                if role:
                    vals.setdefault(role, []).append(float(row["Counter_Value"]) * unit)
        return {k: statistics.median(v) for k, v in vals.items()}

    rd = counter("dram", "TCC_EA0_RDREQ_DRAM_32B_sum", 32.0)
    wr = counter("dram", "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum", 32.0)
    fetch = counter("fetch", "FETCH_SIZE", 1024.0)
    write = counter("write", "WRITE_SIZE", 1024.0)
    r32 = counter("rdsize", "TCC_EA0_RDREQ_32B_sum", 32.0)
    r64 = counter("rdsize", "TCC_EA0_RDREQ_64B_sum", 64.0)
    r128 = counter("rdsize", "TCC_EA0_RDREQ_128B_sum", 128.0)
    sized = {k: r32.get(k, 0.0) + r64.get(k, 0.0) + r128.get(k, 0.0) for k in r32}
    copy_bytes = run["copy_reference"]["bytes"] // 2 if run else None
    wl = run["config"]["workload"] if run else "?"
    key_wl = args.workload
    table = json.load(open(args.traffic)) if os.path.exists(args.traffic) else {}
    table.setdefault("workloads", {})
    sha = csrc_sha()

    def ratio(v, role="copy"):
        return v.get(role, 0.0) / copy_bytes if copy_bytes and v.get(role) else float("nan")

    lines = [f"workload {key_wl}: {wl}", "",
             f"Plain copy kernel `{COPY_KERNEL}`, {copy_bytes} B read and {copy_bytes} B "
             "written per launch; what each counter reads for it, over the true bytes:", "",
             "| counter | read | write |", "|---|---|---|",
             f"| TCC_EA0_RDREQ_DRAM_32B x 32 / TCC_EA0_WRREQ_WRITE_DRAM_32B x 32 | "
             f"{ratio(rd):.4f} | {ratio(wr):.4f} |",
             f"| TCC_EA0_RDREQ_{{32B,64B,128B}} x size | {ratio(sized):.4f} | - |",
             f"| FETCH_SIZE / WRITE_SIZE (KiB x 1024) | {ratio(fetch):.4f} | {ratio(write):.4f} |",
             "", "| kernel | calls | avg us, all calls (rocprofv3) | avg us, timed calls (rocprofv3) "
             "| avg us (HIP events) | algorithmic B | DRAM read B | DRAM write B | "
             "traffic / algorithmic | RDREQ by size B | FETCH_SIZE B | WRITE_SIZE B |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for role in ("forward", "backward"):
        if role not in avg:
            continue
        name, calls, us = avg[role]
        r_b, w_b = rd.get(role, 0.0), wr.get(role, 0.0)
        alg = run["kernels"][role]["bytes"] if run else None
        ev = run["kernels"][role]["avg_us"] if run else None
        t_us = timed.get(role)
        table["workloads"][f"{key_wl}_{role}"] = {
            "kernel": name, "dram_read_bytes": round(r_b), "dram_write_bytes": round(w_b),
            "traffic": round(r_b + w_b), "algorithmic_bytes": alg,
            "rocprof_avg_us": round(us, 2),
            "rocprof_timed_avg_us": round(t_us, 2) if t_us else None,
            "fetch_size_bytes": round(fetch.get(role, 0.0)),
            "write_size_bytes": round(write.get(role, 0.0)),
            "rdreq_sized_bytes": round(sized.get(role, 0.0)),
            "copy_read_ratio": ratio(rd), "copy_write_ratio": ratio(wr), "csrc_sha": sha}
        q = (r_b + w_b) / alg if alg else float("nan")
        t_txt = f"{t_us:.2f}" if t_us else "-"
        lines.append(f"| `{name}` | {calls} | {us:.2f} | {t_txt} | {ev} | {alg} | {r_b:.0f} | "
                     f"{w_b:.0f} | {q:.4f} | {sized.get(role, 0.0):.0f} | "
                     f"{fetch.get(role, 0.0):.0f} | {write.get(role, 0.0):.0f} |")
    os.makedirs(os.path.dirname(args.traffic), exist_ok=True)
    with open(args.traffic, "w") as fh:
        json.dump(table, fh, indent=1, sort_keys=True)
    print("\n".join(lines))


def load_traffic(path, workload, role):
    """Traffic bytes per launch if measured on the current kernel sources, else None."""
    if not path or not os.path.exists(path):
        return None
    e = json.load(open(path)).get("workloads", {}).get(f"{workload}_{role}")
    if not e or e.get("csrc_sha") != csrc_sha():
        return None
    return e["traffic"]


_GO = None     # set by the parent when every worker holds its rows
_READY = None  # number of workers holding their rows


def _init_worker(go, ready):
    global _GO, _READY
    _GO, _READY = go, ready


def _oracle_rows(dt, xr, mr, yr, dyr, qs, scale, causal, wait=True):
    """Worker side of the CPU baseline: the float64 oracle, as it stands, on a
    block of rows (forward, then backward on the GPU's y), one BLAS thread.
    With ``wait`` it reports that it holds its rows and starts when the parent
    says so. Returns the (start, end) of its work on the system's monotonic
    clock."""
    from threadpoolctl import threadpool_limits

    import oracle

    with threadpool_limits(limits=1):
        if wait:
            with _READY.get_lock():
                _READY.value += 1
            _GO.wait()
        t0 = time.monotonic()
        for i in range(len(qs)):
            oracle.forward_row(xr[i], dt, None if mr is None else mr[i], scale, causal, int(qs[i]))
            oracle.backward_row(yr[i], dyr[i], dt, scale)
        return t0, time.monotonic()


def _worker_ready():
    import oracle  # noqa: F401  (import cost paid before the timed sample)
    time.sleep(0.2)  # so that every worker takes one of these
    return os.getpid()


def start_cpu_pool(n_workers):
    """Worker processes for the CPU baseline, started fresh ("spawn") before
    this process touches the GPU; each imports numpy and the oracle only."""
    import concurrent.futures as cf
    import multiprocessing as mp

    ctx = mp.get_context("spawn")
    go, ready = ctx.Event(), ctx.Value("i", 0)
    pool = cf.ProcessPoolExecutor(n_workers, mp_context=ctx, initializer=_init_worker,
                                  initargs=(go, ready))
    pids = {f.result() for f in [pool.submit(_worker_ready) for _ in range(n_workers)]}
    return {"pool": pool, "go": go, "ready": ready}, len(pids)


def cpu_baseline(cp, n_workers, w, y, dy, fwd_b, bwd_b, cpu_seconds, cap_bytes=6 << 30):
    """The float64 oracle over a bounded, seeded sample of the workload's rows
    (forward + backward per row). The sample is sized for about ``cpu_seconds``
    of CPU work (from a short calibration) and at most ``cap_bytes`` of row
    data, split evenly over the worker processes, and handed to them before
    the clock starts; all start together, and the time is from the first
    start to the last end. GB/s of the same algorithmic bytes per row as the
    GPU figure."""
    import concurrent.futures as cf

    import numpy as np

    from tests.parity import gather_mask_rows, gather_rows

    B, H, Sq, Sk = w["x"].shape
    rows_total = B * H * Sq
    dt, causal = w["dtype"], w["causal"]
    esz = w["x"].element_size()
    # bytes of row r: the x (and mask share) it reads, y written; the backward
    # reads y and dy where y can be nonzero and writes dx. Summed over every row
    # these are exactly the forward's and the backward's algorithmic bytes.
    full = rows_total * Sk
    kept_all = (fwd_b // esz) - full          # x and mask elements read by the forward
    x_all = (bwd_b // esz - full) // 2        # x elements read (= y, dy read by the backward)
    mfrac = kept_all / x_all - 1.0 if x_all else 0.0

    def row_bytes(q):
        kept = np.minimum(q + 1, Sk) if causal else np.full_like(q, Sk)
        return ((kept * (1.0 + mfrac) + Sk) + (2 * kept + Sk)) * esz

    def gather(rows):
        return (gather_rows(w["x"], rows), gather_mask_rows(w["mask"], w["mode"],
                                                            w["x"].shape, rows),
                gather_rows(y, rows), gather_rows(dy, rows))

    order = np.random.default_rng(12345).permutation(rows_total)
    # calibration: one worker, no barrier
    cal = order[:64].tolist()
    xr, mr, yr, dyr = gather(cal)
    t0, t1 = cp["pool"].submit(_oracle_rows, dt, xr, mr, yr, dyr, np.asarray(cal) % Sq,
                               w["scale"], causal, False).result()
    per_row = (t1 - t0) / len(cal)
    n = int(min(rows_total, cpu_seconds / per_row, cap_bytes // (4 * Sk * esz)))
    n = max(n_workers, n - n % n_workers)
    rows = order[:n].tolist()
    xr, mr, yr, dyr = gather(rows)
    qs = np.asarray(rows) % Sq
    share = n // n_workers
    cp["ready"].value = 0
    cp["go"].clear()
    futs = []
    for i in range(n_workers):
        sl = slice(i * share, (i + 1) * share)
        futs.append(cp["pool"].submit(_oracle_rows, dt, xr[sl], None if mr is None else mr[sl],
                                      yr[sl], dyr[sl], qs[sl], w["scale"], causal, True))
    deadline = time.monotonic() + 300
    while cp["ready"].value < n_workers and time.monotonic() < deadline:
        time.sleep(0.01)
    cp["go"].set()
    spans = [f.result() for f in cf.as_completed(futs)]
    wall = max(e for _, e in spans) - min(s for s, _ in spans)
    cpu_s = sum(e - s for s, e in spans)
    done = share * n_workers
    done_bytes = float(row_bytes(qs[:done]).sum())
    return {"value": round(done_bytes / wall / 1e9, 4), "unit": "GB/s", "cores": n_workers,
            "kind": "oracle",
            "sample": f"forward+backward of {done} of {rows_total} rows (seeded random order), "
                      f"{share} rows per worker process, one thread each, all started together "
                      f"with their rows in memory: {wall:.2f} s wall, {cpu_s:.1f} s of CPU "
                      f"work; float64 numpy oracle",
            "threads": n_workers, "host_cpu_count": os.cpu_count(),
            "rows_per_s": round(done / wall, 1)}


def settle(torch, fn, seconds, sync_every):
    """Run ``fn`` untimed for ``seconds`` of wall time; returns the number of calls."""
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        fn()
        n += 1
        if n % sync_every == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def time_workload(torch, cfg_id, dev, stream, launches, settle_s):
    """Per-kernel rate of one workload: forward and backward (dy ~ N(0,1)),
    HIP events on the launch stream around each launch, after a settle phase."""
    from attention_softmax_amd import sms_backward, sms_forward
    from attention_softmax_amd.workloads import CONFIGS, make_config

    c = CONFIGS[cfg_id]
    w = make_config(cfg_id, dev, with_dy=True)
    x, mask, dy = w["x"], w["mask"], w["dy"]
    fwd_b, bwd_b = min_bytes(x.shape, x.element_size(), w["mode"], w["causal"])
    y, dx = torch.empty_like(x), torch.empty_like(x)

    def step():
        sms_forward(x, mask, y, w["scale"], w["causal"], stream=stream)
        sms_backward(y, dy, dx, w["scale"], w["causal"], stream=stream)

    n_settle = settle(torch, step, settle_s, 64 if x.numel() < 1 << 20 else 4)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(launches)]
    for e in ev:
        e[0].record(stream)
        sms_forward(x, mask, y, w["scale"], w["causal"], stream=stream)
        e[1].record(stream)
        sms_backward(y, dy, dx, w["scale"], w["causal"], stream=stream)
        e[2].record(stream)
    torch.cuda.synchronize()
    out = {"workload": c["name"].rsplit(", ", 1)[0], "settle_s": settle_s,
           "settle_steps": n_settle, "launches": launches}
    for role, b, i in (("forward", fwd_b, 0), ("backward", bwd_b, 1)):
        ms = sum(e[i].elapsed_time(e[i + 1]) for e in ev) / launches
        gbps = b / (ms * 1e-3) / 1e9
        out[role] = {"avg_us": round(ms * 1e3, 2), "bytes": b, "GBps": round(gbps, 1),
                     "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
    S = x.shape[3]
    out["target"] = ("80 % of HBM peak (S >= 1024)" if S >= 1024 else
                     "reported only (S < 1024)")
    del x, mask, dy, y, dx, w
    torch.cuda.empty_cache()
    return out


def torch_reference(torch, w, stream, fwd_b, bwd_b, fwd_ms, bwd_ms):
    """Unfused PyTorch on the same inputs, as context: softmax(x*scale + mask)
    with torch's own kernels (scale, mask add and softmax as separate passes;
    the mask broadcast as a view), and torch's softmax backward times scale."""
    x, dy, scale = w["x"], w["dy"], w["scale"]
    B, H, Sq, Sk = x.shape
    m = w["mask"]
    if m is not None:
        m = {"sq_sk": lambda t: t.view(1, 1, Sq, Sk), "b_sq_sk": lambda t: t.view(B, 1, Sq, Sk),
             "b_1_sk": lambda t: t.view(B, 1, 1, Sk), "full": lambda t: t}[w["mode"]](m)
    causal = None
    if w["causal"]:
        causal = torch.triu(torch.ones(Sq, Sk, dtype=torch.bool, device=x.device), diagonal=1)

    def fwd():
        s = x * scale
        if m is not None:
            s = s + m
        if causal is not None:
            s = s.masked_fill(causal, float("-inf"))
        return torch.softmax(s, dim=-1)

    def bwd(yt):
        return torch._softmax_backward_data(dy, yt, -1, x.dtype) * scale

    yt = fwd()
    for _ in range(2):
        fwd()
        bwd(yt)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    n = 5
    e[0].record(stream)
    for _ in range(n):
        fwd()
    e[1].record(stream)
    for _ in range(n):
        bwd(yt)
    e[2].record(stream)
    torch.cuda.synchronize()
    tf = e[0].elapsed_time(e[1]) / n
    tb = e[1].elapsed_time(e[2]) / n
    del yt
    torch.cuda.empty_cache()
    return {"what": "unfused PyTorch: x*scale (+mask) (masked_fill causal) softmax; "
                    "_softmax_backward_data * scale",
            "forward_us": round(tf * 1e3, 1), "backward_us": round(tb * 1e3, 1),
            "forward_GBps_algorithmic": round(fwd_b / (tf * 1e-3) / 1e9, 1),
            "backward_GBps_algorithmic": round(bwd_b / (tb * 1e-3) / 1e9, 1),
            "speedup_forward": round(tf / fwd_ms, 2), "speedup_backward": round(tb / bwd_ms, 2)}


def _time_launches(torch, fn, stream, n):
    """Average ms of ``fn()`` over n back-to-back calls, HIP events on ``stream``."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def bench_attention(args):
    """Fused attention forward + backward: fp16 [4,32,4096,128] Q, K, V, dO,
    causal, scale 1/sqrt(128)."""
    import torch

    import oracle
    from attention_softmax_amd import (sms_attention_backward, sms_attention_forward,
                                       sms_attention_workspace_bytes)
    from attention_softmax_amd.workloads import draw_x
    from tests.parity import to_np

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, H, S, D, causal = 4, 32, 4096, 128, True
    scale = D ** -0.5
    q = draw_x((B, H, S, D), "f16", ("normal", 1.0), 11, dev)
    k = draw_x((B, H, S, D), "f16", ("normal", 1.0), 12, dev)
    v = draw_x((B, H, S, D), "f16", ("normal", 1.0), 13, dev)
    do = draw_x((B, H, S, D), "f16", ("normal", 1.0), 14, dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(sms_attention_workspace_bytes(B, H, S), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    half = 0.5 if causal else 1.0
    # Algorithmic flops: forward Q K^T and P V; backward Q K^T (recomputed
    # once), dO V^T, P^T dO, dS K and dS^T Q.
    fwd_flops = 4.0 * B * H * S * S * D * half
    bwd_flops = 10.0 * B * H * S * S * D * half

    def fwd():
        sms_attention_forward(q, k, v, None, scale, causal, o=o, stream=stream)

    def fwd_lse():
        lse.copy_(sms_attention_forward(q, k, v, None, scale, causal, o=o, return_lse=True,
                                        stream=stream)[1])

    def bwd():
        sms_attention_backward(q, k, v, o, lse, do, None, scale, causal, dq=dq, dk=dk, dv=dv,
                               workspace=ws, stream=stream)

    fwd_lse()
    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    fwd_ms = _time_launches(torch, fwd, stream, args.steps)
    bwd_ms = _time_launches(torch, bwd, stream, args.steps)
    wall = time.perf_counter() - wall0
    step_ms = fwd_ms + bwd_ms
    tflops = (fwd_flops + bwd_flops) / (step_ms * 1e-3) / 1e12
    fwd_tf = fwd_flops / (fwd_ms * 1e-3) / 1e12
    bwd_tf = bwd_flops / (bwd_ms * 1e-3) / 1e12
    sdpa = None
    try:
        qg, kg, vg = (t.detach().clone().requires_grad_() for t in (q, k, v))
        F = torch.nn.functional.scaled_dot_product_attention

        def t_fwd():
            F(qg, kg, vg, is_causal=causal)

        out = F(qg, kg, vg, is_causal=causal)

        def t_bwd():
            torch.autograd.grad(out, (qg, kg, vg), do, retain_graph=True)

        for _ in range(3):
            t_fwd()
            t_bwd()
        torch.cuda.synchronize()
        tf_ms = _time_launches(torch, t_fwd, stream, 5)
        tb_ms = _time_launches(torch, t_bwd, stream, 5)
        sdpa = {"what": "torch.nn.functional.scaled_dot_product_attention, same tensors",
                "forward_us": round(tf_ms * 1e3, 1),
                "forward_TFLOPs": round(fwd_flops / (tf_ms * 1e-3) / 1e12, 1),
                "backward_us": round(tb_ms * 1e3, 1),
                "backward_TFLOPs": round(bwd_flops / (tb_ms * 1e-3) / 1e12, 1)}
    except RuntimeError as ex:  # context only
        sdpa = {"error": type(ex).__name__}
    cpu = None
    if args.cpu_seconds > 0:
        # the float64 oracle (forward, then backward) on the first n queries of
        # head (0, 0), n doubling until the time budget is spent; its matrix
        # products run on BLAS threads over the host's cores (at most 16)
        from threadpoolctl import threadpool_limits

        n, spent, done_flops = 16, 0.0, 0.0
        threads = max(1, min(args.cpu_workers, os.cpu_count() or 1))
        qn, kn, vn, don = (to_np(t[:1, :1]) for t in (q, k, v, do))
        with threadpool_limits(limits=threads):
            while spent < args.cpu_seconds and n <= S:
                t0 = time.perf_counter()
                oracle.attention.forward(qn[:, :, :n], kn, vn, "f16", scale=scale,
                                         is_causal=causal)
                oracle.attention.backward(qn[:, :, :n], kn, vn, don[:, :, :n], "f16",
                                          scale=scale, is_causal=causal)
                spent += time.perf_counter() - t0
                # the oracle multiplies every key (no causal skip)
                done_flops += 14.0 * n * S * D
                n *= 2
        cpu = {"value": round(done_flops / spent / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
               "kind": "oracle", "threads": threads, "host_cpu_count": os.cpu_count(),
               "sample": f"forward + backward of queries 0..{n // 2 - 1} of head (0,0) against "
                         f"all {S} keys, {spent:.1f} s, float64 numpy, BLAS on {threads} "
                         f"threads"}
    out = {
        "metric": "fused attention forward + backward TFLOP/s, 1 MI355X",
        "value": round(tflops, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "attention fp16 Q,K,V,dO [4,32,4096,128] N(0,1), causal",
                   "shape": [B, H, S, D], "causal": causal, "scale": scale},
        "forward": {"us": round(fwd_ms * 1e3, 1), "TFLOPs": round(fwd_tf, 1)},
        "backward": {"us": round(bwd_ms * 1e3, 1), "TFLOPs": round(bwd_tf, 1),
                     "launches": "dQ with rowsum(dO*O), dK + dV in one pass"},
        "roofline": {"bound": "mfma", "kernel": "backward (3 launches)",
                     "achieved": round(bwd_tf, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(bwd_tf / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": None},
        "torch_reference": sdpa, "cpu_baseline": cpu, "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.ingest:
        ingest(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): rows are "
              "independent, so a multi-GPU run is the same kernel on each GPU's share", file=sys.stderr)
        sys.exit(2)
    if args.op == "attention":
        bench_attention(args)
        return

    # CPU baseline workers first, while this process has not touched the GPU.
    pool, n_workers = None, 0
    if args.cpu_seconds > 0:
        n_workers = max(1, min(args.cpu_workers, os.cpu_count() or 1))
        pool, n_workers = start_cpu_pool(n_workers)

    import torch

    from attention_softmax_amd import sms_backward, sms_copy_reference, sms_forward, sms_path
    from attention_softmax_amd.workloads import CONFIGS, make_config

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = CONFIGS[args.workload]
    w = make_config(args.workload, dev, with_dy=True)
    x, mask, dy = w["x"], w["mask"], w["dy"]
    B, H, Sq, Sk = x.shape
    rows = B * H * Sq
    dbytes = x.element_size()
    fwd_b, bwd_b = min_bytes(x.shape, dbytes, w["mode"], w["causal"])
    step_b = fwd_b + bwd_b
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    stream = torch.cuda.current_stream(dev)
    log(f"workload {args.workload}: {cfg['name']}; path fwd={sms_path(x.dtype, Sk)}")

    def step():
        sms_forward(x, mask, y, w["scale"], w["causal"], stream=stream)
        sms_backward(y, dy, dx, w["scale"], w["causal"], stream=stream)

    n_settle = settle(torch, step, args.settle_seconds, 4) if args.settle_seconds > 0 else 0
    log(f"settle: {n_settle} steps in {args.settle_seconds} s")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K steps, HIP events between the two launches on their stream.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        ev[i][0].record(stream)
        sms_forward(x, mask, y, w["scale"], w["causal"], stream=stream)
        ev[i][1].record(stream)
        sms_backward(y, dy, dx, w["scale"], w["causal"], stream=stream)
        ev[i][2].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    value = step_b / (ms_step * 1e-3) / 1e9
    kern = {
        "forward": {"avg_us": round(fwd_ms * 1e3, 2), "bytes": fwd_b,
                    "GBps": round(fwd_b / (fwd_ms * 1e-3) / 1e9, 1)},
        "backward": {"avg_us": round(bwd_ms * 1e3, 2), "bytes": bwd_b,
                     "GBps": round(bwd_b / (bwd_ms * 1e-3) / 1e9, 1)},
    }
    for k in kern.values():
        k["frac_hbm_peak"] = round(k["GBps"] / HBM_PEAK_GBPS, 4)
    dom = "forward" if fwd_ms >= bwd_ms else "backward"
    log(f"timed: {ms_step:.4f} ms/step, {value:.1f} GB/s; {kern}")

    traffic = load_traffic(args.traffic, args.workload, dom)

    copy = ceiling = None
    if not args.no_copy:
        # Plain device copies moving the forward's byte count: torch's (whose
        # counters calibrate the traffic figures) and the library's own.
        n = fwd_b // 2
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(10):
            dst.copy_(src)
        c1.record(stream)
        torch.cuda.synchronize()
        cms = c0.elapsed_time(c1) / 10
        copy = {"bytes": 2 * n, "avg_us": round(cms * 1e3, 2),
                "GBps": round(2 * n / (cms * 1e-3) / 1e9, 1),
                "kernel": "torch's device copy (" + COPY_KERNEL + ")"}
        # The library's plain 16-byte copy of the same bytes (no arithmetic):
        # what a kernel that reads and writes them once reaches on this chip.
        n16 = n // 16 * 16
        for _ in range(3):
            sms_copy_reference(src[:n16], dst[:n16], stream=stream)
        c0.record(stream)
        for _ in range(20):
            sms_copy_reference(src[:n16], dst[:n16], stream=stream)
        c1.record(stream)
        torch.cuda.synchronize()
        cms = c0.elapsed_time(c1) / 20
        cgb = 2 * n16 / (cms * 1e-3) / 1e9
        ceiling = {"kernel": "sms_copy_reference (16-byte nontemporal loads and stores, "
                             "64 lanes per KB)",
                   "bytes": 2 * n16, "avg_us": round(cms * 1e3, 2), "GBps": round(cgb, 1),
                   "frac_hbm_peak": round(cgb / HBM_PEAK_GBPS, 4),
                   "forward_frac_of_copy": round(kern["forward"]["GBps"] / cgb, 4),
                   "backward_frac_of_copy": round(kern["backward"]["GBps"] / cgb, 4)}
        log(f"copy ceiling: {ceiling}")
        del src, dst

    torch_ref = None
    if not args.no_torch:
        torch_ref = torch_reference(torch, w, stream, fwd_b, bwd_b, fwd_ms, bwd_ms)

    cpu = None
    if pool is not None:
        cpu = cpu_baseline(pool, n_workers, w, y, dy, fwd_b, bwd_b, args.cpu_seconds)
        pool["pool"].shutdown()
        log(f"cpu baseline: {cpu}")

    del x, mask, dy, y, dx, w
    torch.cuda.empty_cache()
    others = {}
    for o in [int(t) for t in args.others.split(",") if t.strip()]:
        if o == args.workload:
            continue
        others[str(o)] = time_workload(torch, o, dev, stream, args.other_launches,
                                       min(1.0, args.settle_seconds))
        log(f"workload {o}: {others[str(o)]}")

    out = {
        "metric": "fused masked-softmax GB/s and % of HBM peak, fwd+bwd, 1 MI355X",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic",
        # The step times both passes on every workload: the name states that
        # instead of the passes the workload's own description lists.
        "config": {"workload": cfg["name"].rsplit(", ", 1)[0] + ", forward+backward step",
                   "shape": [B, H, Sq, Sk], "mask": cfg["mask"],
                   "causal": cfg["causal"], "scale": cfg["scale"], "pass": "forward+backward",
                   "dy": "N(0,1)"},
        "settle": {"seconds": args.settle_seconds, "steps": n_settle,
                   "what": "untimed steps before the warm-up, for the clocks to leave idle"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "rows_per_s": round(rows / (ms_step * 1e-3), 1),
        "step_bytes": step_b,
        "kernels": kern,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": kern[dom]["GBps"],
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": kern[dom]["frac_hbm_peak"], "traffic": traffic},
        "other_workloads": others,
        "copy_reference": copy,
        "copy_ceiling": ceiling,
        "torch_reference": torch_ref,
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
