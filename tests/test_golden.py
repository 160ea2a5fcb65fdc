"""Rows worked by hand from the definitions (tests/golden/hand_rows.txt).

Each case states its inputs as exact values and its expected output as a
closed form; the file cites the passage each case follows. The CPU test pins
the float64 oracle to them (1e-15 relative, zeros exact); the GPU test runs
the same rows through the C ABI and holds the HIP path to the ordinary
tolerances (fp32: 1e-6 absolute; fp16: 2 ulp; exact zeros).
"""

import ast
import math
import os

import numpy as np
import pytest

import oracle.softmax as S

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_rows.txt")
NP_DTYPE = {"f32": np.float32, "f16": np.float16}
_NAMES = {"exp": math.exp, "log": math.log, "sqrt": math.sqrt, "e": math.e, "inf": math.inf}


def evaluate(expr):
    """Float64 value of an arithmetic expression over numbers and _NAMES."""
    def ev(n):
        if isinstance(n, ast.Expression):
            return ev(n.body)
        if isinstance(n, ast.Constant) and isinstance(n.value, (int, float)):
            return float(n.value)
        if isinstance(n, ast.Name) and n.id in _NAMES:
            return _NAMES[n.id]
        if isinstance(n, ast.UnaryOp) and isinstance(n.op, (ast.USub, ast.UAdd)):
            v = ev(n.operand)
            return -v if isinstance(n.op, ast.USub) else v
        if isinstance(n, ast.BinOp) and isinstance(n.op, (ast.Add, ast.Sub, ast.Mult, ast.Div)):
            a, b = ev(n.left), ev(n.right)
            if isinstance(n.op, ast.Add):
                return a + b
            if isinstance(n.op, ast.Sub):
                return a - b
            return a * b if isinstance(n.op, ast.Mult) else a / b
        if (isinstance(n, ast.Call) and isinstance(n.func, ast.Name) and n.func.id in _NAMES
                and len(n.args) == 1 and not n.keywords):
            return _NAMES[n.func.id](ev(n.args[0]))
        raise ValueError(f"unsupported expression: {expr!r}")
    return ev(ast.parse(expr, mode="eval"))


def _values(text):
    return [evaluate(t) for t in text.split()]


def load_cases(path=GOLDEN):
    cases, cur = [], {}
    with open(path) as fh:
        for raw in fh.read().splitlines() + [""]:
            line = raw.split("#", 1)[0].rstrip()
            if not line.strip():
                if cur:
                    cases.append(cur)
                    cur = {}
                continue
            key, _, rest = line.partition(" ")
            cur[key] = rest.strip()
    for c in cases:
        missing = {"case", "cite", "pass", "dtype", "scale", "want"} - set(c)
        assert not missing, (c.get("case"), missing)
        assert c["cite"], c["case"]
    return cases


CASES = load_cases()


def _inputs(c):
    """(typed inputs, scale, expected float64) of a case; inputs must be exact."""
    npt = NP_DTYPE[c["dtype"]]
    names = ("x", "mask") if c["pass"] == "forward" else ("y", "dy")
    typed = {}
    for n in names:
        if c.get(n, "none") == "none":
            typed[n] = None
            continue
        v = np.array(_values(c[n]), dtype=np.float64)
        t = v.astype(npt)
        assert np.array_equal(t.astype(np.float64), v), f"{c['case']}: {n} not exact in {c['dtype']}"
        typed[n] = t
    return typed, evaluate(c["scale"]), np.array(_values(c["want"]), dtype=np.float64)


def _causal_q(c):
    v = c.get("causal", "none")
    return None if v == "none" else int(v)


def test_golden_file_is_well_formed():
    names = [c["case"] for c in CASES]
    assert len(names) == len(set(names)) and len(names) >= 10
    for c in CASES:
        typed, _, want = _inputs(c)
        n = len(typed["x" if c["pass"] == "forward" else "y"])
        assert len(want) == n, c["case"]
        for t in typed.values():
            assert t is None or len(t) == n, c["case"]


@pytest.mark.parametrize("c", CASES, ids=lambda c: c["case"])
def test_oracle_matches_hand_rows(c):
    typed, scale, want = _inputs(c)
    if c["pass"] == "forward":
        q = _causal_q(c)
        got = S.forward_row(typed["x"], c["dtype"], mrow=typed["mask"], scale=scale,
                            is_causal=q is not None, q=q or 0)
    else:
        got = S.backward_row(typed["y"], typed["dy"], c["dtype"], scale=scale)
    got = np.asarray(got, dtype=np.float64)
    assert np.array_equal(got == 0.0, want == 0.0), (c["case"], got, want)
    nz = want != 0.0
    np.testing.assert_allclose(got[nz], want[nz], rtol=1e-15, atol=0, err_msg=c["case"])


@pytest.mark.gpu
@pytest.mark.parametrize("c", CASES, ids=lambda c: c["case"])
def test_hip_path_matches_hand_rows(c):
    import torch

    from attention_softmax_amd import sms_backward, sms_forward
    from tests.tolerance import compare

    dev = torch.device("cuda:0")
    tdt = {"f32": torch.float32, "f16": torch.float16}[c["dtype"]]
    typed, scale, want = _inputs(c)
    print(f"golden case {c['case']}", flush=True)
    if c["pass"] == "forward":
        q = _causal_q(c)
        n = len(typed["x"])
        Sq = n if q is not None else 1
        row = 0 if q is None else q
        x = torch.zeros((1, 1, Sq, n), dtype=tdt)
        x[0, 0, row] = torch.from_numpy(typed["x"].astype(np.float32)).to(tdt)
        mask = None
        if typed["mask"] is not None:
            mask = torch.zeros((Sq, n), dtype=tdt)
            mask[row] = torch.from_numpy(typed["mask"].astype(np.float32)).to(tdt)
            mask = mask.to(dev)
        x = x.to(dev)
        y = torch.empty_like(x)
        sms_forward(x, mask, y, scale, q is not None)
        torch.cuda.synchronize()
        got = y[0, 0, row].double().cpu().numpy()
    else:
        y = torch.from_numpy(typed["y"].astype(np.float32)).to(tdt).reshape(1, 1, 1, -1).to(dev)
        dy = torch.from_numpy(typed["dy"].astype(np.float32)).to(tdt).reshape(1, 1, 1, -1).to(dev)
        dx = torch.empty_like(y)
        sms_backward(y, dy, dx, scale, False)
        torch.cuda.synchronize()
        got = dx[0, 0, 0].double().cpu().numpy()
    compare(got[None], want[None], c["dtype"], what=c["case"])
