"""Parity of the split-KV forward (fa_fwd_splitkv) and of the FA1-order ablation
(fa_fwd_fa1) with the float64 oracle, through the C ABI. Same bars as the FA2-order
forward: max-abs 1.5e-2 (bfloat16) / 5e-3 (float16) on O and 1e-3 on L."""
import json
import os

import numpy as np
import pytest
import torch

import io_aware_exact_fa2_amd as fa
import oracle
import workloads
from workloads import Workload, to_f64

pytestmark = pytest.mark.gpu

TOL_O = {"bf16": 1.5e-2, "fp16": 5e-3}
TOL_L = 1e-3
DEV = "cuda:0"
_REPORT = []


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.lib()
    yield
    path = os.environ.get("FA_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            for r in _REPORT:
                f.write(json.dumps(r) + "\n")


def _check(name, dtype, o, lse, O, L):
    og, lg = to_f64(o), to_f64(lse)
    assert np.isfinite(og).all() and np.isfinite(lg).all(), name
    rec = {"case": name, "dtype": dtype, "max_abs_O": float(np.abs(og - O).max()),
           "max_abs_L": float(np.abs(lg - L).max())}
    _REPORT.append(rec)
    print(json.dumps(rec), flush=True)
    assert rec["max_abs_O"] <= TOL_O[dtype] and rec["max_abs_L"] <= TOL_L, rec


def _run(w, path, n_splits=4):
    q, k, v = workloads.make_inputs(w)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    if path == "splitkv":
        o, lse = fa.forward_splitkv(qd, kd, vd, causal=w.causal, scale=w.scale, n_splits=n_splits)
    else:
        o, lse = fa.forward_fa1(qd, kd, vd, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    return q, k, v, o, lse


CASES = [
    # name, B, H, N, d, dtype, causal, dist
    ("d128_bf16", 1, 3, 700, 128, "bf16", False, "normal"),
    ("d128_bf16_causal", 1, 3, 1000, 128, "bf16", True, "normal"),
    ("d64_fp16_stress", 2, 2, 1000, 64, "fp16", False, "stress"),
    ("d64_fp16_stress_causal", 1, 2, 777, 64, "fp16", True, "stress"),
    ("d128_fp16_causal_tile_multiple", 2, 4, 512, 128, "fp16", True, "normal"),
    ("short", 1, 2, 65, 64, "bf16", True, "normal"),
    ("one_row", 1, 2, 1, 128, "bf16", False, "normal"),
]


@pytest.mark.parametrize("path", ["splitkv", "fa1"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_variant_parity(path, case):
    name, B, H, N, d, dt, causal, dist = case
    w = Workload(name, B, H, N, d, dt, causal, seed=8000 + N + d, dist=dist)
    q, k, v, o, lse = _run(w, path)
    O, L = oracle.attention(to_f64(q), to_f64(k), to_f64(v), w.scale, causal)
    _check(f"{path}/{name}", dt, o, lse, O, L)


@pytest.mark.parametrize("n_splits", [1, 2, 3, 7, 16, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_splitkv_split_counts(n_splits, causal):
    """Every split count gives the same result; at N = 1800 and 16 requested splits the
    keys per split round up to 256, so 8 splits run and the last is ragged."""
    w = Workload("splits", 1, 2, 1800, 128, "bf16", causal, seed=8100)
    q, k, v, o, lse = _run(w, "splitkv", n_splits)
    O, L = oracle.attention(to_f64(q), to_f64(k), to_f64(v), w.scale, causal)
    _check(f"splitkv/n{n_splits}/causal={causal}", "bf16", o, lse, O, L)


def test_splitkv_negative_scale():
    w = Workload("neg", 1, 2, 600, 64, "bf16", True, seed=8200)
    q, k, v = workloads.make_inputs(w)
    o, lse = fa.forward_splitkv(*(t.to(DEV) for t in (q, k, v)), causal=True, scale=-0.2,
                                n_splits=3)
    torch.cuda.synchronize()
    O, L = oracle.attention(to_f64(q), to_f64(k), to_f64(v), -0.2, True)
    _check("splitkv/negative_scale", "bf16", o, lse, O, L)


@pytest.mark.parametrize("path", ["splitkv", "fa1"])
def test_variant_full_ai2048_sampled(path):
    """The full non-causal B=4, H=16, N=2048, d=128 shape, sampled rows of two heads."""
    w = workloads.get("ai2048")
    q, k, v, o, lse = _run(w, path, n_splits=4)
    heads = [(0, 0), (3, 15)]
    rows = np.array([0, 1, 255, 256, 1023, 1024, 2046, 2047])
    O, L = oracle.attention_rows(to_f64(q), to_f64(k), to_f64(v), w.scale, False, heads, rows)
    og = torch.stack([o[b, h, torch.as_tensor(rows)] for b, h in heads])
    lg = torch.stack([lse[b, h, torch.as_tensor(rows)] for b, h in heads])
    _check(f"{path}/ai2048/sampled", "bf16", og, lg, O, L)


@pytest.mark.parametrize("name", ["few16k", "fewc16k"])
def test_splitkv_full_few_tile_every_row(name):
    """Every row of the full few-tile shapes that the split-KV pass is for (64 or 128
    query tiles for 256 compute units), through fa_fwd_splitkv with the split count the
    benchmark times and through fa_fwd, against the float64 oracle."""
    import bench

    w = workloads.get(name)
    q, k, v = workloads.make_inputs(w)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    O, L = oracle.attention(to_f64(q), to_f64(k), to_f64(v), w.scale, w.causal)
    o, lse = fa.forward_splitkv(qd, kd, vd, causal=w.causal, scale=w.scale,
                                n_splits=bench.SPLITKV[name])
    torch.cuda.synchronize()
    _check(f"splitkv/{name}/every_row", "bf16", o, lse, O, L)
    o, lse = fa.forward(qd, kd, vd, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    _check(f"fwd/{name}/every_row", "bf16", o, lse, O, L)


def test_variants_agree_with_fa2():
    """The three loop organisations give the same O and L up to rounding on one input."""
    w = Workload("agree", 2, 4, 900, 128, "bf16", True, seed=8300)
    q, k, v = (t.to(DEV) for t in workloads.make_inputs(w))
    o2, l2 = fa.forward(q, k, v, causal=True, scale=w.scale)
    o1, l1 = fa.forward_fa1(q, k, v, causal=True, scale=w.scale)
    os_, ls = fa.forward_splitkv(q, k, v, causal=True, scale=w.scale, n_splits=3)
    torch.cuda.synchronize()
    for o, l in ((o1, l1), (os_, ls)):
        assert (o.float() - o2.float()).abs().max().item() <= 2 * TOL_O["bf16"]
        assert (l - l2).abs().max().item() <= 2 * TOL_L
