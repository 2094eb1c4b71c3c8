"""Parity of the backward kernels (dQ, dK, dV) with the float64 oracle, through the C ABI.

The forward outputs O and L come from the HIP forward pass (as a caller would use
them); the oracle recomputes everything from Q, K, V and dO in float64.

Bar: for each of dQ, dK, dV, max |kernel - oracle| <= TOL_G * max |oracle| over the
compared elements, TOL_G = 2e-2 (bfloat16) and 5e-3 (float16). The kernels round
three intermediates to the input type before a matrix-core product (P, dS and, in
the forward, O, which enters D = rowsum(dO * O)) and round the result once more;
each is a relative error of at most u (2^-8 for bfloat16, 2^-11 for float16), so
an error of a few u of the largest gradient is the expected size: 5u for
bfloat16, 10u for float16. A gradient that is exactly zero in real arithmetic
(dQ and dK at N = 1) is held to the same fraction of 1e-3 of the case's largest
gradient.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import io_aware_exact_fa2_amd as fa
import oracle
import workloads
from workloads import Workload, to_f64

pytestmark = pytest.mark.gpu

TOL_G = {"bf16": 2e-2, "fp16": 5e-3}
DEV = "cuda:0"
_REPORT = []


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.lib()  # raises when the library is missing: no fallback
    yield
    path = os.environ.get("FA_PARITY_REPORT")
    if path:
        os.makedirs(os.path.dirname(path) or ".", exist_ok=True)
        with open(path, "a") as f:
            for r in _REPORT:
                f.write(json.dumps(r) + "\n")


def _gpu_grads(q, k, v, do, causal, scale):
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dod, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def _check(name, dtype, got, ref):
    rec = {"case": name, "dtype": dtype}
    ok = True
    # a gradient that is exactly zero in real arithmetic (dQ and dK at N = 1, where
    # dS = 0) is measured against 1e-3 of the largest of the three instead
    floor = 1e-3 * max(np.abs(r).max(initial=0.0) for r in ref)
    for tag, g, r in zip(("dQ", "dK", "dV"), got, ref):
        g = np.asarray(g, dtype=np.float64)
        assert np.isfinite(g).all(), (name, tag)
        err = np.abs(g - r).max(initial=0.0)
        mx = max(np.abs(r).max(initial=0.0), floor)
        rec[f"rel_max_{tag}"] = float(err / mx) if mx > 0 else float(err)
        ok &= err <= TOL_G[dtype] * mx
    _REPORT.append(rec)
    print(json.dumps(rec), flush=True)
    assert ok, rec


def _case(w: Workload, causal=None, scale=None):
    causal = w.causal if causal is None else causal
    scale = w.scale if scale is None else scale
    q, k, v = workloads.make_inputs(w)
    do = workloads.make_grad(w)
    got = _gpu_grads(q, k, v, do, causal, scale)
    ref = oracle.attention_backward(to_f64(q), to_f64(k), to_f64(v), to_f64(do), scale, causal)
    _check(f"{w.name}/{w.B}x{w.H}x{w.N}x{w.d}/causal={causal}/scale={scale:.4g}", w.dtype,
           [to_f64(t) for t in got], ref)


REDUCED = [
    # name, B, H, N, d, dtype, causal, dist
    ("ai_shape_small", 2, 3, 640, 128, "bf16", False, "normal"),
    ("causal_ragged", 1, 4, 1000, 128, "bf16", True, "normal"),
    ("causal_tile_multiple", 2, 2, 512, 128, "bf16", True, "normal"),
    ("d128_fp16", 1, 2, 300, 128, "fp16", False, "normal"),
    ("d128_fp16_causal", 1, 2, 300, 128, "fp16", True, "normal"),
    ("d64_bf16", 2, 2, 333, 64, "bf16", False, "normal"),
    ("d64_bf16_causal", 1, 3, 333, 64, "bf16", True, "normal"),
    ("stress_small", 2, 2, 1000, 64, "fp16", False, "stress"),
    ("stress_causal", 1, 2, 777, 64, "fp16", True, "stress"),
]


@pytest.mark.parametrize("case", REDUCED, ids=[c[0] for c in REDUCED])
def test_backward_reduced_shapes(case):
    name, B, H, N, d, dt, causal, dist = case
    _case(Workload(name, B, H, N, d, dt, causal, seed=7000 + N + d, dist=dist))


@pytest.mark.parametrize("N", [1, 2, 31, 63, 64, 65, 127, 128, 129, 255, 257])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_sequence_lengths(N, causal):
    _case(Workload(f"N{N}", 1, 2, N, 128, "bf16", causal, seed=7500 + N))


@pytest.mark.parametrize("N", [1, 65, 127, 128, 129, 255, 257, 383])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_sequence_lengths_d64(N, causal):
    # d = 64 stages 128-query tiles in the dK/dV kernel: lengths around its tile edges
    _case(Workload(f"N{N}d64", 1, 2, N, 64, "fp16", causal, seed=7700 + N))


@pytest.mark.parametrize("scale", [-0.3, 0.0, 0.02, 0.5])
@pytest.mark.parametrize("d", [64, 128])
def test_backward_scale_values(scale, d):
    # at d = 128 a zero scale takes the 32-key dK/dV kernel, any other the slot-scheduled one
    for causal in (False, True):
        _case(Workload("scale", 1, 2, 200, d, "bf16", causal, seed=7900 + d), scale=scale)


# Grids of several workgroups per CU with B*H not a multiple of 8 (the non-XCD tile
# order), ragged N at both head dims, and fp16 at d = 128 under the causal mask: every
# element against the oracle.
GRIDS = [
    # name, B, H, N, d, dtype, causal
    ("bh15_causal", 3, 5, 1100, 128, "bf16", True),
    ("bh15", 3, 5, 1100, 128, "bf16", False),
    ("bh7_d64_causal", 1, 7, 2047, 64, "fp16", True),
    ("bh6_fp16_causal", 2, 3, 1500, 128, "fp16", True),
]


@pytest.mark.parametrize("case", GRIDS, ids=[c[0] for c in GRIDS])
def test_backward_grid_shapes(case):
    name, B, H, N, d, dt, causal = case
    _case(Workload(name, B, H, N, d, dt, causal, seed=8100 + N + d))


# ------------------------------------------------------ full-size workloads, sampled heads
@pytest.mark.parametrize("name", ["ai2048", "causal8k", "stress4000"])
def test_backward_full_workload_sampled_heads(name):
    """The full shape in one launch; the oracle recomputes two of its heads."""
    w = workloads.get(name)
    q, k, v = workloads.make_inputs(w)
    do = workloads.make_grad(w)
    got = _gpu_grads(q, k, v, do, w.causal, w.scale)
    assert all(bool(torch.isfinite(t.float()).all()) for t in got)
    for b, h in ((0, 0), (w.B - 1, w.H - 1)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = oracle.attention_backward(to_f64(q[sl]), to_f64(k[sl]), to_f64(v[sl]),
                                        to_f64(do[sl]), w.scale, w.causal)
        _check(f"{name}/head{b},{h}", w.dtype, [to_f64(t[sl]) for t in got], ref)
    del got
    torch.cuda.empty_cache()


def test_backward_full_ai2048_every_head():
    """The full B=4, H=16, N=2048, d=128 shape in the launch the benchmark times: every
    element of every head against the float64 oracle, each head held to the bar of the
    reduced cases on its own."""
    w = workloads.get("ai2048")
    q, k, v = workloads.make_inputs(w)
    do = workloads.make_grad(w)
    got = [to_f64(t) for t in _gpu_grads(q, k, v, do, w.causal, w.scale)]
    ref = oracle.attention_backward(to_f64(q), to_f64(k), to_f64(v), to_f64(do), w.scale,
                                    w.causal)
    rec = {"case": "ai2048/every_head", "dtype": w.dtype}
    for tag, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert np.isfinite(g).all(), tag
        err = np.abs(g - r).max(axis=(2, 3))
        mx = np.abs(r).max(axis=(2, 3))
        rec[f"worst_head_rel_max_{tag}"] = float((err / mx).max())
    _REPORT.append(rec)
    print(json.dumps(rec), flush=True)
    assert all(rec[f"worst_head_rel_max_{t}"] <= TOL_G[w.dtype] for t in ("dQ", "dK", "dV")), rec
    del got, ref
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["ai2048", "causal8k", "long32k", "stress4000"])
def test_backward_constant_keys(name):
    """Identical key rows make each softmax row uniform over its allowed keys, so
    dS has zero row sums against a constant K: dQ = 0 exactly in real arithmetic,
    and dV_j = sum over queries i that see j of dO_i / (#keys i sees), in closed form.
    At the full shapes (every tile, every head)."""
    w = workloads.get(name)
    q, k, v = workloads.make_inputs(w)
    k = k[:, :, :1, :].expand_as(k).contiguous()
    do = workloads.make_grad(w)
    dq, dk, dv = _gpu_grads(q, k, v, do, w.causal, w.scale)
    dod = do.to(DEV).double()
    n = torch.arange(1, w.N + 1, device=DEV, dtype=torch.float64)
    if w.causal:
        t = dod / n[:, None]
        DV = torch.flip(torch.cumsum(torch.flip(t, [2]), 2), [2])  # sum over i >= j
    else:
        DV = (dod.sum(dim=2, keepdim=True) / w.N).expand_as(dod)
    ev = ((dv.double() - DV).abs().max() / DV.abs().max()).item()
    # dQ: each element is a sum of N terms dS_ij K_j whose exact total is 0; the
    # rounding of dS to the input type leaves at most about u * sum_j |dS_ij K_j|
    dqmax = dq.double().abs().max().item()
    dkmax = dk.double().abs().max().item()
    rec = {"case": f"{name}/constant_keys", "dtype": w.dtype, "rel_max_dV": ev,
           "max_dQ_over_max_dK": dqmax / max(dkmax, 1e-300)}
    _REPORT.append(rec)
    print(json.dumps(rec), flush=True)
    assert ev <= TOL_G[w.dtype], rec
    assert dqmax <= TOL_G[w.dtype] * dkmax, rec
    del dq, dk, dv, dod, DV
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["ai2048", "long32k", "stress4000"])
def test_backward_key_sums_vanish(name):
    """sum_j dK_j = scale * sum_i Q_i (sum_j dS_ij) = 0, since every row of dS sums to
    zero: a property of the exact gradient at any size, checked on every head."""
    w = workloads.get(name)
    q, k, v = workloads.make_inputs(w)
    do = workloads.make_grad(w)
    dq, dk, dv = _gpu_grads(q, k, v, do, w.causal, w.scale)
    s = dk.double().sum(dim=2)
    mag = dk.double().abs().sum(dim=2)
    worst = (s.abs() / mag.clamp_min(1e-300)).max().item()
    rec = {"case": f"{name}/key_sums", "dtype": w.dtype, "max_rel_key_sum": worst}
    _REPORT.append(rec)
    print(json.dumps(rec), flush=True)
    assert worst <= TOL_G[w.dtype], rec
    del dq, dk, dv
    torch.cuda.empty_cache()


def test_backward_deterministic():
    w = Workload("det", 1, 4, 700, 128, "bf16", True, seed=7777)
    q, k, v = workloads.make_inputs(w)
    do = workloads.make_grad(w)
    a = _gpu_grads(q, k, v, do, True, w.scale)
    b = _gpu_grads(q, k, v, do, True, w.scale)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_raw_abi_and_errors():
    """The raw C entry point writes the same bits as the tensor wrapper; invalid calls
    are rejected on the host (unsupported d, aliasing output)."""
    w = Workload("raw", 1, 2, 200, 64, "fp16", False, seed=7800)
    q, k, v = (t.to(DEV) for t in workloads.make_inputs(w))
    do = workloads.make_grad(w).to(DEV)
    o, lse = fa.forward(q, k, v, scale=w.scale)
    ref = fa.backward(q, k, v, o, lse, do, scale=w.scale)
    outs = [torch.empty_like(q) for _ in range(3)]
    st = fa.fa_bwd_fp16(q, k, v, o, lse, do, *outs, 1, 2, 200, 64, w.scale, 0,
                        torch.cuda.current_stream())
    assert st == fa.FA_OK
    torch.cuda.synchronize()
    for x, y in zip(ref, outs):
        assert torch.equal(x, y)
    assert fa.fa_bwd_fp16(q, k, v, o, lse, do, *outs, 1, 2, 200, 96, w.scale, 0,
                          None) == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_bwd_fp16(q, k, v, o, lse, do, q, outs[1], outs[2], 1, 2, 200, 64,
                          w.scale, 0, None) == fa.FA_ERR_ALIAS
    assert fa.fa_bwd(q, k, v, o, lse, do, outs[0], outs[0], outs[2], 1, 2, 200, 64,
                     w.scale, 0, None) == fa.FA_ERR_ALIAS
