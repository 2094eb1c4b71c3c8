"""Parity of the HIP kernel with the float64 oracle, through the C ABI.

Bars (max-abs over every compared element): O within 1.5e-2 for bfloat16 and
5e-3 for float16, L within 1e-3. Reduced shapes that span several tiles and a
ragged tail are compared element by element, and so is every row of every head of the four
full-size workloads (one launch each, as the benchmark times them); a sampled-row
variant and properties that hold at any size run beside them.
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

TOL_O = {"bf16": 1.5e-2, "fp16": 5e-3}
TOL_L = 1e-3
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


def _gpu(q, k, v, causal, scale, rescale_log2=None):
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale, rescale_log2=rescale_log2)
    torch.cuda.synchronize()
    return o, lse


def _check(name, dtype, o_gpu, l_gpu, o_ref, l_ref):
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    l_gpu = np.asarray(l_gpu, dtype=np.float64)
    assert np.isfinite(o_gpu).all() and np.isfinite(l_gpu).all(), name
    eo = np.abs(o_gpu - o_ref)
    el = np.abs(l_gpu - l_ref)
    rec = {"case": name, "dtype": dtype, "max_abs_O": float(eo.max(initial=0)),
           "mean_abs_O": float(eo.mean()) if eo.size else 0.0,
           "max_abs_L": float(el.max(initial=0)),
           "rel_l2_O": float(np.linalg.norm(o_gpu - o_ref) / max(np.linalg.norm(o_ref), 1e-300))}
    _REPORT.append(rec)
    print(json.dumps(rec), flush=True)
    assert rec["max_abs_O"] <= TOL_O[dtype], rec
    assert rec["max_abs_L"] <= TOL_L, rec


def _full_case(w: Workload, causal=None, scale=None, q=None, k=None, v=None, name=None,
               rescale_log2=None):
    causal = w.causal if causal is None else causal
    scale = w.scale if scale is None else scale
    if q is None:
        q, k, v = workloads.make_inputs(w)
    o, lse = _gpu(q, k, v, causal, scale, rescale_log2)
    O, L = oracle.attention(to_f64(q), to_f64(k), to_f64(v), scale, causal)
    _check(name or f"{w.name}/{w.B}x{w.H}x{w.N}x{w.d}/causal={causal}", w.dtype,
           to_f64(o), to_f64(lse), O, L)
    return o, lse


# ------------------------------------------------------------- small, full compare
@pytest.mark.parametrize("causal", [False, True])
def test_tiny_workload(causal):
    _full_case(workloads.get("tiny"), causal=causal)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_tiny4_bruteforce_size(causal, dtype):
    w = workloads.scaled(workloads.get("tiny4"), dtype=dtype)
    q, k, v = workloads.make_inputs(w)
    o, lse = _gpu(q, k, v, causal, w.scale)
    Ob, Lb = oracle.attention_bruteforce(to_f64(q).tolist(), to_f64(k).tolist(),
                                         to_f64(v).tolist(), w.scale, causal)
    _check(f"tiny4/{dtype}/causal={causal}", dtype, to_f64(o), to_f64(lse),
           np.array(Ob), np.array(Lb))


def _embed(x, dtype):
    n = len(x)
    q = torch.zeros(1, 1, n, 4)
    k = torch.zeros(1, 1, n, 4)
    q[0, 0, :, 0] = 1.0
    k[0, 0, :, 0] = torch.tensor(x, dtype=torch.float32)
    v = torch.zeros(1, 1, n, 4)
    v[0, 0, :, :n] = torch.eye(n)
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    return q.to(dt), k.to(dt), v.to(dt)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("x", [[1.0, 3.0, 2.0], [1.0, 2.0, 3.0, 4.0]])
@pytest.mark.parametrize("causal", [False, True])
def test_page_examples(dtype, x, causal):
    """The pages' scalar examples as attention: S_ij = x_j, V = I, so every O row is
    the softmax of (a prefix of) x and L its logsumexp, by closed form."""
    q, k, v = _embed(x, dtype)
    o, lse = _gpu(q, k, v, causal, 1.0)
    n = len(x)
    O = np.zeros((1, 1, n, 4))
    L = np.zeros((1, 1, n))
    for i in range(n):
        keys = range(i + 1) if causal else range(n)
        den = math.fsum(math.exp(x[j]) for j in keys)
        for j in keys:
            O[0, 0, i, j] = math.exp(x[j]) / den
        L[0, 0, i] = math.log(den)
    _check(f"page_example/{x}/{dtype}/causal={causal}", dtype, to_f64(o), to_f64(lse), O, L)


REDUCED = [
    # name, B, H, N, d, dtype, causal, dist
    ("ai_shape_small", 2, 3, 640, 128, "bf16", False, "normal"),
    ("causal_small", 1, 4, 1000, 128, "bf16", True, "normal"),
    ("causal_tile_multiple", 2, 8, 512, 128, "bf16", True, "normal"),
    ("stress_small", 2, 4, 1000, 64, "fp16", False, "stress"),
    ("stress_causal", 1, 2, 777, 64, "fp16", True, "stress"),
    ("d64_bf16_causal", 1, 3, 333, 64, "bf16", True, "normal"),
    ("d128_fp16", 1, 2, 300, 128, "fp16", False, "normal"),
    # causal with a last query tile that is only partly inside N: some of a wave's two
    # 32-query blocks are valid, some are not
    ("d128_causal_ragged_fp16", 1, 2, 300, 128, "fp16", True, "normal"),
    ("d128_causal_short_tail", 2, 2, 260, 128, "bf16", True, "normal"),
]


@pytest.mark.parametrize("case", REDUCED, ids=[c[0] for c in REDUCED])
def test_reduced_shapes(case):
    name, B, H, N, d, dt, causal, dist = case
    w = Workload(name, B, H, N, d, dt, causal, seed=1000 + N + d, dist=dist)
    _full_case(w)


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
@pytest.mark.parametrize("scale_sign", [1.0, -1.0])
def test_several_items_per_workgroup(dt, scale_sign):
    """A grid several times the CU count at d = 128 without the causal mask: 600 heads of
    N = 300 give 1200 workgroups of 256 queries, and every head's second one has waves
    wholly past N; both signs of the scale."""
    w = Workload(f"items_{dt}", 2, 300, 300, 128, dt, False, seed=5100 + (dt == "fp16"))
    _full_case(w, scale=scale_sign * w.scale,
               name=f"items/{dt}/2x300x300x128/scale{'-' if scale_sign < 0 else '+'}")


def test_several_items_lazy_rescale_off():
    """The same grid with the literal per-block update on spiked inputs: tiles are fixed
    often, their scores recomputed from the K rows of the workgroup's own head."""
    w = Workload("items_tau0", 1, 600, 300, 128, "bf16", False, seed=5103, dist="stress")
    _full_case(w, rescale_log2=0.0, name="items/tau0/1x600x300x128/stress")


@pytest.mark.parametrize("d", [1, 2, 8, 16, 33, 48, 63, 65, 96, 100, 127])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_head_dims(d, causal):
    w = Workload(f"d{d}", 1, 2, 200, d, "bf16", causal, seed=2000 + d)
    _full_case(w)


@pytest.mark.parametrize("N", [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 257])
@pytest.mark.parametrize("causal", [False, True])
def test_sequence_lengths(N, causal):
    w = Workload(f"N{N}", 1, 3, N, 128, "bf16", causal, seed=3000 + N)
    _full_case(w)


@pytest.mark.parametrize("BH", [(1, 1), (1, 7), (2, 4), (3, 8)])
def test_head_counts(BH):
    B, H = BH
    for causal in (False, True):
        w = Workload(f"heads{B}x{H}", B, H, 200, 64, "fp16", causal, seed=4000 + B * H)
        _full_case(w)


RESCALE_CASES = [
    ("ai_small", 1, 4, 700, 128, "bf16", False, "normal"),
    ("causal_small", 1, 4, 900, 128, "bf16", True, "normal"),
    ("stress_small", 2, 4, 1000, 64, "fp16", False, "stress"),
    ("stress_causal", 1, 4, 1000, 128, "fp16", True, "stress"),
]


@pytest.mark.parametrize("tau", [0.0, 3.0, 15.0])
@pytest.mark.parametrize("case", RESCALE_CASES, ids=[c[0] for c in RESCALE_CASES])
def test_rescale_threshold(case, tau):
    """fa_fwd_ex at the literal per-block max update (0), an intermediate and the
    largest threshold: same results as the oracle; the spiked-key inputs force
    rescales mid-stream in every mode."""
    name, B, H, N, d, dt, causal, dist = case
    w = Workload(name, B, H, N, d, dt, causal, seed=8000 + N + d, dist=dist)
    _full_case(w, rescale_log2=tau, name=f"{name}/tau={tau}")


def test_rescale_threshold_modes_agree():
    w = workloads.scaled(workloads.get("stress4000"), B=1, H=8)
    q, k, v = (t.to(DEV) for t in workloads.make_inputs(w))
    outs = [fa.forward(q, k, v, rescale_log2=t) for t in (0.0, 8.0, 15.0)]
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert (o.float() - outs[0][0].float()).abs().max().item() <= 2 * TOL_O["fp16"]
        assert (l - outs[0][1]).abs().max().item() <= TOL_L


@pytest.mark.parametrize("scale", [-0.125, 0.0, 1.0, 3.0])
def test_scale_values(scale):
    w = Workload("scale", 1, 2, 150, 64, "bf16", True, seed=5000)
    _full_case(w, scale=scale, name=f"scale={scale}")


# ------------------------------------------------- full-size workloads, sampled rows
FULL = ["ai2048", "causal8k", "long32k", "stress4000"]


def _sample(w, rng):
    heads = sorted({(0, 0), (w.B - 1, w.H - 1),
                    (int(rng.integers(w.B)), int(rng.integers(w.H))),
                    (int(rng.integers(w.B)), int(rng.integers(w.H)))})
    fixed = [0, 1, 2, 63, 64, 65, 127, 128, 129, w.N // 2, w.N - 3, w.N - 2, w.N - 1]
    rows = np.unique(np.concatenate([np.array(fixed), rng.integers(0, w.N, 64)]))
    return heads, rows[rows < w.N]


@pytest.mark.parametrize("name", FULL)
def test_full_workload_sampled(name):
    w = workloads.get(name)
    q, k, v = workloads.make_inputs(w)
    o, lse = _gpu(q, k, v, w.causal, w.scale)
    rng = np.random.Generator(np.random.PCG64(w.seed + 77))
    heads, rows = _sample(w, rng)
    qf, kf, vf = to_f64(q), to_f64(k), to_f64(v)
    O, L = oracle.attention_rows(qf, kf, vf, w.scale, w.causal, heads, rows)
    og = np.stack([to_f64(o[b, h, torch.as_tensor(rows)]) for b, h in heads])
    lg = np.stack([to_f64(lse[b, h, torch.as_tensor(rows)]) for b, h in heads])
    _check(f"{name}/sampled", w.dtype, og, lg, O, L)

    # every row: finite, and O inside the per-column range of the values it averages
    assert torch.isfinite(lse).all() and torch.isfinite(o.float()).all()
    vd = v.to(DEV).float()
    if w.causal:
        lo = torch.cummin(vd, dim=2).values
        hi = torch.cummax(vd, dim=2).values
    else:
        lo = vd.amin(dim=2, keepdim=True)
        hi = vd.amax(dim=2, keepdim=True)
    of = o.float()
    tol = TOL_O[w.dtype]
    assert bool(((of >= lo - tol) & (of <= hi + tol)).all())
    # every row: L is at least the score of key 0 (always allowed) and at most
    # max score + log(#keys)
    qd, kd = q.to(DEV).float(), k.to(DEV).float()
    s0 = w.scale * (qd * kd[:, :, :1, :]).sum(-1)
    assert bool((lse >= s0 - TOL_L).all())
    del qd, kd, vd, of, lo, hi
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", FULL)
def test_full_workload_every_row(name):
    """Every row of every head of the full-size workload, element by element against the
    float64 oracle, in the launch configuration the benchmark times (one launch over the
    whole batch, so the full grid's tile order and the next-round cache warming run)."""
    w = workloads.get(name)
    _full_case(w, name=f"{name}/every_row")


def test_full_stress_every_row_literal_update():
    """The per-block max update as the pages write it (threshold 0: the reference max is
    raised on every key block that exceeds it), on every row of the full spiked-key
    workload, against the oracle."""
    w = workloads.get("stress4000")
    _full_case(w, rescale_log2=0.0, name="stress4000/every_row/tau=0")


@pytest.mark.parametrize("name", ["causal8k", "long32k"])
def test_causal_first_row(name):
    """Row 0 sees only key 0: O_0 = V_0 exactly and L_0 = S_00."""
    w = workloads.get(name)
    q, k, v = workloads.make_inputs(w)
    o, lse = _gpu(q, k, v, True, w.scale)
    assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])
    s00 = w.scale * (to_f64(q[:, :, 0]) * to_f64(k[:, :, 0])).sum(-1)
    assert np.abs(to_f64(lse[:, :, 0]) - s00).max() <= TOL_L


@pytest.mark.parametrize("name", ["ai2048", "causal8k", "long32k", "stress4000"])
def test_uniform_scores_closed_form(name):
    """Q = 0 makes every allowed score 0: L_i = ln(#allowed keys) and O_i is the
    mean of the allowed values, by closed form, at the full shapes. At N = 4000
    a kernel that let the zero-filled pad keys of the last tile into the sum
    would miss L by ln(4032/4000) > 1e-3."""
    w = workloads.get(name)
    _, k, v = workloads.make_inputs(w)
    q = torch.zeros_like(k)
    o, lse = _gpu(q, k, v, w.causal, w.scale)
    vd = v.to(DEV).double()
    n = torch.arange(1, w.N + 1, device=DEV, dtype=torch.float64)
    if w.causal:
        L = torch.log(n).expand_as(lse)
        O = torch.cumsum(vd, dim=2) / n[:, None]
    else:
        L = torch.full_like(lse, math.log(w.N), dtype=torch.float64)
        O = vd.mean(dim=2, keepdim=True).expand_as(vd)
    eo = (o.double() - O).abs().max().item()
    el = (lse.double() - L).abs().max().item()
    rec = {"case": f"{name}/uniform", "dtype": w.dtype, "max_abs_O": eo, "max_abs_L": el}
    _REPORT.append(rec)
    print(json.dumps(rec), flush=True)
    assert eo <= TOL_O[w.dtype] and el <= TOL_L, rec


def test_score_shift_invariance():
    """Appending a column that adds c to every score leaves O unchanged and adds c
    to L (the max shift cancels in the softmax)."""
    w = Workload("shift", 1, 2, 300, 63, "bf16", False, seed=6000)
    q, k, v = workloads.make_inputs(w)
    c, scale = 2.5, 0.125
    q2 = torch.cat([q, torch.ones(1, 2, 300, 1, dtype=q.dtype)], -1).contiguous()
    k2 = torch.cat([k, torch.full((1, 2, 300, 1), c / scale, dtype=k.dtype)], -1).contiguous()
    v2 = torch.cat([v, torch.zeros(1, 2, 300, 1, dtype=v.dtype)], -1).contiguous()
    o1, l1 = _gpu(q, k, v, False, scale)
    o2, l2 = _gpu(q2, k2, v2, False, scale)
    assert (o2[..., :63].float() - o1.float()).abs().max().item() <= TOL_O["bf16"]
    assert (l2 - l1 - c).abs().max().item() <= TOL_L


# ------------------------------------------------------------ runtime properties
def test_deterministic():
    w = workloads.get("ai2048")
    q, k, v = (t.to(DEV) for t in workloads.make_inputs(w))
    o1, l1 = fa.forward(q, k, v, causal=False)
    o2, l2 = fa.forward(q, k, v, causal=False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("d", [64, 100, 128])
def test_canaries_untouched(d):
    """Outputs written into the middle of larger buffers: nothing outside is touched."""
    B, H, N = 2, 3, 333
    w = Workload("canary", B, H, N, d, "bf16", True, seed=7000 + d)
    q, k, v = (t.to(DEV) for t in workloads.make_inputs(w))
    n = B * H * N * d
    pad = 4096
    obuf = torch.full((n + 2 * pad,), 7.0, dtype=torch.bfloat16, device=DEV)
    lbuf = torch.full((B * H * N + 2 * pad,), -3.0, dtype=torch.float32, device=DEV)
    o = obuf[pad:pad + n].view(B, H, N, d)
    lse = lbuf[pad:pad + B * H * N].view(B, H, N)
    fa.forward(q, k, v, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert bool((obuf[:pad] == 7.0).all() and (obuf[pad + n:] == 7.0).all())
    assert bool((lbuf[:pad] == -3.0).all() and (lbuf[pad + B * H * N:] == -3.0).all())
    O, L = oracle.attention(to_f64(q), to_f64(k), to_f64(v), w.scale, True)
    _check(f"canary/d={d}", "bf16", to_f64(o), to_f64(lse), O, L)


def test_side_stream():
    w = workloads.scaled(workloads.get("tiny"), H=4)
    q, k, v = (t.to(DEV) for t in workloads.make_inputs(w))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = fa.forward(q, k, v, causal=True)
    s.synchronize()
    O, L = oracle.attention(to_f64(q), to_f64(k), to_f64(v), w.scale, True)
    _check("side_stream", "bf16", to_f64(o), to_f64(lse), O, L)


def test_device_supported():
    """The MI355X this runs on is a gfx950 device; a device index past the last is not."""
    assert fa.fa_device_supported(torch.cuda.current_device()) == 1
    assert fa.fa_device_supported(torch.cuda.device_count()) == 0
    assert fa.fa_device_supported(-1) == 0


def test_device_info():
    """CU count and peak engine clock agree with torch's device properties and with the
    MI355X's published figures (256 CUs, 2.4 GHz); a missing device is an FA_ERR_HIP."""
    dev = torch.cuda.current_device()
    cus, khz = fa.fa_device_info(dev)
    assert cus == torch.cuda.get_device_properties(dev).multi_processor_count
    assert cus == 256
    assert 1_500_000 <= khz <= 3_000_000
    from concurrent.futures import ThreadPoolExecutor

    def missing():  # on a thread of its own: the HIP error it records is per thread
        with pytest.raises(fa.FAError) as e:
            fa.fa_device_info(torch.cuda.device_count())
        return e.value.status

    with ThreadPoolExecutor(1) as ex:
        assert ex.submit(missing).result() == fa.FA_ERR_HIP


def test_raw_abi_call_matches_forward():
    w = workloads.get("tiny")
    q, k, v = (t.to(DEV) for t in workloads.make_inputs(w))
    o = torch.empty_like(q)
    lse = torch.empty(1, 1, 256, dtype=torch.float32, device=DEV)
    st = fa.fa_fwd(q, k, v, o, lse, 1, 1, 256, 64, w.scale, 0,
                   torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK
    o2, l2 = fa.forward(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)
