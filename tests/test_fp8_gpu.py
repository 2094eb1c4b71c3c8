"""Parity of the 8-bit forward (fa_fwd_fp8) with the float64 oracle on the decoded
inputs, through the C ABI.

Bar. Two effects separate the kernel from the exact result on the decoded inputs.
(1) Each unnormalised probability (at most 4 times the row's reference max, scaled by
2^6) is rounded to E4M3 before the P V product: a relative error of at most u8 = 2^-4
(3 mantissa bits, round to nearest even), independent across keys, and an absolute one
of at most 2^-10 / 2^6 = 2^-16 (in units of the reference, which the row max is at
least) where the scaled value is subnormal; so output element (i, c) is off by a sum of
such errors weighted by V_jc, of size u8 r_ic + 2^-16 z_c with
r_ic = sqrt(sum_j P_ij^2 V_jc^2) and z_c = sqrt(sum_j V_jc^2). (2) The 8-bit matrix instruction
sums the products of each group of 8 consecutive head dims aligned to the group's
largest product and truncates every product toward zero at 2^-13 of it (measured on
gfx950: 2^16 + 8 is exact, 2^16 + 4 gives 2^16, 2^16 + 12 gives 2^16 + 8), so a score is
off by at most dS_ij = 7 2^-13 |scale| sum_g max_{k in g} |Q_ik K_jk|, which moves L by
at most sum_j P_ij dS_ij and O by at most sum_j P_ij dS_ij |V_jc - O_ic| (first order).
The test requires, for every compared element,
    |O - O_ref| <= 8 (u8 r_ic + 2^-16 z_c) + 1.5 sum_j P_ij dS_ij |V_jc - O_ic|
                   + 2^-8 |O_ref| + 1e-6,
    |L - L_ref| <= 1e-3 + 1.5 sum_j P_ij dS_ij
(8 u8 r is about 14 standard deviations of the rounding sum; a wrong key or column order
gives errors of order r, 16 times larger than u8 r).
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

U8 = 2.0 ** -4
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


def _bounds(q, k, v, scale, causal, L, rows=None):
    """Per (b, h, row, c): r = sqrt(sum_j P^2 V^2), e = sum_j P dS |V - O|, and per row
    l = sum_j P dS, with P from the oracle's L and O = P V; q, k, v decoded values."""
    B, H, N, d = q.shape
    rows = np.arange(N) if rows is None else np.asarray(rows)
    r = np.empty((B, H, len(rows), d))
    e = np.empty_like(r)
    lb = np.empty((B, H, len(rows)))
    for b in range(B):
        for h in range(H):
            qh, kh, vh = q[b, h], k[b, h], v[b, h]
            s = scale * (qh[rows] @ kh.T)
            allowed = np.ones_like(s, dtype=bool)
            if causal:
                allowed = np.arange(N)[None, :] <= rows[:, None]
            s = np.where(allowed, s, -np.inf)
            lrow = L[b, h] if L.shape[2] == len(rows) else L[b, h, rows]
            p = np.exp(s - lrow[:, None])
            r[b, h] = np.sqrt((p * p) @ (vh * vh)) + 2.0 ** -12 * np.sqrt(
                allowed.astype(np.float64) @ (vh * vh))  # u8 r + 2^-16 z = u8 (r + 2^-12 z)
            o = p @ vh
            for c0 in range(0, len(rows), 64):  # row chunks keep the temporaries small
                sl = slice(c0, c0 + 64)
                ds = np.zeros((len(rows[sl]), N))
                for g in range(d // 8):
                    qa = np.abs(qh[rows[sl], 8 * g:8 * g + 8])
                    ka = np.abs(kh[:, 8 * g:8 * g + 8])
                    ds += (qa[:, None, :] * ka[None, :, :]).max(axis=-1)
                pd = p[sl] * ds * (7 * 2.0 ** -13 * abs(scale))
                lb[b, h, sl] = pd.sum(axis=1)
                e[b, h, sl] = np.einsum("ij,ijc->ic", pd,
                                        np.abs(vh[None, :, :] - o[sl][:, None, :]))
    return r, e, lb


def _check(name, o, lse, O, L, bounds):
    r, e, lb = bounds
    og, lg = to_f64(o), to_f64(lse)
    assert np.isfinite(og).all() and np.isfinite(lg).all(), name
    err = np.abs(og - O)
    bound = 8 * U8 * r + 1.5 * e + 2.0 ** -8 * np.abs(O) + 1e-6
    errl = np.abs(lg - L)
    rec = {"case": name, "dtype": "fp8", "max_abs_O": float(err.max()),
           "max_err_over_bound_O": float((err / bound).max()),
           "max_err_over_u8r": float((err / (U8 * r + 1e-30)).max()),
           "rel_l2_O": float(np.linalg.norm(og - O) / np.linalg.norm(O)),
           "max_abs_L": float(errl.max()),
           "max_err_over_bound_L": float((errl / (TOL_L + 1.5 * lb)).max())}
    _REPORT.append(rec)
    print(json.dumps(rec), flush=True)
    assert bool((err <= bound).all()), rec
    assert bool((errl <= TOL_L + 1.5 * lb).all()), rec


def _case(w, causal=None, scale=None):
    causal = w.causal if causal is None else causal
    scale = w.scale if scale is None else scale
    q8, k8, v8, qs, ks, vs = workloads.make_fp8_inputs(w)
    o, lse = fa.forward_fp8(q8.to(DEV), k8.to(DEV), v8.to(DEV), qs, ks, vs, causal=causal,
                            scale=scale)
    torch.cuda.synchronize()
    q, k, v = (oracle.decode_e4m3(t.numpy()) * s for t, s in ((q8, qs), (k8, ks), (v8, vs)))
    O, L = oracle.attention_fp8(q8.numpy(), k8.numpy(), v8.numpy(), qs, ks, vs, scale, causal)
    _check(f"fp8/{w.name}/{w.B}x{w.H}x{w.N}x{w.d}/causal={causal}/scale={scale:.4g}", o, lse,
           O, L, _bounds(q, k, v, scale, causal, L))


CASES = [
    # name, B, H, N, d, causal, dist
    ("d128", 1, 3, 700, 128, False, "normal"),
    ("d128_causal", 1, 3, 1000, 128, True, "normal"),
    ("d128_tile_multiple_causal", 2, 2, 512, 128, True, "normal"),
    ("d64", 2, 2, 333, 64, False, "normal"),
    ("d64_causal", 1, 3, 333, 64, True, "normal"),
    ("d64_stress", 2, 2, 1000, 64, False, "stress"),
    ("d128_stress_causal", 1, 2, 777, 128, True, "stress"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fp8_reduced_shapes(case):
    name, B, H, N, d, causal, dist = case
    _case(Workload(name, B, H, N, d, "bf16", causal, seed=9000 + N + d, dist=dist))


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 255, 256, 257])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_sequence_lengths(N, causal):
    _case(Workload(f"N{N}", 1, 2, N, 128, "bf16", causal, seed=9300 + N))


@pytest.mark.parametrize("scale", [-0.2, 0.01, 0.4])
def test_fp8_scale_values(scale):
    _case(Workload("scale", 1, 2, 300, 64, "bf16", True, seed=9400), scale=scale)


def test_fp8_full_ai2048_sampled():
    """The full B=4, H=16, N=2048, d=128 shape in one launch; sampled rows of 4 heads."""
    w = workloads.get("ai2048")
    q8, k8, v8, qs, ks, vs = workloads.make_fp8_inputs(w)
    o, lse = fa.forward_fp8(q8.to(DEV), k8.to(DEV), v8.to(DEV), qs, ks, vs, scale=w.scale)
    torch.cuda.synchronize()
    heads = [(0, 0), (1, 7), (2, 9), (3, 15)]
    rows = np.array([0, 1, 63, 64, 255, 256, 1000, 2046, 2047])
    O, L = oracle.attention_fp8_rows(q8.numpy(), k8.numpy(), v8.numpy(), qs, ks, vs, w.scale,
                                     False, heads, rows)
    q, k, v = (oracle.decode_e4m3(t.numpy()) * s for t, s in ((q8, qs), (k8, ks), (v8, vs)))
    parts = [_bounds(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1],
                     w.scale, False, L[i][None, None], rows)
             for i, (b, h) in enumerate(heads)]
    bounds = tuple(np.stack([pt[j][0, 0] for pt in parts]) for j in range(3))
    og = torch.stack([o[b, h, torch.as_tensor(rows)] for b, h in heads])
    lg = torch.stack([lse[b, h, torch.as_tensor(rows)] for b, h in heads])
    _check("fp8/ai2048/sampled", og, lg, O, L, bounds)
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())


@pytest.mark.parametrize("name", ["causal8k", "long32k"])
def test_fp8_full_causal_sampled(name):
    """The full causal shapes in one launch (the benchmark's 8-bit configurations):
    sampled rows of the first and last head, at tile edges and near the end."""
    w = workloads.get(name)
    q8, k8, v8, qs, ks, vs = workloads.make_fp8_inputs(w)
    o, lse = fa.forward_fp8(q8.to(DEV), k8.to(DEV), v8.to(DEV), qs, ks, vs, scale=w.scale,
                            causal=True)
    torch.cuda.synchronize()
    heads = [(0, 0), (w.B - 1, w.H - 1)]
    rows = np.array([0, 1, 31, 32, 63, 64, 127, 128, 1000, w.N // 2 - 1, w.N // 2,
                     w.N - 65, w.N - 64, w.N - 2, w.N - 1])
    O, L = oracle.attention_fp8_rows(q8.numpy(), k8.numpy(), v8.numpy(), qs, ks, vs, w.scale,
                                     True, heads, rows)
    q, k, v = (oracle.decode_e4m3(t.numpy()) * s for t, s in ((q8, qs), (k8, ks), (v8, vs)))
    parts = [_bounds(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1],
                     w.scale, True, L[i][None, None], rows)
             for i, (b, h) in enumerate(heads)]
    bounds = tuple(np.stack([pt[j][0, 0] for pt in parts]) for j in range(3))
    og = torch.stack([o[b, h, torch.as_tensor(rows)] for b, h in heads])
    lg = torch.stack([lse[b, h, torch.as_tensor(rows)] for b, h in heads])
    _check(f"fp8/{name}/sampled", og, lg, O, L, bounds)
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())
    del o, lse
    torch.cuda.empty_cache()


def test_fp8_full_ai2048_every_row():
    """The full B=4, H=16, N=2048, d=128 shape in one launch: every row of every head
    against the oracle on the decoded inputs, under the bar above (the per-head bound
    terms are computed on the host cores in parallel)."""
    from concurrent.futures import ThreadPoolExecutor

    w = workloads.get("ai2048")
    q8, k8, v8, qs, ks, vs = workloads.make_fp8_inputs(w)
    o, lse = fa.forward_fp8(q8.to(DEV), k8.to(DEV), v8.to(DEV), qs, ks, vs, scale=w.scale)
    torch.cuda.synchronize()
    O, L = oracle.attention_fp8(q8.numpy(), k8.numpy(), v8.numpy(), qs, ks, vs, w.scale, False)
    q, k, v = (oracle.decode_e4m3(t.numpy()) * s for t, s in ((q8, qs), (k8, ks), (v8, vs)))
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]

    def one(bh):
        b, h = bh
        return _bounds(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1],
                       w.scale, False, L[b:b + 1, h:h + 1])

    from oracle.attention import default_workers

    with ThreadPoolExecutor(max_workers=default_workers()) as ex:
        parts = list(ex.map(one, heads))
    bounds = tuple(np.stack([pt[j][0, 0] for pt in parts]).reshape(
        (w.B, w.H) + parts[0][j].shape[2:]) for j in range(3))
    _check("fp8/ai2048/every_row", o, lse, O, L, bounds)


def test_fp8_raw_abi_errors():
    w = Workload("raw", 1, 2, 100, 64, "bf16", False, seed=9500)
    q8, k8, v8, qs, ks, vs = (x.to(DEV) if torch.is_tensor(x) else x
                              for x in workloads.make_fp8_inputs(w))
    o = torch.empty((1, 2, 100, 64), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((1, 2, 100), dtype=torch.float32, device=DEV)
    args = dict(B=1, H=2, N=100)
    assert fa.fa_fwd_fp8(q8, k8, v8, qs, ks, vs, o, lse, 1, 2, 100, 96, 0.1, 0, None) == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_fwd_fp8(q8, k8, v8, qs, 0.0, vs, o, lse, 1, 2, 100, 64, 0.1, 0, None) == fa.FA_ERR_SHAPE
    assert fa.fa_fwd_fp8(q8, k8, v8, qs, ks, vs, q8, lse, 1, 2, 100, 64, 0.1, 0, None) == fa.FA_ERR_ALIAS
    assert fa.fa_fwd_fp8(q8, k8, v8, qs, ks, vs, o, lse, 1, 2, 100, 64, 0.1, 0, None) == fa.FA_OK
    torch.cuda.synchronize()
    del args


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_accumulation_model(causal):
    """The score error term of the bar, observed through the C ABI. With one key, L is the
    score itself (L = S_00 = scale qs ks <q8, k8>), so L shows how the 8-bit matrix core
    sums the products: those of each group of 8 consecutive head dims are aligned to the
    group's largest and truncated toward zero at 2^-13 of it. A group holding 256 * 256
    and seven 1 * 1 products sums to 2^16 (the exact 2^16 + 7 loses the ones), while
    products of equal size sum exactly."""
    d = 64
    ONE, P256 = 0x38, 0x78  # E4M3 codes of 1.0 and 256.0
    o = torch.empty((1, 1, 1, d), dtype=torch.bfloat16, device=DEV)
    v8 = torch.full((1, 1, 1, d), ONE, dtype=torch.uint8, device=DEV)
    cases = []
    # (q codes, k codes, the hardware dot product, the exact one)
    q = np.zeros(d, np.uint8); k = np.zeros(d, np.uint8)
    q[:8] = ONE; k[:8] = ONE; q[0] = k[0] = P256
    cases.append((q.copy(), k.copy(), 65536.0, 65536.0 + 7))
    q = np.zeros(d, np.uint8); k = np.zeros(d, np.uint8)
    q[:8] = ONE; k[:8] = ONE
    q[8:16] = ONE; k[8:16] = ONE                 # 16 products of 1 in two groups: exact
    cases.append((q.copy(), k.copy(), 16.0, 16.0))
    for qc, kc, hw, exact in cases:
        q8 = torch.from_numpy(qc.reshape(1, 1, 1, d)).to(DEV)
        k8 = torch.from_numpy(kc.reshape(1, 1, 1, d)).to(DEV)
        lse = torch.empty((1, 1, 1), dtype=torch.float32, device=DEV)
        sc = 1.0 / hw  # scale * qs * ks: the hardware's score becomes 1
        st = fa.fa_fwd_fp8(q8, k8, v8, 1.0, 1.0, 1.0, o, lse, 1, 1, 1, d, sc, int(causal), None)
        assert st == fa.FA_OK
        torch.cuda.synchronize()
        L = float(lse.item())
        # oracle on the decoded codes: the exact score
        O_ref, L_ref = oracle.attention_fp8(qc.reshape(1, 1, 1, d), kc.reshape(1, 1, 1, d),
                                            np.full((1, 1, 1, d), ONE, np.uint8), 1.0, 1.0,
                                            1.0, sc, bool(causal))
        rec = {"case": f"fp8/accumulation/{hw:g}", "L": L, "L_exact": float(L_ref[0, 0, 0]),
               "model": 1.0}
        _REPORT.append(rec)
        print(json.dumps(rec), flush=True)
        assert abs(L - 1.0) <= 2e-6, rec                       # the truncation model (fp32 path)
        if hw != exact:
            assert abs(L - exact / hw) >= 5e-5, rec            # and not the exact sum
        assert abs(float(L_ref[0, 0, 0]) - exact / hw) <= 1e-12  # the oracle's exact score
        # the bar's score term covers the difference
        ds = 7 * 2.0 ** -13 * sc * sum(
            max(abs(oracle.decode_e4m3(qc[i]) * oracle.decode_e4m3(kc[i])) for i in range(g, g + 8))
            for g in range(0, d, 8))
        assert abs(L - float(L_ref[0, 0, 0])) <= ds + 2e-6
        assert torch.equal(o.float().cpu(), torch.ones_like(o, dtype=torch.float32).cpu())
