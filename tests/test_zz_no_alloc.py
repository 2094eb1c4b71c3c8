"""fa_fwd_splitkv_static (the split-KV pass on the library's own device scratch, for callers
that cannot allocate) against fa_fwd_splitkv with a caller workspace, through the C ABI:
two calls in a row, the second on a smaller input, each compared with the workspace entry
point's output on the same inputs and with the float64 oracle."""
import json

import numpy as np
import pytest
import torch

import io_aware_exact_fa2_amd as fa
import oracle
import workloads
from workloads import Workload, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL_O = {"bf16": 1.5e-2, "fp16": 5e-3}
TOL_L = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.lib()


def _run(w, n_splits):
    q, k, v = workloads.make_inputs(w)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    dt = fa.FA_DTYPE_BF16 if w.dtype == "bf16" else fa.FA_DTYPE_FP16
    stream = torch.cuda.current_stream()
    need = fa.fa_fwd_splitkv_workspace_size(w.B, w.H, w.N, w.d, n_splits)
    assert 0 < need <= fa.FA_STATIC_SCRATCH_BYTES
    # the workspace entry point
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    o_ws, l_ws = torch.empty_like(qd), torch.empty(w.B, w.H, w.N, device=DEV)
    st = fa.fa_fwd_splitkv(qd, kd, vd, o_ws, l_ws, ws, need, w.B, w.H, w.N, w.d, w.scale,
                           int(w.causal), n_splits, dt, stream)
    assert st == fa.FA_OK
    # the static-scratch entry point (outputs pre-filled so unwritten elements show)
    o_st = torch.full_like(qd, float("nan"))
    l_st = torch.full((w.B, w.H, w.N), float("nan"), device=DEV)
    st = fa.fa_fwd_splitkv_static(qd, kd, vd, o_st, l_st, w.B, w.H, w.N, w.d, w.scale,
                                  int(w.causal), n_splits, dt, stream)
    assert st == fa.FA_OK, fa.fa_strerror(st)
    torch.cuda.synchronize()
    O, L = oracle.attention(to_f64(q), to_f64(k), to_f64(v), w.scale, w.causal)
    eo = float(np.abs(to_f64(o_st) - O).max())
    el = float(np.abs(to_f64(l_st) - L).max())
    same = bool(torch.equal(o_st, o_ws) and torch.equal(l_st, l_ws))
    print(json.dumps({"case": f"static/{w.name}", "max_abs_O": eo, "max_abs_L": el,
                      "equal_to_workspace_call": same}), flush=True)
    # same kernels on the same inputs: bitwise equal to the workspace call
    assert same
    assert eo <= TOL_O[w.dtype] and el <= TOL_L


def test_static_scratch_two_calls_second_smaller():
    """A large call, then a smaller one: the second must not see the first's partials."""
    _run(Workload("static_big", 1, 8, 4096, 128, "bf16", False, seed=9700), 2)
    _run(Workload("static_small", 1, 2, 1000, 64, "fp16", True, seed=9701, dist="stress"), 3)


def test_static_scratch_refuses_oversize():
    """Partials beyond the static scratch are refused with FA_ERR_SCRATCH, nothing launched."""
    B, H, N, d = 1, 64, 16384, 128
    assert fa.fa_fwd_splitkv_workspace_size(B, H, N, d, 4) > fa.FA_STATIC_SCRATCH_BYTES
    q = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, device=DEV)
    st = fa.fa_fwd_splitkv_static(q, q, q, o, lse, B, H, N, d, 0.1, 0, 4, fa.FA_DTYPE_BF16,
                                  torch.cuda.current_stream())
    assert st == fa.FA_ERR_SCRATCH
