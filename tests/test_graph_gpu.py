"""The entry points under HIP graph capture: the library allocates nothing, never
synchronises and issues no memset, so a forward + backward sequence captured once
replays to the same bits as eager calls (checked on several replays, with eager work
and synchronisations between them)."""
import pytest
import torch

import io_aware_exact_fa2_amd as fa
import workloads
from workloads import Workload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.lib()


@pytest.mark.parametrize("d,dtype,causal", [(128, "bf16", True), (64, "fp16", False)])
def test_graph_replays_match_eager(d, dtype, causal):
    w = Workload("graph", 2, 4, 700, d, dtype, causal, seed=9900 + d)
    q, k, v = (t.to(DEV) for t in workloads.make_inputs(w))
    do = workloads.make_grad(w).to(DEV)
    # eager reference
    o_ref, l_ref = fa.forward(q, k, v, causal=causal)
    g_ref = fa.backward(q, k, v, o_ref, l_ref, do, causal=causal)
    torch.cuda.synchronize()
    # static buffers, captured once
    o = torch.empty_like(q)
    lse = torch.empty_like(l_ref)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    fa.forward(q, k, v, causal=causal, out=o, lse=lse)  # warm up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fa.forward(q, k, v, causal=causal, out=o, lse=lse)
        fa.backward(q, k, v, o, lse, do, causal=causal, dq=dq, dk=dk, dv=dv)
    for rep in range(3):
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))  # eager work between replays; replay must overwrite all
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), rep
        assert torch.equal(lse, l_ref), rep
        for a, b in zip((dq, dk, dv), g_ref):
            assert torch.equal(a, b), rep
