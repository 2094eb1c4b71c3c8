"""Host logic of the seeded input generators."""
import numpy as np
import torch

import workloads


def test_table_matches_the_five_workloads():
    w = workloads.WORKLOADS
    assert (w["tiny"].B, w["tiny"].H, w["tiny"].N, w["tiny"].d) == (1, 1, 256, 64)
    assert (w["ai2048"].B, w["ai2048"].H, w["ai2048"].N, w["ai2048"].d) == (4, 16, 2048, 128)
    assert w["causal8k"].causal and w["long32k"].causal
    assert not w["ai2048"].causal and not w["stress4000"].causal
    assert w["stress4000"].dtype == "fp16" and w["stress4000"].N % 64 != 0
    assert w["ai2048"].flops() == 4 * 4 * 16 * 2048 ** 2 * 128
    assert w["causal8k"].flops() == 4 * 2 * 16 * 8192 ** 2 * 128 / 2


def test_seeded_and_rounded():
    w = workloads.scaled(workloads.get("tiny"), N=100)
    a = workloads.make_inputs(w)
    b = workloads.make_inputs(w)
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16 and x.shape == (1, 1, 100, 64)
        assert torch.equal(x, y)
        assert x.is_contiguous()
    c = workloads.make_inputs(w, seed=w.seed + 1)
    assert not torch.equal(a[0], c[0])
    # the fp64 view is an exact upcast of the rounded values
    f = workloads.to_f64(a[0])
    assert np.array_equal(torch.from_numpy(f).to(torch.bfloat16).to(torch.float64).numpy(), f)


def test_stress_distribution():
    w = workloads.scaled(workloads.get("stress4000"), B=1, H=2)
    q, k, v = workloads.make_inputs(w)
    assert q.dtype == torch.float16
    vf = v.float()
    assert vf.min() >= -1 and vf.max() <= 1
    assert 2.8 < q.float().std() < 3.2
    spikes = workloads.spike_rows(w)
    kf = k.float()
    for bh, idx in enumerate(spikes):
        norms = kf[0, bh].norm(dim=-1)
        spiked = torch.zeros(w.N, dtype=torch.bool)
        spiked[torch.as_tensor(idx)] = True
        assert norms[spiked].mean() > 2.0 * norms[~spiked].mean()
