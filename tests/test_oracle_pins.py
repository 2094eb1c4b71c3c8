"""Pins for the CPU oracle: each test fixes part of it with something other than
itself — the pages' worked examples, closed forms, library routines, brute force
and invariants that any correct attention must satisfy.

Sources are the pages named in ``oracle/__init__.py`` ([P1], [P2], [P3]).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
from oracle import online
import workloads

from conftest import GOLDEN


def _closed(expr: str) -> float:
    return float(eval(expr, {"__builtins__": {}}, {"exp": math.exp, "log": math.log}))


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(shape, seed, scale=1.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal(shape) * scale


def _compositions(n):
    """Every composition of n (2^(n-1) of them)."""
    for cuts in itertools.product([0, 1], repeat=n - 1):
        sizes, run = [], 1
        for c in cuts:
            if c:
                sizes.append(run)
                run = 1
            else:
                run += 1
        sizes.append(run)
        yield sizes


def _embed_scores(x, causal=False):
    """Attention whose score matrix is S_ij = x_j: q_i = e1, k_j = x_j e1, V = I
    (the attention form of the pages' scalar examples), scale 1."""
    n = len(x)
    q = np.zeros((1, 1, n, n))
    k = np.zeros((1, 1, n, n))
    q[0, 0, :, 0] = 1.0
    k[0, 0, :, 0] = x
    v = np.eye(n)[None, None]
    return q, k, v


# --------------------------------------------------------------------------- P1
def test_p1_online_walkthrough_x132():
    g = _golden("online_softmax_x132.json")
    states = online.online_softmax_scalar(g["x"])
    for (m, l), (m_expr, l_expr) in zip(states, g["states_closed_form"]):
        assert m == _closed(m_expr)
        assert l == pytest.approx(_closed(l_expr), rel=1e-15)
    # final running sum is the safe-softmax denominator
    assert states[-1][1] == pytest.approx(_closed(g["safe_denominator_closed_form"]), rel=1e-15)


def test_p1_online_recurrence_matches_library_logsumexp():
    x = _rand(1000, 7, 5.0)
    m, l = online.online_softmax_scalar(x)[-1]
    assert m == x.max()
    assert m + math.log(l) == pytest.approx(scipy.special.logsumexp(x), rel=1e-13)


# --------------------------------------------------------------------------- P2
def test_p2_block_merge_1234():
    g = _golden("split_softmax_1234.json")
    b1, b2 = g["blocks"]
    s1 = online.block_stats(b1)
    s2 = online.block_stats(b2)
    assert [s1[0], s2[0]] == g["block_max"]
    for s, expr in zip((s1, s2), g["block_sum_closed_form"]):
        assert s[1] == pytest.approx(_closed(expr), rel=1e-15)
    m, l = online.merge_stats(s1, s2)
    assert m == 4
    assert l == pytest.approx(_closed(g["merged_sum_closed_form"]), rel=1e-15)
    # the merge is exactly "scale the first block by exp(2-4) and add the second"
    assert l == pytest.approx(s1[1] * _closed(g["rescale_closed_form"]) + s2[1], rel=1e-15)
    # naive concatenation of per-block softmaxes is wrong: it sums to 2
    naive = np.concatenate([scipy.special.softmax(b1), scipy.special.softmax(b2)])
    assert naive.sum() == pytest.approx(g["naive_concat_sum"], rel=1e-15)
    assert abs(naive.sum() - 1.0) > 0.5


def test_p2_merge_order_free():
    x = _rand(64, 3, 4.0)
    parts = [x[:5], x[5:20], x[20:21], x[21:]]
    ref = online.block_stats(x)
    for perm in itertools.permutations(range(4)):
        acc = online.block_stats(parts[perm[0]])
        for p in perm[1:]:
            acc = online.merge_stats(acc, online.block_stats(parts[p]))
        assert acc[0] == ref[0]
        assert acc[1] == pytest.approx(ref[1], rel=1e-13)


# --------------------------------------------------------------------------- P3
@pytest.mark.parametrize("name,key", [("online_softmax_x132.json", "x"),
                                      ("split_softmax_1234.json", "scores")])
def test_p3_attention_form_noncausal(name, key):
    g = _golden(name)
    x = np.array(g[key], dtype=np.float64)
    q, k, v = _embed_scores(x)
    O, L = oracle.attention(q, k, v, 1.0, False)
    if "softmax_denominator_S" in g:
        S = _closed(g["softmax_denominator_S"])
        probs = [_closed(e.replace("S", repr(S))) for e in g["softmax_closed_form"]]
    else:
        probs = [_closed(e) for e in g["softmax_closed_form"]]
    for i in range(len(x)):
        np.testing.assert_allclose(O[0, 0, i], probs, rtol=1e-14, atol=1e-16)
        assert L[0, 0, i] == pytest.approx(_closed(g["logsumexp_closed_form"]), rel=1e-15)


def test_p3_attention_form_causal():
    g = _golden("split_softmax_1234.json")
    x = np.array(g["scores"], dtype=np.float64)
    q, k, v = _embed_scores(x)
    O, L = oracle.attention(q, k, v, 1.0, True)
    for i, expr in enumerate(g["causal_rows_closed_form"]["L"]):
        assert L[0, 0, i] == pytest.approx(_closed(expr), rel=1e-15)
        w = np.exp(x[: i + 1] - x[i])
        np.testing.assert_allclose(O[0, 0, i, : i + 1], w / w.sum(), rtol=1e-14)
        assert np.all(O[0, 0, i, i + 1:] == 0.0)
    assert O[0, 0, 0, 0] == 1.0


# --------------------------------------------------------------------------- P4
@pytest.mark.parametrize("causal", [False, True])
def test_p4_bruteforce_matches_oracle(causal):
    for n in range(1, 9):
        q = _rand((1, 2, n, 4), 100 + n)
        k = _rand((1, 2, n, 4), 200 + n)
        v = _rand((1, 2, n, 4), 300 + n)
        O, L = oracle.attention(q, k, v, 0.5, causal)
        Ob, Lb = oracle.attention_bruteforce(q.tolist(), k.tolist(), v.tolist(), 0.5, causal)
        np.testing.assert_allclose(O, np.array(Ob), rtol=0, atol=1e-13)
        np.testing.assert_allclose(L, np.array(Lb), rtol=0, atol=1e-13)


def test_p4_bruteforce_closed_form():
    g = _golden("split_softmax_1234.json")
    q, k, v = _embed_scores(np.array(g["scores"], dtype=np.float64))
    Ob, Lb = oracle.attention_bruteforce(q.tolist(), k.tolist(), v.tolist(), 1.0, True)
    for i, expr in enumerate(g["causal_rows_closed_form"]["L"]):
        assert Lb[0][0][i] == pytest.approx(_closed(expr), rel=1e-15)


def test_p4_tiny4_workload_bruteforce():
    w = workloads.get("tiny4")
    q, k, v = (workloads.to_f64(t) for t in workloads.make_inputs(w))
    for causal in (False, True):
        O, L = oracle.attention(q, k, v, w.scale, causal)
        Ob, Lb = oracle.attention_bruteforce(q.tolist(), k.tolist(), v.tolist(), w.scale, causal)
        np.testing.assert_allclose(O, np.array(Ob), atol=1e-13)
        np.testing.assert_allclose(L, np.array(Lb), atol=1e-13)


# --------------------------------------------------------------------------- P5
@pytest.mark.parametrize("n", [4, 8])
@pytest.mark.parametrize("causal", [False, True])
def test_p5_every_block_split(n, causal):
    q, k, v = (_rand((n, 4), s) for s in (1, 2, 3))
    O, L = oracle.attention(q[None, None], k[None, None], v[None, None], 0.5, causal)
    for kb in _compositions(n):
        Om, Lm = online.fa2_forward(q, k, v, 0.5, causal, kb)
        np.testing.assert_allclose(Om, O[0, 0], atol=1e-12)
        np.testing.assert_allclose(Lm, L[0, 0], atol=1e-12)
    for rb in _compositions(n):
        Om, Lm = online.fa2_forward(q, k, v, 0.5, causal, [n], rb)
        np.testing.assert_allclose(Om, O[0, 0], atol=1e-12)
        np.testing.assert_allclose(Lm, L[0, 0], atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_p5_random_splits_tiny_workload(causal):
    w = workloads.get("tiny")
    q, k, v = (workloads.to_f64(t)[0, 0] for t in workloads.make_inputs(w))
    O, L = oracle.attention(q[None, None], k[None, None], v[None, None], w.scale, causal)
    rng = np.random.Generator(np.random.PCG64(99))
    for _ in range(100):
        cuts = np.sort(rng.choice(np.arange(1, w.N), size=rng.integers(1, 20), replace=False))
        sizes = np.diff(np.concatenate([[0], cuts, [w.N]])).tolist()
        Om, Lm = online.fa2_forward(q, k, v, w.scale, causal, sizes, [64, 64, 128])
        np.testing.assert_allclose(Om, O[0, 0], atol=1e-12)
        np.testing.assert_allclose(Lm, L[0, 0], atol=1e-12)


def test_p5_model_is_not_trivially_exact():
    """Dropping the alpha rescale (the [P2] pseudocode read literally) must break
    the blockwise model: this is what makes the split tests meaningful."""
    q, k, v = (_rand((16, 4), s, 3.0) for s in (4, 5, 6))
    O, _ = online.fa2_forward(q, k, v, 1.0, False, [4, 4, 4, 4])
    # literal accumulation without the rescale
    acc = np.zeros((16, 4))
    l = np.zeros(16)
    m = np.full(16, -np.inf)
    for c0 in range(0, 16, 4):
        S = q @ k[c0:c0 + 4].T
        m = np.maximum(m, S.max(axis=1))
        P = np.exp(S - m[:, None])
        l = l + P.sum(axis=1)
        acc = acc + P @ v[c0:c0 + 4]
    assert np.abs(acc / l[:, None] - O).max() > 1e-3


# --------------------------------------------------------------------------- P6
@pytest.mark.parametrize("causal", [False, True])
def test_p6_fa1_order_equals_fa2_order(causal):
    q, k, v = (_rand((40, 8), s, 2.0) for s in (7, 8, 9))
    O, L = oracle.attention(q[None, None], k[None, None], v[None, None], 0.3, causal)
    for kb, rb in [([40], [40]), ([8] * 5, [16, 16, 8]), ([3, 17, 20], [1, 39]), ([1] * 40, [40])]:
        O1, L1 = online.fa1_forward(q, k, v, 0.3, causal, kb, rb)
        O2, L2 = online.fa2_forward(q, k, v, 0.3, causal, kb, rb)
        np.testing.assert_allclose(O1, O[0, 0], atol=1e-12)
        np.testing.assert_allclose(L1, L[0, 0], atol=1e-12)
        np.testing.assert_allclose(O1, O2, atol=1e-12)
        np.testing.assert_allclose(L1, L2, atol=1e-12)


# --------------------------------------------------------------------------- P7
@pytest.mark.parametrize("causal", [False, True])
def test_p7_lse_identity(causal):
    q, k, v = (_rand((1, 1, 50, 16), s) for s in (10, 11, 12))
    scale = 0.25
    O, L = oracle.attention(q, k, v, scale, causal)
    S = scale * (q[0, 0] @ k[0, 0].T)
    if causal:
        S = np.where(np.tril(np.ones((50, 50), bool)), S, -np.inf)
    P = np.exp(S - L[0, 0][:, None])
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-12)
    np.testing.assert_allclose(P, scipy.special.softmax(S, axis=1), atol=1e-12)
    np.testing.assert_allclose(O[0, 0], P @ v[0, 0], atol=1e-12)
    np.testing.assert_allclose(L[0, 0], scipy.special.logsumexp(S, axis=1), atol=1e-12)


# --------------------------------------------------------------------------- P8
@pytest.mark.parametrize("N", [2048, 4000])
def test_p8_uniform_scores_noncausal(N):
    v = _rand((1, 1, N, 8), 13)
    q = np.zeros((1, 1, N, 8))
    k = _rand((1, 1, N, 8), 14)
    rows = np.array([0, 1, N // 2, N - 1])
    O, L = oracle.attention_rows(q, k, v, 0.125, False, [(0, 0)], rows)
    np.testing.assert_allclose(L[0], math.log(N), atol=1e-12)
    np.testing.assert_allclose(O[0], np.broadcast_to(v[0, 0].mean(axis=0), O[0].shape), atol=1e-12)


def test_p8_uniform_scores_causal():
    N = 300
    v = _rand((1, 1, N, 8), 15)
    q = np.zeros((1, 1, N, 8))
    k = _rand((1, 1, N, 8), 16)
    O, L = oracle.attention(q, k, v, 0.125, True)
    np.testing.assert_allclose(L[0, 0], np.log(np.arange(1, N + 1)), atol=1e-12)
    prefix_mean = np.cumsum(v[0, 0], axis=0) / np.arange(1, N + 1)[:, None]
    np.testing.assert_allclose(O[0, 0], prefix_mean, atol=1e-12)


# --------------------------------------------------------------------------- P9
def test_p9_ragged_leak_is_detectable():
    """A kernel that let the zero-filled pad keys of the last 64- or 128-key tile
    into the sum at N=4000 would be off by more than the 1e-3 tolerance on L."""
    assert math.log(4032) - math.log(4000) > 1e-3
    assert math.log(4096) - math.log(4000) > 1e-3
    q = np.zeros((1, 1, 4000, 4))
    k = _rand((1, 1, 4000, 4), 17)
    v = _rand((1, 1, 4000, 4), 18)
    _, L = oracle.attention_rows(q, k, v, 1.0, False, [(0, 0)], np.array([0, 3999]))
    np.testing.assert_allclose(L, math.log(4000), atol=1e-12)


# -------------------------------------------------------------------------- P10
def test_p10_score_shift():
    q, k, v = (_rand((1, 1, 30, 6), s) for s in (20, 21, 22))
    scale, c = 0.5, 3.75
    O, L = oracle.attention(q, k, v, scale, False)
    q2 = np.concatenate([q, np.ones((1, 1, 30, 1))], axis=-1)
    k2 = np.concatenate([k, np.full((1, 1, 30, 1), c / scale)], axis=-1)
    v2 = v
    O2, L2 = oracle.attention(q2, k2, v2, scale, False)
    np.testing.assert_allclose(O2, O, atol=1e-12)
    np.testing.assert_allclose(L2, L + c, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_p10_linear_in_v(causal):
    q, k, v1, v2 = (_rand((1, 2, 25, 8), s) for s in (23, 24, 25, 26))
    O1, _ = oracle.attention(q, k, v1, 0.4, causal)
    O2, _ = oracle.attention(q, k, v2, 0.4, causal)
    O3, _ = oracle.attention(q, k, 2.0 * v1 - 3.0 * v2, 0.4, causal)
    np.testing.assert_allclose(O3, 2.0 * O1 - 3.0 * O2, atol=1e-12)


def test_p10_joint_key_permutation():
    q, k, v = (_rand((1, 1, 40, 8), s) for s in (27, 28, 29))
    O, L = oracle.attention(q, k, v, 0.4, False)
    perm = np.random.Generator(np.random.PCG64(30)).permutation(40)
    O2, L2 = oracle.attention(q, k[:, :, perm], v[:, :, perm], 0.4, False)
    np.testing.assert_allclose(O2, O, atol=1e-12)
    np.testing.assert_allclose(L2, L, atol=1e-12)


def test_p10_constant_value_rows():
    q, k = (_rand((1, 1, 33, 8), s, 3.0) for s in (31, 32))
    row = _rand(8, 33)
    v = np.broadcast_to(row, (1, 1, 33, 8)).copy()
    for causal in (False, True):
        O, _ = oracle.attention(q, k, v, 0.7, causal)
        np.testing.assert_allclose(O[0, 0], np.broadcast_to(row, (33, 8)), atol=1e-12)


# -------------------------------------------------------------------------- P11
def test_p11_stress_workload_moves_row_maxima():
    """On the generated stress inputs, most query rows take their maximum at a
    spiked key, so the running maximum jumps when a spike tile arrives."""
    w = workloads.get("stress4000")
    small = workloads.scaled(w, B=1, H=2)
    q, k, _ = workloads.make_inputs(small)
    q, k = workloads.to_f64(q), workloads.to_f64(k)
    spikes = workloads.spike_rows(small)
    assert all(len(s) == 40 for s in spikes)
    hits = 0
    for bh, idx in enumerate(spikes):
        b, h = divmod(bh, small.H)
        s = q[b, h] @ k[b, h].T
        hits += np.isin(s.argmax(axis=1), idx).sum()
    frac = hits / (small.H * small.N)
    assert frac >= 0.9, frac


# -------------------------------------------------------------------------- P12
def test_p12_causal_first_row():
    q, k, v = (_rand((2, 3, 20, 8), s) for s in (34, 35, 36))
    O, L = oracle.attention(q, k, v, 0.3, True)
    np.testing.assert_allclose(O[:, :, 0], v[:, :, 0], atol=1e-15)
    np.testing.assert_allclose(L[:, :, 0], 0.3 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
                               atol=1e-14)


# ----------------------------------------------------------- library routines
@pytest.mark.parametrize("causal", [False, True])
def test_oracle_matches_scipy_softmax(causal):
    q, k, v = (_rand((2, 2, 70, 16), s, 2.0) for s in (37, 38, 39))
    O, L = oracle.attention(q, k, v, 0.25, causal)
    for b in range(2):
        for h in range(2):
            S = 0.25 * q[b, h] @ k[b, h].T
            if causal:
                S = np.where(np.tril(np.ones((70, 70), bool)), S, -np.inf)
            np.testing.assert_allclose(L[b, h], scipy.special.logsumexp(S, axis=1), atol=1e-12)
            np.testing.assert_allclose(O[b, h], scipy.special.softmax(S, axis=1) @ v[b, h],
                                       atol=1e-12)


def test_single_key():
    q, k, v = (_rand((1, 1, 1, 5), s) for s in (40, 41, 42))
    for causal in (False, True):
        O, L = oracle.attention(q, k, v, 0.9, causal)
        np.testing.assert_allclose(O, v, atol=1e-15)
        assert L[0, 0, 0] == pytest.approx(0.9 * float(q[0, 0, 0] @ k[0, 0, 0]), rel=1e-14)


def test_rows_subset_equals_full():
    q, k, v = (_rand((2, 2, 90, 8), s) for s in (43, 44, 45))
    for causal in (False, True):
        O, L = oracle.attention(q, k, v, 0.5, causal)
        rows = np.array([0, 7, 63, 64, 89])
        heads = [(0, 1), (1, 0)]
        Os, Ls = oracle.attention_rows(q, k, v, 0.5, causal, heads, rows, chunk=2)
        for hi, (b, h) in enumerate(heads):
            np.testing.assert_allclose(Os[hi], O[b, h, rows], atol=1e-14)
            np.testing.assert_allclose(Ls[hi], L[b, h, rows], atol=1e-14)


def test_planted_mistakes_are_caught():
    """Plant plausible mistakes in a copy of the oracle on the CPU and check that
    the pins above would see them: each altered result disagrees with scipy."""
    q, k, v = (_rand((1, 1, 20, 8), s, 2.0) for s in (46, 47, 48))
    S = 0.5 * q[0, 0] @ k[0, 0].T
    ref_L = scipy.special.logsumexp(S, axis=1)
    ref_O = scipy.special.softmax(S, axis=1) @ v[0, 0]
    # dropped max term in L, transposed operand, wrong sign, missing scale
    bad = {
        "no_m_in_L": np.log(np.exp(S - S.max(1, keepdims=True)).sum(1)),
        "transposed": scipy.special.logsumexp(0.5 * (k[0, 0] @ q[0, 0].T), axis=1),
        "wrong_sign": scipy.special.logsumexp(-S, axis=1),
        "no_scale": scipy.special.logsumexp(S / 0.5, axis=1),
    }
    for name, L in bad.items():
        assert np.abs(L - ref_L).max() > 1e-3, name
    O_unnorm = np.exp(S - S.max(1, keepdims=True)) @ v[0, 0]
    assert np.abs(O_unnorm - ref_O).max() > 1e-3


# ------------------------------------------------------------------ backward (NEXT-1)
# oracle.attention_backward is the chain rule written out; these pins fix it with
# things other than itself: a library's automatic differentiation of the forward
# definition, finite differences of the (pinned) forward oracle, closed forms and
# identities of the softmax Jacobian.

def _bwd_inputs(B, H, N, d, seed):
    return (_rand((B, H, N, d), seed), _rand((B, H, N, d), seed + 1),
            _rand((B, H, N, d), seed + 2), _rand((B, H, N, d), seed + 3))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_autograd(causal):
    """torch's float64 autograd of the plain forward formula (a library routine)."""
    import torch
    q, k, v, do = _bwd_inputs(2, 2, 11, 5, 300)
    scale = 0.7
    tq, tk, tv = (torch.tensor(t, requires_grad=True) for t in (q, k, v))
    s = scale * tq @ tk.transpose(-1, -2)
    if causal:
        n = s.shape[-1]
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    o = torch.softmax(s, dim=-1) @ tv
    (o * torch.tensor(do)).sum().backward()
    dq, dk, dv = oracle.attention_backward(q, k, v, do, scale, causal)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences(causal):
    """Central differences of sum(O * dO) through the forward oracle (itself pinned)."""
    q, k, v, do = _bwd_inputs(1, 1, 6, 4, 310)
    scale = 0.9
    dq, dk, dv = oracle.attention_backward(q, k, v, do, scale, causal)

    def loss(q_, k_, v_):
        o, _ = oracle.attention(q_, k_, v_, scale, causal, workers=1)
        return float((o * do).sum())

    eps = 1e-6
    rng = np.random.Generator(np.random.PCG64(311))
    for which, grad in (("q", dq), ("k", dk), ("v", dv)):
        for _ in range(6):
            idx = (0, 0, int(rng.integers(6)), int(rng.integers(4)))
            args = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
            args[which][idx] += eps
            up = loss(args["q"], args["k"], args["v"])
            args[which][idx] -= 2 * eps
            dn = loss(args["q"], args["k"], args["v"])
            assert abs((up - dn) / (2 * eps) - grad[idx]) < 1e-7, (which, idx)


def test_backward_uniform_scores_closed_form():
    """Q = 0: P_ij = 1/N, so dV_j = mean_i dO_i, dK = 0 and
    dQ_i = scale/N * sum_j <dO_i, V_j - mean V> K_j."""
    _, k, v, do = _bwd_inputs(1, 2, 7, 3, 320)
    q = np.zeros_like(k)
    scale = 1.3
    dq, dk, dv = oracle.attention_backward(q, k, v, do, scale, False)
    n = q.shape[2]
    vbar = v.mean(axis=2, keepdims=True)
    want_dv = np.broadcast_to(do.mean(axis=2, keepdims=True), dv.shape)
    w = np.einsum("bhid,bhjd->bhij", do, v - vbar)
    want_dq = scale / n * np.einsum("bhij,bhjd->bhid", w, k)
    np.testing.assert_allclose(dv, want_dv, atol=1e-13)
    np.testing.assert_allclose(dk, 0.0, atol=1e-13)
    np.testing.assert_allclose(dq, want_dq, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_row_sums_vanish(causal):
    """Each row of dS sums to 0 (the softmax Jacobian annihilates constants): with all
    keys equal, dQ = scale * sum_j dS_ij K = 0; and the causal row 0 (one allowed key,
    P = 1) gets dQ_0 = 0 whatever its inputs."""
    q, _, v, do = _bwd_inputs(1, 1, 9, 4, 330)
    k = np.broadcast_to(_rand((1, 1, 1, 4), 331), q.shape).copy()
    dq, _, _ = oracle.attention_backward(q, k, v, do, 0.8, causal)
    np.testing.assert_allclose(dq, 0.0, atol=1e-13)
    q, k, v, do = _bwd_inputs(1, 1, 9, 4, 332)
    dq, _, _ = oracle.attention_backward(q, k, v, do, 0.8, True)
    np.testing.assert_allclose(dq[0, 0, 0], 0.0, atol=1e-13)


def test_backward_linear_in_do():
    """The gradients are linear in dO (a planted sign or scale mistake breaks this)."""
    q, k, v, do = _bwd_inputs(1, 1, 8, 4, 340)
    do2 = _rand(do.shape, 341)
    a = oracle.attention_backward(q, k, v, do, 0.6, False)
    b = oracle.attention_backward(q, k, v, do2, 0.6, False)
    c = oracle.attention_backward(q, k, v, 2.0 * do - 3.0 * do2, 0.6, False)
    for x, y, z in zip(a, b, c):
        np.testing.assert_allclose(z, 2.0 * x - 3.0 * y, atol=1e-12)


# ---------------------------------------------------------------- FP8 E4M3 decoding
def test_e4m3_decoder_named_values():
    """Values the OCP E4M3 definition fixes: 1.0, the largest finite (448), the
    smallest normal (2^-6) and subnormal (2^-9), signed zero, NaN at 0x7F / 0xFF."""
    d = oracle.decode_e4m3
    assert d(0x38) == 1.0 and d(0xB8) == -1.0
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert d(0x08) == 2.0 ** -6 and d(0x07) == 7 * 2.0 ** -9 and d(0x01) == 2.0 ** -9
    assert d(0x00) == 0.0 and np.signbit(d(0x80))
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0x30) == 0.5 and d(0x40) == 2.0 and d(0x2A) == 0.3125


def test_e4m3_decoder_matches_torch_for_every_code():
    """All 256 codes against torch's float8_e4m3fn conversion (an independent decoder)."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.decode_e4m3(codes)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    # monotone over the positive finite codes, and the round trip of the generator
    pos = got[:0x7F]
    assert np.all(np.diff(pos) > 0)


def test_attention_fp8_is_attention_of_the_decoded_inputs():
    """Codes whose decoded values are small dyadic numbers: the 8-bit oracle equals the
    brute force on the decoded tensors, and the per-tensor scales act as Q·qs etc."""
    rng = np.random.default_rng(99)
    shape = (1, 2, 6, 4)
    # exponent fields 6..8 -> |value| in [0.5, 4): exact in float64
    codes = [((rng.integers(0, 2, shape) << 7) | (rng.integers(6, 9, shape) << 3)
              | rng.integers(0, 8, shape)).astype(np.uint8) for _ in range(3)]
    qs, ks, vs, scale = 0.25, 2.0, 0.5, 0.7
    for causal in (False, True):
        O, L = oracle.attention_fp8(*codes, qs, ks, vs, scale, causal)
        q, k, v = (oracle.decode_e4m3(c) for c in codes)
        Ob, Lb = oracle.attention_bruteforce(q * qs, k * ks, v * vs, scale, causal)
        np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
        np.testing.assert_allclose(L, Lb, rtol=0, atol=1e-12)
        # scales fold into the scores and the output
        O2, L2 = oracle.attention(q, k, v, scale * qs * ks, causal)
        np.testing.assert_allclose(O, O2 * vs, rtol=0, atol=1e-12)
        np.testing.assert_allclose(L, L2, rtol=0, atol=1e-12)


def test_fp8_generator_codes_round_trip():
    """The input generator's codes decode to within one E4M3 rounding of the draws and
    use the full range (the largest magnitude maps to 448)."""
    w = workloads.Workload("f8", 1, 2, 64, 64, "bf16", False, seed=5)
    q8, k8, v8, qs, ks, vs = workloads.make_fp8_inputs(w)
    for c, s in ((q8, qs), (k8, ks), (v8, vs)):
        x = oracle.decode_e4m3(c.numpy())
        assert np.isfinite(x).all()
        assert np.abs(x).max() == 448.0
        assert s > 0
