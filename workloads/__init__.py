"""Seeded synthetic inputs for the attention forward pass.

This module is shared by the tests, the benchmark and the smoke check. It
produces Q, K and V tensors and nothing else: it holds none of the attention
arithmetic, so the CPU oracle and the HIP path can both consume its output
without sharing any code with each other.

Every tensor is drawn in float32 with numpy's PCG64 generator and then rounded
to bfloat16 or float16 on the CPU with round-to-nearest-even. Both sides of a
parity check read the same rounded tensors; the oracle upcasts them exactly to
float64.

Workloads (shapes are [B, H, N, d], row-major, contiguous):

* ``tiny``      1,1,256,64  bf16, Q,K,V ~ N(0,1), non-causal, scale 1/8
* ``tiny4``     1,1,4,4     bf16, Q,K,V ~ N(0,1), scale 1/2 (brute-force size)
* ``ai2048``    4,16,2048,128 bf16, N(0,1), non-causal: the N=2048, D=128
                arithmetic-intensity example of the iq-universe page
                ("How FlashAttention got over the O(N^2) memory wall",
                section on the standard-attention bottleneck)
* ``causal8k``  2,16,8192,128 bf16, N(0,1), causal
* ``long32k``   1,8,32768,128 bf16, N(0,1), causal, small batch
* ``stress4000`` 8,32,4000,64 fp16: Q,K ~ N(0, 3^2); in every (b, h) head,
                round(1% of N) key rows get a spike of 8*sqrt(d)*u added, each
                with its own direction u = g/|g|, g ~ N(0, I_d); V ~ U(-1, 1).
                N is not a multiple of any tile size.
* ``few16k``    1,1,16384,128 bf16, N(0,1), non-causal: one long head, whose 64
                query tiles of 256 rows leave most of the 256 compute units idle
                (the shape the split-KV pass is for)
* ``fewc16k``   1,2,16384,128 bf16, N(0,1), causal: the same with two heads and
                the causal mask

Draw order inside one call: Q, K, V, then the spike row indices (one
``choice`` per head, heads in (b, h) order), then the spike directions. The
output gradient dO of the backward pass is drawn by ``make_grad`` from a
separate stream, N(0, 1) for every workload.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "get", "make_inputs", "make_grad", "make_fp8_inputs",
           "to_f64", "scaled"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "bf16" or "fp16"
    causal: bool
    seed: int
    dist: str = "normal"  # "normal" or "stress"

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"bf16": torch.bfloat16, "fp16": torch.float16}[self.dtype]

    def flops(self) -> float:
        """Metric work: 4*B*H*N^2*d, halved for the causal mask."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2.0 if self.causal else f

    def min_bytes(self) -> int:
        """Read Q, K, V once, write O once (2-byte elements), 4 bytes of L per row."""
        rows = self.B * self.H * self.N
        return rows * self.d * 2 * 4 + rows * 4


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 256, 64, "bf16", False, 1),
    "tiny4": Workload("tiny4", 1, 1, 4, 4, "bf16", False, 11),
    "ai2048": Workload("ai2048", 4, 16, 2048, 128, "bf16", False, 2),
    "causal8k": Workload("causal8k", 2, 16, 8192, 128, "bf16", True, 3),
    "long32k": Workload("long32k", 1, 8, 32768, 128, "bf16", True, 4),
    "stress4000": Workload("stress4000", 8, 32, 4000, 64, "fp16", False, 5, "stress"),
    "few16k": Workload("few16k", 1, 1, 16384, 128, "bf16", False, 6),
    "fewc16k": Workload("fewc16k", 1, 2, 16384, 128, "bf16", True, 7),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def scaled(w: Workload, **kw) -> Workload:
    """The same distribution at another shape (for parity cases the CPU finishes fast)."""
    return replace(w, **kw)


def _round(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dtype)


def make_inputs(w: Workload, seed: int | None = None):
    """Return (q, k, v) as contiguous CPU tensors of the workload's dtype."""
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    shape = (w.B, w.H, w.N, w.d)
    if w.dist == "normal":
        q = rng.standard_normal(shape, dtype=np.float32)
        k = rng.standard_normal(shape, dtype=np.float32)
        v = rng.standard_normal(shape, dtype=np.float32)
    elif w.dist == "stress":
        q = rng.standard_normal(shape, dtype=np.float32) * np.float32(3.0)
        k = rng.standard_normal(shape, dtype=np.float32) * np.float32(3.0)
        v = rng.random(shape, dtype=np.float32) * np.float32(2.0) - np.float32(1.0)
        n_spike = max(1, int(round(0.01 * w.N)))
        rows = [rng.choice(w.N, size=n_spike, replace=False)
                for _ in range(w.B * w.H)]
        g = rng.standard_normal((w.B, w.H, n_spike, w.d))
        u = g / np.linalg.norm(g, axis=-1, keepdims=True)
        amp = 8.0 * math.sqrt(w.d)
        for bh, idx in enumerate(rows):
            b, h = divmod(bh, w.H)
            k[b, h, idx, :] += (amp * u[b, h]).astype(np.float32)
    else:
        raise ValueError(f"unknown distribution {w.dist!r}")
    dt = w.torch_dtype
    return _round(q, dt), _round(k, dt), _round(v, dt)


def make_grad(w: Workload, seed: int | None = None) -> torch.Tensor:
    """dO for the backward pass: [B, H, N, d] ~ N(0, 1), rounded to the workload's dtype,
    from its own stream (seed + 10007 unless given), so Q, K, V are unchanged."""
    rng = np.random.Generator(np.random.PCG64(w.seed + 10007 if seed is None else seed))
    g = rng.standard_normal((w.B, w.H, w.N, w.d), dtype=np.float32)
    return _round(g, w.torch_dtype)


def make_fp8_inputs(w: Workload, seed: int | None = None):
    """The workload's Q, K, V (drawn as by ``make_inputs``, before the 16-bit rounding)
    encoded as FP8 E4M3 codes with one scale per tensor: scale = max|x| / 448 (the
    largest E4M3 value), code = E4M3(x / scale) by torch's float8_e4m3fn conversion
    (round to nearest even). Returns (q8, k8, v8) as uint8 CPU tensors and the three
    scales as Python floats."""
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    shape = (w.B, w.H, w.N, w.d)
    if w.dist == "normal":
        xs = [rng.standard_normal(shape, dtype=np.float32) for _ in range(3)]
    elif w.dist == "stress":
        q, k, v = make_inputs(replace(w, dtype="bf16"), seed)  # same draws, incl. spikes
        xs = [t.float().numpy() for t in (q, k, v)]
    else:
        raise ValueError(f"unknown distribution {w.dist!r}")
    out, scales = [], []
    for x in xs:
        s = float(np.abs(x).max()) / 448.0
        t = torch.from_numpy(np.ascontiguousarray(x / np.float32(s), dtype=np.float32))
        out.append(t.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).contiguous())
        scales.append(s)
    return out[0], out[1], out[2], scales[0], scales[1], scales[2]


def spike_rows(w: Workload, seed: int | None = None):
    """The spiked key rows of a ``stress`` workload, per (b, h), in draw order."""
    if w.dist != "stress":
        return None
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    shape = (w.B, w.H, w.N, w.d)
    rng.standard_normal(shape, dtype=np.float32)
    rng.standard_normal(shape, dtype=np.float32)
    rng.random(shape, dtype=np.float32)
    n_spike = max(1, int(round(0.01 * w.N)))
    return [rng.choice(w.N, size=n_spike, replace=False) for _ in range(w.B * w.H)]


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a bf16/fp16/fp32 tensor (any device) to a float64 array."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)
