"""Attention on FP8 E4M3 inputs with per-tensor scales, in float64 — TEST INFRASTRUCTURE.

The 8-bit path computes the same attention as the 16-bit one ([P1] problem statement
and FA2 section) on the decoded tensors Q = q_scale * decode(q8), and likewise for K
and V; the FP8 variant is the one [P2] ("v2와 v3") names as doubling the matrix
throughput. The pages do not define the 8-bit format; the reading here is OCP FP8 E4M3
(the format of the gfx950 8-bit matrix instructions): 1 sign bit, 4 exponent bits with
bias 7, 3 mantissa bits, subnormals at exponent 0, the two all-ones codes 0x7F / 0xFF
NaN and no infinity. The decoder below is written from that definition.
"""
from __future__ import annotations

import numpy as np

from .attention import attention, attention_rows

__all__ = ["decode_e4m3", "attention_fp8", "attention_fp8_rows"]


def decode_e4m3(codes) -> np.ndarray:
    """float64 values of E4M3 codes (any integer array of bytes)."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = m * 2.0 ** -9          # exponent field 0: m/8 * 2^(1 - 7)
    val = np.where(e == 0, sub, normal)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def _decoded(q8, k8, v8, qs, ks, vs):
    return (decode_e4m3(q8) * qs, decode_e4m3(k8) * ks, decode_e4m3(v8) * vs)


def attention_fp8(q8, k8, v8, q_scale, k_scale, v_scale, scale, causal):
    """O, L (float64) of the decoded tensors; codes [B, H, N, d]."""
    q, k, v = _decoded(q8, k8, v8, q_scale, k_scale, v_scale)
    return attention(q, k, v, scale, causal)


def attention_fp8_rows(q8, k8, v8, q_scale, k_scale, v_scale, scale, causal, heads, rows):
    """Sampled rows of the same result (see ``attention_rows``)."""
    q, k, v = _decoded(q8, k8, v8, q_scale, k_scale, v_scale)
    return attention_rows(q, k, v, scale, causal, heads, rows)
