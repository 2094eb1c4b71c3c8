"""CPU oracle for the attention forward pass — TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
anything from this package. The product path (the C-ABI library and its Python
binding) never imports, calls or links it, and this package never imports the
product path: the two share no code. Inputs reach both sides from the separate
``workloads`` module.

Sources (the three web pages the method is taken from):

* [P1] currybab.bearblog.dev, "Triton으로 FlashAttention 구현하기 전에 -
  FA1, 2 forward pass" — sections "왜 필요한가", "Online Softmax 개념",
  "FlashAttention 1 forward pass 알고리즘 분석",
  "FlashAttention 2 forward pass 알고리즘 분석", "정리".
* [P2] iq-universe.github.io, "FlashAttention은 어떻게 O(N²) 메모리 벽을
  넘었나" — sections "Online Softmax: 결합법칙이 tiling을 가능하게 한다",
  "FlashAttention: SRAM tiling으로 O(N²) HBM을 우회하다", "v2와 v3".
* [P3] ariser.io, "FlashAttention: 어텐션을 빠르게 만든 건 계산량보다 데이터
  이동이었다" — sections "N×N 행렬은 꼭 저장해야 할까",
  "소프트맥스는 나누어 계산할 수 있다".

Modules:

* ``attention``  — the plain definition in float64 (the parity reference).
* ``bruteforce`` — pure-Python loops without the max shift, for tiny inputs.
* ``online``     — the pages' algorithm steps (scalar online softmax, block
  merge, FA2 and FA1 loop orders) in float64, used to pin the pages' claims.
* ``backward``   — the gradients of the same definition (dQ, dK, dV) in float64,
  the reference for the backward pass that recomputes P from L.
* ``fp8``        — the OCP E4M3 decoder and attention on decoded 8-bit inputs with
  per-tensor scales, the reference for the 8-bit forward.

Every function here is pinned by ``tests/test_oracle_pins.py``; none is
"parity unpinned".
"""
from .attention import attention, attention_rows
from .bruteforce import attention_bruteforce
from .backward import attention_backward
from .fp8 import attention_fp8, attention_fp8_rows, decode_e4m3
from . import online

__all__ = ["attention", "attention_rows", "attention_bruteforce", "attention_backward",
           "attention_fp8", "attention_fp8_rows", "decode_e4m3", "online"]
