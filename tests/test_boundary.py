"""The C-ABI boundary on the CPU: the library loads, exports every entry point
include/fa.h declares, and rejects invalid arguments on the host before any HIP
call (so these calls never touch a device; the fake addresses below are never
dereferenced)."""
import ctypes
import os
import re
import subprocess

import pytest

import io_aware_exact_fa2_amd as fa
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "fa.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fa.library_path()):
        pytest.fail("libfa.so is not built (run __graft_entry__.build())")
    return fa.lib()


@pytest.fixture
def no_gpu():
    """Calls below pass fake device addresses that validation must reject. They run
    only where no GPU exists, so a validation bug can never reach a real launch."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("fake-pointer validation tests run on GPU-less hosts only")


def test_header_declares_the_boundary():
    assert _declared_functions() == sorted(fa.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", fa.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fa_\w+)$", out, flags=re.M))
    for name in _declared_functions():
        assert name in exported, name
        assert hasattr(L, name)


def test_strerror_and_version(L):
    for code in (fa.FA_OK, fa.FA_ERR_NULL, fa.FA_ERR_SHAPE, fa.FA_ERR_UNSUPPORTED,
                 fa.FA_ERR_ALIAS, fa.FA_ERR_ALIGN, fa.FA_ERR_HIP, fa.FA_ERR_SCRATCH):
        assert fa.fa_strerror(code) and fa.fa_strerror(code) != "unknown status"
    assert fa.fa_strerror(12345) == "unknown status"
    assert "gfx950" in fa.fa_version()
    assert fa.fa_last_hip_error() == 0


def test_device_query_without_a_gpu(L, no_gpu):
    """On a host without a GPU no device is supported, and the query leaves no error."""
    assert fa.fa_device_supported(0) == 0
    assert fa.fa_device_supported(-1) == 0
    assert fa.fa_last_hip_error() == 0


def test_device_info_without_a_gpu(L, no_gpu):
    """Without a GPU the device query fails with FA_ERR_HIP and zeroed outputs; NULL
    outputs are rejected before any HIP call."""
    import ctypes
    from concurrent.futures import ThreadPoolExecutor

    def probe():
        # on a thread of its own: the HIP error it records is per thread
        cus, khz = ctypes.c_int(7), ctypes.c_int(7)
        st = L.fa_device_info(0, ctypes.byref(cus), ctypes.byref(khz))
        with pytest.raises(fa.FAError):
            fa.fa_device_info(0)
        return st, cus.value, khz.value, fa.fa_last_hip_error()

    with ThreadPoolExecutor(1) as ex:
        st, cus, khz, err = ex.submit(probe).result()
    assert st == fa.FA_ERR_HIP and (cus, khz) == (0, 0) and err != 0
    c = ctypes.c_int(0)
    assert L.fa_device_info(0, None, ctypes.byref(c)) == fa.FA_ERR_NULL
    assert L.fa_device_info(0, ctypes.byref(c), None) == fa.FA_ERR_NULL
    assert fa.fa_last_hip_error() == 0


def test_supported_query(L):
    for d in (1, 4, 63, 64, 65, 127, 128):
        for dt in (fa.FA_DTYPE_BF16, fa.FA_DTYPE_FP16):
            for c in (0, 1):
                assert fa.fa_fwd_supported(d, dt, c) == 1
    assert fa.fa_fwd_supported(0, 0, 0) == 0
    assert fa.fa_fwd_supported(129, 0, 0) == 0
    assert fa.fa_fwd_supported(64, 2, 0) == 0


# Fake, never-dereferenced device addresses: far apart, 256-byte aligned.
QA, KA, VA, OA, LA = (0x7f0000000000 + i * 0x100000000 for i in range(5))
GOOD = dict(B=2, H=3, N=100, d=64, scale=0.125, causal=0)


def _call(fn, q=QA, k=KA, v=VA, o=OA, lse=LA, **kw):
    a = dict(GOOD, **kw)
    return fn(q, k, v, o, lse, a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"], None)


@pytest.mark.parametrize("fn", [fa.fa_fwd, fa.fa_fwd_fp16])
def test_validation_errors(L, no_gpu, fn):
    assert _call(fn, q=0) == fa.FA_ERR_NULL
    assert _call(fn, k=0) == fa.FA_ERR_NULL
    assert _call(fn, v=0) == fa.FA_ERR_NULL
    assert _call(fn, o=0) == fa.FA_ERR_NULL
    assert _call(fn, lse=0) == fa.FA_ERR_NULL
    for bad in (dict(B=0), dict(H=0), dict(N=0), dict(d=0), dict(B=-1), dict(N=-5)):
        assert _call(fn, **bad) == fa.FA_ERR_SHAPE, bad
    for s in (float("nan"), float("inf"), float("-inf")):
        assert _call(fn, scale=s) == fa.FA_ERR_SHAPE
    assert _call(fn, d=129) == fa.FA_ERR_UNSUPPORTED
    assert _call(fn, d=100000) == fa.FA_ERR_UNSUPPORTED
    # N*d must stay below 2^31
    assert _call(fn, N=2 ** 24, d=128) == fa.FA_ERR_SHAPE
    # grid limit
    assert _call(fn, B=2 ** 20, H=2 ** 10, N=1024) == fa.FA_ERR_SHAPE
    # alignment
    assert _call(fn, q=QA + 8) == fa.FA_ERR_ALIGN
    assert _call(fn, o=OA + 2) == fa.FA_ERR_ALIGN
    assert _call(fn, lse=LA + 2) == fa.FA_ERR_ALIGN
    # aliasing of outputs with inputs or each other
    tbytes = GOOD["B"] * GOOD["H"] * GOOD["N"] * GOOD["d"] * 2
    assert _call(fn, o=QA) == fa.FA_ERR_ALIAS
    assert _call(fn, o=KA + 16 * ((tbytes - 16) // 16)) == fa.FA_ERR_ALIAS
    assert _call(fn, lse=VA + 64) == fa.FA_ERR_ALIAS
    assert _call(fn, lse=OA + tbytes - 16) == fa.FA_ERR_ALIAS
    # no HIP call was made by any of the above
    assert fa.fa_last_hip_error() == 0


def test_fa_fwd_ex_validation(L, no_gpu):
    def ex(dtype=fa.FA_DTYPE_BF16, tau=8.0, q=QA, k=KA, v=VA, o=OA, lse=LA, **kw):
        a = dict(GOOD, **kw)
        return fa.fa_fwd_ex(q, k, v, o, lse, a["B"], a["H"], a["N"], a["d"], a["scale"],
                            a["causal"], dtype, tau, None)
    assert ex(dtype=2) == fa.FA_ERR_UNSUPPORTED
    assert ex(dtype=-1) == fa.FA_ERR_UNSUPPORTED
    for tau in (-0.5, 15.5, 100.0, float("nan"), float("inf")):
        assert ex(tau=tau) == fa.FA_ERR_SHAPE, tau
    assert ex(tau=0.0, N=0) == fa.FA_ERR_SHAPE
    assert ex(tau=fa.FA_MAX_RESCALE_LOG2, o=QA) == fa.FA_ERR_ALIAS
    assert ex(dtype=fa.FA_DTYPE_FP16, tau=0.0, q=0) == fa.FA_ERR_NULL
    assert fa.fa_last_hip_error() == 0


# fake addresses of the backward's extra buffers (same spacing as above)
DOA, DQA, DKA, DVA = (0x7f0000000000 + i * 0x100000000 for i in range(5, 9))


@pytest.mark.parametrize("fn", [fa.fa_bwd, fa.fa_bwd_fp16])
def test_backward_validation_errors(L, no_gpu, fn):
    def call(q=QA, k=KA, v=VA, o=OA, lse=LA, do=DOA, dq=DQA, dk=DKA, dv=DVA, **kw):
        a = dict(GOOD, **kw)
        return fn(q, k, v, o, lse, do, dq, dk, dv, a["B"], a["H"], a["N"], a["d"],
                  a["scale"], a["causal"], None)
    for name in ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv"):
        assert call(**{name: 0}) == fa.FA_ERR_NULL, name
    for bad in (dict(B=0), dict(H=0), dict(N=0), dict(d=0), dict(N=-5)):
        assert call(**bad) == fa.FA_ERR_SHAPE, bad
    for s in (float("nan"), float("inf")):
        assert call(scale=s) == fa.FA_ERR_SHAPE
    for d in (1, 32, 63, 65, 96, 127, 129):
        assert call(d=d) == fa.FA_ERR_UNSUPPORTED, d
    assert call(N=2 ** 24, d=128) == fa.FA_ERR_SHAPE
    assert call(B=2 ** 20, H=2 ** 10, N=1024) == fa.FA_ERR_SHAPE
    for name in ("q", "do", "dq", "dk", "dv"):
        assert call(**{name: DQA + 0x40000008}) == fa.FA_ERR_ALIGN, name
    assert call(lse=LA + 2) == fa.FA_ERR_ALIGN
    tbytes = GOOD["B"] * GOOD["H"] * GOOD["N"] * GOOD["d"] * 2
    # outputs overlapping an input or each other
    assert call(dq=QA) == fa.FA_ERR_ALIAS
    assert call(dk=OA + 16 * ((tbytes - 16) // 16)) == fa.FA_ERR_ALIAS
    assert call(dv=DOA) == fa.FA_ERR_ALIAS
    assert call(dv=LA - 16 * ((tbytes - 16) // 16)) == fa.FA_ERR_ALIAS
    assert call(dk=DQA) == fa.FA_ERR_ALIAS
    assert call(dv=DKA + 16) == fa.FA_ERR_ALIAS
    # inputs may alias each other
    assert call(k=QA, v=QA, dq=QA) == fa.FA_ERR_ALIAS
    assert fa.fa_last_hip_error() == 0


WSA = 0x7f0000000000 + 9 * 0x100000000  # fake workspace address


@pytest.mark.parametrize("which", ["splitkv", "fa1"])
def test_workspace_pass_validation(L, no_gpu, which):
    G = dict(GOOD, d=64)
    if which == "splitkv":
        size = lambda **kw: fa.fa_fwd_splitkv_workspace_size(  # noqa: E731
            *(dict(G, **kw)[x] for x in ("B", "H", "N", "d")), kw.get("ns", 4))

        def call(ws=WSA, nbytes=None, ns=4, dtype=fa.FA_DTYPE_BF16, o=OA, lse=LA, **kw):
            a = dict(G, **kw)
            nb = size(ns=ns) if nbytes is None else nbytes
            return fa.fa_fwd_splitkv(QA, KA, VA, o, lse, ws, nb, a["B"], a["H"], a["N"],
                                     a["d"], a["scale"], a["causal"], ns, dtype, None)
    else:
        size = lambda **kw: fa.fa_fwd_fa1_workspace_size(  # noqa: E731
            *(dict(G, **kw)[x] for x in ("B", "H", "N", "d")))

        def call(ws=WSA, nbytes=None, ns=None, dtype=fa.FA_DTYPE_BF16, o=OA, lse=LA, **kw):
            a = dict(G, **kw)
            nb = size() if nbytes is None else nbytes
            return fa.fa_fwd_fa1(QA, KA, VA, o, lse, ws, nb, a["B"], a["H"], a["N"], a["d"],
                                 a["scale"], a["causal"], dtype, None)
    rows = G["B"] * G["H"] * G["N"]
    assert size() >= rows * G["d"] * 4
    assert size() % 256 == 0
    assert call(ws=0) == fa.FA_ERR_NULL
    assert call(nbytes=size() - 1) == fa.FA_ERR_SHAPE
    assert call(ws=WSA + 16) == fa.FA_ERR_ALIGN
    assert call(ws=QA) == fa.FA_ERR_ALIAS
    assert call(ws=LA - 256) == fa.FA_ERR_ALIAS
    assert call(scale=0.0) == fa.FA_ERR_SHAPE
    assert call(d=96, nbytes=1 << 30) == fa.FA_ERR_UNSUPPORTED
    assert call(d=32, nbytes=1 << 30) == fa.FA_ERR_UNSUPPORTED
    assert call(dtype=2) == fa.FA_ERR_UNSUPPORTED
    assert call(o=0) == fa.FA_ERR_NULL
    assert call(o=QA) == fa.FA_ERR_ALIAS
    assert call(N=0, nbytes=1 << 30) == fa.FA_ERR_SHAPE
    if which == "splitkv":
        assert fa.fa_fwd_splitkv_workspace_size(1, 1, 100, 64, 0) == 0
        assert fa.fa_fwd_splitkv_workspace_size(1, 1, 100, 64, fa.FA_MAX_SPLITS + 1) == 0
        assert call(ns=0, nbytes=1 << 30) == fa.FA_ERR_SHAPE
        assert call(ns=fa.FA_MAX_SPLITS + 1, nbytes=1 << 30) == fa.FA_ERR_SHAPE
        # keys per split are a multiple of the 128-query tile: N = 300 with 8 requested
        # splits runs 3 (128 keys each), N = 1000 with 8 runs 8
        per_split = lambda n: n * 64 * 4 + n * 4  # noqa: E731
        assert 3 * per_split(300) <= fa.fa_fwd_splitkv_workspace_size(1, 1, 300, 64, 8) \
            <= 3 * per_split(300) + 512
        assert 8 * per_split(1000) <= fa.fa_fwd_splitkv_workspace_size(1, 1, 1000, 64, 8) \
            <= 8 * per_split(1000) + 512
        # at d = 128 the tile is the wide kernel's 256 rows: N = 300 with 8 requested splits
        # runs 2 (256 keys each), N = 1000 with 8 runs 4
        per_split128 = lambda n: n * 128 * 4 + n * 4  # noqa: E731
        assert 2 * per_split128(300) <= fa.fa_fwd_splitkv_workspace_size(1, 1, 300, 128, 8) \
            <= 2 * per_split128(300) + 512
        assert 4 * per_split128(1000) <= fa.fa_fwd_splitkv_workspace_size(1, 1, 1000, 128, 8) \
            <= 4 * per_split128(1000) + 512
    assert fa.fa_last_hip_error() == 0


def test_static_scratch_splitkv_validation(L, no_gpu):
    """fa_fwd_splitkv_static refuses, before any HIP call, everything fa_fwd_splitkv
    refuses apart from the workspace checks, and partials larger than its static scratch
    (FA_ERR_SCRATCH)."""
    G = dict(GOOD, d=64)

    def call(ns=4, dtype=fa.FA_DTYPE_BF16, o=OA, lse=LA, **kw):
        a = dict(G, **kw)
        return fa.fa_fwd_splitkv_static(QA, KA, VA, o, lse, a["B"], a["H"], a["N"], a["d"],
                                        a["scale"], a["causal"], ns, dtype, None)

    assert call(o=0) == fa.FA_ERR_NULL
    assert call(o=QA) == fa.FA_ERR_ALIAS
    assert call(N=0) == fa.FA_ERR_SHAPE
    assert call(scale=0.0) == fa.FA_ERR_SHAPE
    assert call(ns=0) == fa.FA_ERR_SHAPE
    assert call(ns=fa.FA_MAX_SPLITS + 1) == fa.FA_ERR_SHAPE
    assert call(d=96) == fa.FA_ERR_UNSUPPORTED
    assert call(dtype=2) == fa.FA_ERR_UNSUPPORTED
    # 4 splits of B*H*N = 2^20 rows at d = 128 need 2 GiB of partials
    big = dict(B=1, H=64, N=16384, d=128)
    assert fa.fa_fwd_splitkv_workspace_size(*big.values(), 4) > fa.FA_STATIC_SCRATCH_BYTES
    assert call(**big) == fa.FA_ERR_SCRATCH
    assert fa.fa_strerror(fa.FA_ERR_SCRATCH) != "unknown status"
    assert fa.fa_last_hip_error() == 0


def test_fp8_validation(L, no_gpu):
    def call(q=QA, k=KA, v=VA, o=OA, lse=LA, qs=0.01, ks=0.01, vs=0.01, **kw):
        a = dict(GOOD, **kw)
        return fa.fa_fwd_fp8(q, k, v, qs, ks, vs, o, lse, a["B"], a["H"], a["N"], a["d"],
                             a["scale"], a["causal"], None)
    for name in ("q", "k", "v", "o", "lse"):
        assert call(**{name: 0}) == fa.FA_ERR_NULL, name
    for bad in (dict(B=0), dict(N=0), dict(H=-1)):
        assert call(**bad) == fa.FA_ERR_SHAPE, bad
    for kw in (dict(scale=0.0), dict(qs=0.0), dict(ks=float("nan")), dict(vs=float("inf")),
               dict(scale=float("inf"))):
        assert call(**kw) == fa.FA_ERR_SHAPE, kw
    for d in (1, 32, 96, 127, 129):
        assert call(d=d) == fa.FA_ERR_UNSUPPORTED, d
    assert call(q=QA + 8) == fa.FA_ERR_ALIGN
    assert call(lse=LA + 1) == fa.FA_ERR_ALIGN
    # o holds 2-byte elements over 1-byte inputs: its second half overlapping v is caught
    ib = GOOD["B"] * GOOD["H"] * GOOD["N"] * GOOD["d"]
    assert call(o=VA - ib) == fa.FA_ERR_ALIAS
    assert call(lse=OA + 2 * ib - 16) == fa.FA_ERR_ALIAS
    assert call(o=QA) == fa.FA_ERR_ALIAS
    assert fa.fa_last_hip_error() == 0


def test_inputs_may_alias_each_other(L, no_gpu):
    """q, k, v are read-only and may share memory; that is not an alias error.
    Checked through validation only: with o aliasing q the call must still
    fail as ALIAS, proving the q/k/v equality did not short-circuit checks."""
    assert _call(fa.fa_fwd, k=QA, v=QA, o=QA) == fa.FA_ERR_ALIAS


def test_forward_rejects_bad_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 1, 8, 8, dtype=torch.float32)
    with pytest.raises(ValueError):
        fa.forward(x, x, x)
    y = torch.zeros(1, 1, 8, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.forward(y, y, y)  # CPU tensors are refused before any library call
    with pytest.raises(ValueError):
        fa.forward(y, y, torch.zeros(1, 1, 8, 4, dtype=torch.bfloat16))


def test_build_compiles_every_source():
    # the library is linked from one object per HIP source: a source missing from the
    # build list would leave its entry points or kernels out of libfa.so
    from io_aware_exact_fa2_amd import build
    csrc = os.path.join(ROOT, "io_aware_exact_fa2_amd", "csrc")
    hip = {f for f in os.listdir(csrc) if f.endswith(".hip")}
    assert set(build.SOURCES) == hip
    for own in build.SOURCES.values():
        assert all(isinstance(f, str) for f in own)
