"""The C-ABI library without a GPU: it loads, exports every declared symbol,
reports its plan constants, and rejects bad arguments before any device work
(every call here returns from host-side validation; no kernel is launched)."""

import ctypes
import os
import re
import subprocess

import pytest

import oracle
import moe_grouped_precision_amd as w4a8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a8.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a8_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(w4a8.lib_path()):
        pytest.fail("libw4a8.so is not built (python -m moe_grouped_precision_amd.build)")
    return w4a8.load(require_device=False)


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert "w4a8_grouped_gemm" in names and "w4a8_plan" in names and "w4a8_route_prep" in names
    out = subprocess.run(["nm", "-D", "--defined-only", w4a8.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (w4a8_\w+)", out))
    assert set(names) <= exported, set(names) - exported
    for n in names:
        assert hasattr(lib, n)


def test_plan_params_match_oracle(lib):
    assert w4a8.plan_params() == oracle.PLAN_PARAMS


def test_plan_bytes_bound(lib):
    from oracle import plan as P
    import numpy as np
    rng = np.random.default_rng(0)
    for _ in range(200):
        E = int(rng.integers(1, 64))
        counts = rng.integers(0, 600, size=E) * (rng.random(E) < 0.7)
        off = np.concatenate([[0], np.cumsum(counts)])
        need = len(oracle.plan_ref(off, E, 256)) * 4
        assert w4a8.plan_bytes(E, int(off[-1])) >= need
    for E in (2048, 8192, 65536):   # the plan serves the route prep's experts
        counts = rng.integers(0, 40, size=E) * (rng.random(E) < 0.3)
        off = np.concatenate([[0], np.cumsum(counts)])
        assert w4a8.plan_bytes(E, int(off[-1])) >= len(oracle.plan_ref(off, E, 256)) * 4
    assert w4a8.plan_bytes(0, 10) == 0 and w4a8.plan_bytes(65537, 10) == 0
    assert w4a8.plan_bytes(4, -1) == 0
    assert w4a8.plan_bytes(8, 0) == P.HEADER_WORDS * 4


def test_status_strings(lib):
    assert lib.w4a8_status_string(0) == b"W4A8_OK"
    assert lib.w4a8_status_string(4) == b"W4A8_ERR_ALIGN"
    assert lib.w4a8_status_string(99) == b"W4A8_UNKNOWN_STATUS"
    assert lib.w4a8_plan_params(None, 7) == -1


P16 = ctypes.c_void_p(1 << 20)   # a 16-byte aligned, never dereferenced address
P4 = ctypes.c_void_p((1 << 20) + 4)
NUL = ctypes.c_void_p(0)


@pytest.mark.parametrize("args,status", [
    ((P16, P16, 0, P16, P16, P16, 0, 256, 512, P16, NUL), 2),      # E = 0
    ((P16, P16, 0, P16, P16, P16, 2049, 256, 512, P16, NUL), 2),   # E too large
    ((P16, P16, 0, P16, P16, P16, 8, 256, 500, P16, NUL), 2),      # K % 128
    ((P16, P16, 0, P16, P16, P16, 8, 256, (1 << 20) + 128, P16, NUL), 2),  # K above the limit
    ((P16, P16, 0, P16, P16, P16, 8, 48, 512, P16, NUL), 2),       # N % 32
    ((P16, P16, 0, P16, P16, P16, 8, (1 << 24) + 32, 512, P16, NUL), 2),  # N above the limit
    ((P16, P16, 2, P16, P16, P16, 8, 256, 512, P16, NUL), 3),      # bad layout
    ((NUL, P16, 0, P16, P16, P16, 8, 256, 512, P16, NUL), 1),      # null A
    ((P16, P16, 0, P16, P16, P16, 8, 256, 512, NUL, NUL), 1),      # null C
    ((P4, P16, 0, P16, P16, P16, 8, 256, 512, P16, NUL), 4),       # misaligned A
    ((P16, P16, 0, P16, P16, P16, 8, 256, 512, P4, NUL), 4),       # misaligned C
])
def test_gemm_host_validation(lib, args, status):
    assert lib.w4a8_grouped_gemm(*args) == status
    assert lib.w4a8_last_error() != b""


def test_plan_and_route_host_validation(lib):
    assert lib.w4a8_plan(P16, 8, 256, 512, P16, 16, NUL) == 5        # buffer < header
    assert lib.w4a8_plan(NUL, 8, 256, 512, P16, 1024, NUL) == 1
    assert lib.w4a8_plan(P16, 8, 250, 512, P16, 1024, NUL) == 2
    assert lib.w4a8_route_prep(P16, 4, 2, 0, P16, P16, P16, NUL) == 2
    assert lib.w4a8_route_prep(P16, -1, 2, 8, P16, P16, P16, NUL) == 2
    assert lib.w4a8_route_prep(P16, 4, 2, 8, NUL, P16, P16, NUL) == 1
    assert lib.w4a8_route_prep(ctypes.c_void_p((1 << 20) + 2), 4, 2, 8, P16, P16, P16, NUL) == 4
    assert lib.w4a8_route_prep(P16, 4, 2, 65537, P16, P16, P16, NUL) == 2   # above the prep limit
    assert lib.w4a8_plan(P16, 65537, 256, 512, P16, 1024, NUL) == 2
    # the GEMM keeps its own, lower limit (per-expert tables in LDS)
    assert lib.w4a8_grouped_gemm(P16, P16, 0, P16, P16, P16, 4096, 256, 512, P16, NUL) == 2


LDS_160K = 160 * 1024


def test_route_prep_waves_fit():
    """The route prep's LDS fit (MoonEP PR #38, change section): the largest
    wave count from 16 down whose LDS need, (W + 2) * E + 16 int32, fits the
    device's per-workgroup LDS; none -> 0 (the call then reports
    W4A8_ERR_CAPACITY)."""
    def need(E, W):
        return 4 * ((W + 2) * E + 16)
    for E in list(range(1, 300)) + [341, 342, 1024, 2275, 2276, 2409, 2410, 4096, 8192, 13647, 13648, 13649]:
        W = w4a8.route_prep_waves(E, LDS_160K)
        if W:
            assert 1 <= W <= 16 and need(E, W) <= LDS_160K
            assert W == 16 or need(E, W + 1) > LDS_160K
        else:
            assert need(E, 1) > LDS_160K
    assert w4a8.route_prep_waves(32, LDS_160K) == 16          # small E keeps the full workgroup
    assert w4a8.route_prep_waves(1024, LDS_160K) == 16
    assert w4a8.route_prep_waves(6144, LDS_160K) == 4
    assert w4a8.route_prep_waves(13648, LDS_160K) == 1        # the largest E one wave serves
    assert w4a8.route_prep_waves(13649, LDS_160K) == 0
    assert w4a8.route_prep_waves(1024, 64 * 1024) == 13       # a 64 KB device
    assert w4a8.route_prep_waves(0, LDS_160K) == 0 and w4a8.route_prep_waves(65537, 1 << 30) == 0


def test_quantize_gather_host_validation(lib):
    q = lib.w4a8_quantize_gather
    assert q(P16, 4, 512, P16, 0, 8, P16, P16, 0, NUL) == 2        # top_k = 0
    assert q(P16, -1, 512, P16, 2, 8, P16, P16, 0, NUL) == 2       # T < 0
    assert q(P16, 4, 500, P16, 2, 8, P16, P16, 0, NUL) == 2        # K % 128
    assert q(P16, 4, 512, P16, 2, -1, P16, P16, 0, NUL) == 2       # R < 0
    assert q(P16, 4, 512, P16, 2, 8, P16, P16, 2, NUL) == 3        # bad layout
    assert q(NUL, 4, 512, P16, 2, 8, P16, P16, 0, NUL) == 1        # null x
    assert q(P16, 4, 512, P16, 2, 8, NUL, P16, 0, NUL) == 1        # null A
    assert q(P4, 4, 512, P16, 2, 8, P16, P16, 0, NUL) == 4         # misaligned x
    assert q(P16, 4, 512, P16, 2, 8, P4, P16, 0, NUL) == 4         # misaligned A
    assert lib.w4a8_last_error() != b""


def test_combine_host_validation(lib):
    c = lib.w4a8_combine
    assert c(P16, 8, 64, P16, P16, 4, 0, P16, NUL) == 2      # top_k = 0
    assert c(P16, 8, 60, P16, P16, 4, 2, P16, NUL) == 2      # N % 8
    assert c(P16, -1, 64, P16, P16, 4, 2, P16, NUL) == 2     # R < 0
    assert c(P16, 8, 64, NUL, P16, 4, 2, P16, NUL) == 1      # null row map
    assert c(P16, 8, 64, P16, P16, 4, 2, NUL, NUL) == 1      # null out
    assert c(P4, 8, 64, P16, P16, 4, 2, P16, NUL) == 4       # misaligned C
    assert lib.w4a8_last_error() != b""


def test_swiglu_quant_host_validation(lib):
    f = lib.w4a8_swiglu_quant
    assert f(P16, -1, 256, P16, P16, 0, NUL) == 2       # R < 0
    assert f(P16, 8, 200, P16, P16, 0, NUL) == 2        # I % 128
    assert f(P16, 8, 256, P16, P16, 2, NUL) == 3        # bad layout
    assert f(NUL, 8, 256, P16, P16, 0, NUL) == 1        # null C
    assert f(P4, 8, 256, P16, P16, 0, NUL) == 4         # misaligned C
    assert lib.w4a8_last_error() != b""


def test_grouped_gemm_planned_host_validation(lib):
    f = lib.w4a8_grouped_gemm_planned
    ok = [P16, P16, 0, P16, P16, P16, 8, 256, 512, P16, 1024, P16, NUL]

    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a6=0) == 2 and call(a6=65537) == 2       # E outside [1, 65536]
    assert call(a8=500) == 2 and call(a7=48) == 2        # K % 128, N % 32
    assert call(a2=2) == 3                               # bad layout
    assert call(a9=NUL) == 1 and call(a11=NUL) == 1      # null plan, null C
    assert call(a9=ctypes.c_void_p((1 << 20) + 2)) == 4  # misaligned plan
    assert call(a10=16) == 5                             # plan buffer below the header
    assert lib.w4a8_last_error() != b""


def test_grouped_gemm_swiglu_host_validation(lib):
    f = lib.w4a8_grouped_gemm_swiglu
    ok = (P16, P16, 0, P16, P16, P16, 8, 256, 512, P16, P16, 0, NUL)

    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a6=0) == 2                      # E = 0
    assert call(a7=200) == 2                    # I % 128
    assert call(a7=0) == 2                      # I = 0
    assert call(a8=500) == 2                    # K % 128
    assert call(a7=1 << 16, a8=1 << 16) == 2    # one expert's weights past 2^31 bytes
    assert call(a2=2) == 3 and call(a11=2) == 3  # bad layouts
    assert call(a9=NUL) == 1 and call(a10=NUL) == 1 and call(a3=NUL) == 1
    assert call(a9=P4) == 4 and call(a3=P4) == 4 and call(a0=P4) == 4
    assert lib.w4a8_last_error() != b""


def test_grouped_gemm_a16_host_validation(lib):
    f = lib.w4a8_grouped_gemm_a16
    ok = (P16, P16, P16, 0, NUL, P16, 8, 256, 512, P16, NUL)

    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a6=0) == 2                       # E = 0
    assert call(a6=(1 << 16) + 1) == 2           # E past the limit
    assert call(a7=40) == 2 and call(a7=0) == 2  # N % 16, N = 0
    assert call(a8=500) == 2 and call(a8=0) == 2  # K % 128, K = 0
    assert call(a3=2) == 3 and call(a3=-1) == 3  # unknown weight-scale format
    assert call(a0=NUL) == 1 and call(a1=NUL) == 1 and call(a2=NUL) == 1 and call(a5=NUL) == 1 \
        and call(a9=NUL) == 1
    assert call(a0=P4) == 4 and call(a1=P4) == 4 and call(a9=P4) == 4 and call(a4=ctypes.c_void_p(0x1002)) == 4
    assert lib.w4a8_last_error() != b""


def test_binding_fails_loudly_without_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    with pytest.raises(RuntimeError):
        w4a8.load(require_device=True)


def test_probe_library_exports_and_host_checks():
    path = os.path.join(ROOT, "moe_grouped_precision_amd", "libw4a8_probe.so")
    if not os.path.exists(path):
        pytest.skip("probe library not built")
    probe = ctypes.CDLL(path)
    for name in ("w4a8_probe_mfma", "w4a8_probe_mfma_data", "w4a8_probe_mfma_promote", "w4a8_probe_read"):
        assert hasattr(probe, name)
    probe.w4a8_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_void_p]
    probe.w4a8_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_void_p]
    # argument errors are reported before anything is launched
    assert probe.w4a8_probe_mfma(4, 0, 16, 8, None, None) == 1
    assert probe.w4a8_probe_mfma(4, 0, 0, 8, P16, None) == 2
    assert probe.w4a8_probe_mfma(1, 2, 16, 8, P16, None) == 2
    probe.w4a8_probe_mfma_data.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert probe.w4a8_probe_mfma_data(4, 0, 16, 8, None, P16, None) == 1
    assert probe.w4a8_probe_mfma_data(4, 0, 0, 8, P16, P16, None) == 2
    assert probe.w4a8_probe_read(None, 1024, 8, P16, None) == 1
    assert probe.w4a8_probe_read(P16, 1000, 8, P16, None) == 2
    assert probe.w4a8_probe_read(P4, 1024, 8, P16, None) == 4
