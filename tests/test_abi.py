"""The C-ABI library on the CPU: it loads, exports every entry point that
include/crisp.h declares, and its host-side validation rejects bad arguments
before anything is launched (no GPU work is requested here)."""
import ctypes as C
import os
import re

import pytest

import dynamic_sparse_prefill_amd as dsp
from dynamic_sparse_prefill_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions(header="crisp.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(crisp_[a-z0-9_]+)\s*\(", src)))


def test_header_and_exports_agree():
    names = declared_functions()
    assert set(names) == set(api.EXPORTS)
    L = dsp.lib()
    for n in names:
        assert hasattr(L, n), n


def test_probe_header_and_exports_agree():
    names = declared_functions("crisp_probe.h")
    assert names == ["crisp_probe_mfma_bf16", "crisp_probe_mfma_bf16_data"]
    L = api.probe_lib()
    for n in names:
        assert hasattr(L, n), n
    # host-side validation: nothing is launched for invalid arguments
    assert L.crisp_probe_mfma_bf16(None, 1, 1, None) == -1
    assert L.crisp_probe_mfma_bf16(C.c_void_p(16), 0, 1, None) == -1
    assert L.crisp_probe_mfma_bf16(C.c_void_p(16), 1, 0, None) == -1
    assert L.crisp_probe_mfma_bf16_data(None, 1, 2, None) == -1
    assert L.crisp_probe_mfma_bf16_data(C.c_void_p(16), 1, 3, None) == -1   # odd iteration count
    assert L.crisp_probe_mfma_bf16_data(C.c_void_p(16), 0, 2, None) == -1


def _shape(n=4096, hq=4, hkv=2, d=128, dtype=0):
    return api.CrispShape(n, hq, hkv, d, dtype, n * d, d, n * d, d, n * d, d, n * d, d)


def test_workspace_and_capacity_queries():
    s = _shape()
    p = dsp.CrispParams()
    nb = 4096 // 128
    assert dsp.col_capacity(s) == 4 * nb * (nb + 1) // 2
    ws = dsp.select_workspace_bytes(s, p)
    assert ws > 4 * nb * (nb + 1) // 2 * 4          # holds the pooled matrix of every head
    assert dsp.attn_workspace_bytes(s) == 2 * 4096 * 128 * 2 + 256
    assert dsp.workspace_bytes(s, p) == ws + dsp.attn_workspace_bytes(s)
    # invalid shapes and parameters report zero
    assert dsp.select_workspace_bytes(_shape(d=64), p) == 0
    assert dsp.col_capacity(_shape(n=1000)) == 0
    huge = _shape()
    huge.sk_n = (1 << 22) + 8                         # token stride beyond the supported range
    assert dsp.select_workspace_bytes(huge, p) == 0
    bad = dsp.CrispParams(gamma=0.0)
    assert dsp.workspace_bytes(s, bad) == 0


@pytest.mark.parametrize("mut,status", [
    (dict(d=64), -2), (dict(n=1000), -1), (dict(hq=3, hkv=2), -1), (dict(dtype=7), -2), (dict(n=0), -1),
])
def test_select_rejects_bad_shapes(mut, status):
    kw = dict(n=4096, hq=4, hkv=2, d=128, dtype=0)
    kw.update(mut)
    s = _shape(**kw)
    sel = api.CrispSelectionC()
    st = dsp.lib().crisp_select(C.byref(s), 16, 16, C.byref(dsp.CrispParams().c()), C.byref(sel), 256, 1 << 30, None)
    assert st == status


@pytest.mark.parametrize("mut", [dict(gamma=1.5), dict(gamma=0.0), dict(tau=-1.0), dict(alpha=float("nan")),
                                 dict(sink=-1), dict(min_blocks=-2), dict(flags=8), dict(flags=6),
                                 dict(local=10 ** 9)])
def test_select_rejects_bad_params(mut):
    p = dsp.CrispParams(**mut)
    s = _shape()
    sel = api.CrispSelectionC(16, 16, 16, 16, 1 << 40)
    st = dsp.lib().crisp_select(C.byref(s), 16, 16, C.byref(p.c()), C.byref(sel), 256, 1 << 40, None)
    assert st == -1


@pytest.mark.parametrize("flags", [1, 2, 4, 3, 5])
def test_variant_flags_are_accepted(flags):
    s = _shape()
    assert dsp.select_workspace_bytes(s, dsp.CrispParams(flags=flags)) > 0


def test_select_rejects_block_other_than_128_and_small_buffers():
    s = _shape()
    sel = api.CrispSelectionC(16, 16, 16, 16, 1 << 40)
    st = dsp.lib().crisp_select(C.byref(s), 16, 16, C.byref(dsp.CrispParams(block=64).c()), C.byref(sel), 256,
                                1 << 40, None)
    assert st == -2
    small = api.CrispSelectionC(16, 16, 16, 16, 10)
    st = dsp.lib().crisp_select(C.byref(s), 16, 16, C.byref(dsp.CrispParams().c()), C.byref(small), 256, 1 << 40, None)
    assert st == -3
    st = dsp.lib().crisp_select(C.byref(s), 16, 16, C.byref(dsp.CrispParams().c()), C.byref(sel), 256, 1024, None)
    assert st == -3
    st = dsp.lib().crisp_select(C.byref(s), 0, 16, C.byref(dsp.CrispParams().c()), C.byref(sel), 256, 1 << 40, None)
    assert st == -1
    st = dsp.lib().crisp_select(C.byref(s), 8, 16, C.byref(dsp.CrispParams().c()), C.byref(sel), 256, 1 << 40, None)
    assert st == -1                                          # misaligned pointer


def test_attention_entry_points_validate():
    s = _shape()
    L = dsp.lib()
    assert L.crisp_dense_attn(C.byref(s), 16, 16, 16, 0, 256, 1 << 30, None) == -1
    assert L.crisp_dense_attn(C.byref(s), 16, 16, 16, 16, 256, 10, None) == -3
    bad = _shape()
    bad.sk_n = 100                                          # not a multiple of 8
    assert L.crisp_dense_attn(C.byref(bad), 16, 16, 16, 16, 256, 1 << 30, None) == -1
    assert L.crisp_sparse_attn(C.byref(s), 16, 16, 16, None, 16, 256, 1 << 30, None) == -1
    assert L.crisp_prefill(C.byref(s), 16, 16, 16, C.byref(dsp.CrispParams().c()), None, 16, 256, 1 << 40,
                           None) == -1
    assert dsp.api.status_string(-3).startswith("workspace")


def test_varlen_queries_and_validation():
    L = dsp.lib()
    n = 4096 + 1024 + 256
    s = _shape(n=n)
    p = dsp.CrispParams()
    cu = [0, 4096, 5120, n]
    nbs = [32, 8, 2]
    assert dsp.varlen_col_capacity(s, cu) == sum(4 * nb * (nb + 1) // 2 for nb in nbs)
    assert dsp.varlen_workspace_bytes(s, cu, p) > dsp.attn_workspace_bytes(s)
    for bad in ([0, 4096, n - 64, n], [64, 4096, n], [0, 4096, 4096, n], [0, 4096, 5120, n + 128]):
        assert dsp.varlen_col_capacity(s, bad) == 0
    arr = (C.c_int64 * 4)(*cu)
    sel = api.CrispSelectionC(16, 16, 16, 16, 1 << 40)
    args = (16, 16, 16, C.byref(p.c()), C.byref(sel), 16, 256, 1 << 40, None)
    assert L.crisp_prefill_varlen(C.byref(s), 0, arr, *args) == -1
    assert L.crisp_prefill_varlen(C.byref(s), 3, None, *args) == -1
    big = (C.c_int64 * 66)(*([128 * i for i in range(65)] + [0]))
    s65 = _shape(n=128 * 65)
    assert L.crisp_prefill_varlen(C.byref(s65), 65, big, *args) == -2
    small = api.CrispSelectionC(16, 16, 16, 16, 10)
    assert L.crisp_prefill_varlen(C.byref(s), 3, arr, 16, 16, 16, C.byref(p.c()), C.byref(small), 16, 256,
                                  1 << 40, None) == -3


def test_noalloc_entry_point_rejects_before_any_launch():
    """The allocation-free prefill checks everything on the host first: a
    problem whose workspace exceeds the fixed scratch is CRISP_E_TOO_LARGE
    (-5), missing outputs are CRISP_E_ARG, a short list buffer
    CRISP_E_WORKSPACE; none of these touches the device."""
    L = dsp.lib()
    cap = dsp.noalloc_scratch_bytes()
    assert cap == 128 << 20
    p = dsp.CrispParams()
    sel = api.CrispSelectionC(16, 16, 16, 16, 1 << 40)
    small = _shape(n=4096, hq=4, hkv=2)
    assert dsp.workspace_bytes(small, p) <= cap
    big = _shape(n=65536, hq=32, hkv=8)
    assert dsp.workspace_bytes(big, p) > cap
    assert L.crisp_prefill_noalloc(C.byref(big), 16, 16, 16, C.byref(p.c()), C.byref(sel), 16, None) == -5
    assert dsp.api.status_string(-5).startswith("problem needs more workspace")
    assert L.crisp_prefill_noalloc(C.byref(small), 16, 16, 16, C.byref(p.c()), None, 16, None) == -1
    assert L.crisp_prefill_noalloc(C.byref(small), 16, 16, 0, C.byref(p.c()), C.byref(sel), 16, None) == -1
    short = api.CrispSelectionC(16, 16, 16, 16, 10)
    assert L.crisp_prefill_noalloc(C.byref(small), 16, 16, 16, C.byref(p.c()), C.byref(short), 16, None) == -3
    assert L.crisp_prefill_noalloc(C.byref(_shape(d=64)), 16, 16, 16, C.byref(p.c()), C.byref(sel), 16, None) == -2
