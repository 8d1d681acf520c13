"""Thin ctypes binding over libcrisp.so.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (include/crisp.h).  PyTorch provides device memory
and the current stream.  There is no fallback: if the library is missing or a
call fails, an exception is raised.

Tensor layout: q, o [hq, n, 128]; k, v [hkv, n, 128]; dtype torch.bfloat16 or
torch.float32; the last axis contiguous; any head / token strides that are
multiples of 8 elements, token strides at most 2^22 elements.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass, field

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcrisp.so")
PROBE_LIB_PATH = os.path.join(HERE, "libcrisp_probe.so")   # attainable-peak probe (include/crisp_probe.h)

BLOCK = 128
BF16, FP32 = 0, 1
# crisp_params.flags (include/crisp.h): variants the pages compare CRISP against
FLAG_ROUTE_JSD, FLAG_VS_MEDIAN, FLAG_VS_COVERAGE = 1, 2, 4

EXPORTS = ("crisp_select_workspace_bytes", "crisp_attn_workspace_bytes", "crisp_workspace_bytes",
           "crisp_col_capacity", "crisp_select", "crisp_sparse_attn", "crisp_dense_attn",
           "crisp_prefill", "crisp_status_string", "crisp_varlen_col_capacity", "crisp_varlen_workspace_bytes",
           "crisp_prefill_varlen", "crisp_noalloc_scratch_bytes", "crisp_prefill_noalloc")


class CrispShape(C.Structure):
    _fields_ = [("n", C.c_int64), ("hq", C.c_int32), ("hkv", C.c_int32), ("d", C.c_int32), ("dtype", C.c_int32),
                ("sq_h", C.c_int64), ("sq_n", C.c_int64), ("sk_h", C.c_int64), ("sk_n", C.c_int64),
                ("sv_h", C.c_int64), ("sv_n", C.c_int64), ("so_h", C.c_int64), ("so_n", C.c_int64)]


class CrispParamsC(C.Structure):
    _fields_ = [("block", C.c_int32), ("sink", C.c_int32), ("local", C.c_int32), ("tau", C.c_float),
                ("alpha", C.c_float), ("gamma", C.c_float), ("min_blocks", C.c_int32),
                ("dense_below_n", C.c_int32), ("flags", C.c_int32)]


class CrispSelectionC(C.Structure):
    _fields_ = [("route", C.c_void_p), ("c_struct", C.c_void_p), ("row_ptr", C.c_void_p), ("col_idx", C.c_void_p),
                ("col_capacity", C.c_int64), ("pv", C.c_void_p), ("ps", C.c_void_p), ("sv", C.c_void_p),
                ("nv", C.c_void_p), ("ss", C.c_void_p), ("ns", C.c_void_p), ("pe_prob", C.c_void_p),
                ("jsd", C.c_void_p), ("abar", C.c_void_p)]


class CrispError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


_LIB = None


_PROBE = None


def probe_lib() -> C.CDLL:
    """Load libcrisp_probe.so, the MFMA peak probe the benchmark times (raises if not built)."""
    global _PROBE
    if _PROBE is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise RuntimeError(f"{PROBE_LIB_PATH} is missing: build it with dynamic_sparse_prefill_amd.build.build()")
        L = C.CDLL(PROBE_LIB_PATH)
        L.crisp_probe_mfma_bf16.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_void_p]
        L.crisp_probe_mfma_bf16.restype = C.c_int
        L.crisp_probe_mfma_bf16_data.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_void_p]
        L.crisp_probe_mfma_bf16_data.restype = C.c_int
        _PROBE = L
    return _PROBE


def lib() -> C.CDLL:
    """Load libcrisp.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with dynamic_sparse_prefill_amd.build.build()")
        L = C.CDLL(LIB_PATH)
        vp, sp, pp, selp = C.c_void_p, C.POINTER(CrispShape), C.POINTER(CrispParamsC), C.POINTER(CrispSelectionC)
        L.crisp_select_workspace_bytes.argtypes = [sp, pp]
        L.crisp_select_workspace_bytes.restype = C.c_size_t
        L.crisp_attn_workspace_bytes.argtypes = [sp]
        L.crisp_attn_workspace_bytes.restype = C.c_size_t
        L.crisp_workspace_bytes.argtypes = [sp, pp]
        L.crisp_workspace_bytes.restype = C.c_size_t
        L.crisp_col_capacity.argtypes = [sp]
        L.crisp_col_capacity.restype = C.c_int64
        L.crisp_select.argtypes = [sp, vp, vp, pp, selp, vp, C.c_size_t, vp]
        L.crisp_sparse_attn.argtypes = [sp, vp, vp, vp, selp, vp, vp, C.c_size_t, vp]
        L.crisp_dense_attn.argtypes = [sp, vp, vp, vp, vp, vp, C.c_size_t, vp]
        L.crisp_prefill.argtypes = [sp, vp, vp, vp, pp, selp, vp, vp, C.c_size_t, vp]
        for f in ("crisp_select", "crisp_sparse_attn", "crisp_dense_attn", "crisp_prefill"):
            getattr(L, f).restype = C.c_int
        L.crisp_status_string.argtypes = [C.c_int]
        L.crisp_status_string.restype = C.c_char_p
        i64p = C.POINTER(C.c_int64)
        L.crisp_varlen_col_capacity.argtypes = [sp, C.c_int32, i64p]
        L.crisp_varlen_col_capacity.restype = C.c_int64
        L.crisp_varlen_workspace_bytes.argtypes = [sp, C.c_int32, i64p, pp]
        L.crisp_varlen_workspace_bytes.restype = C.c_size_t
        L.crisp_prefill_varlen.argtypes = [sp, C.c_int32, i64p, vp, vp, vp, pp, selp, vp, vp, C.c_size_t, vp]
        L.crisp_prefill_varlen.restype = C.c_int
        L.crisp_noalloc_scratch_bytes.argtypes = []
        L.crisp_noalloc_scratch_bytes.restype = C.c_size_t
        L.crisp_prefill_noalloc.argtypes = [sp, vp, vp, vp, pp, selp, vp, vp]
        L.crisp_prefill_noalloc.restype = C.c_int
        _LIB = L
    return _LIB


def status_string(status: int) -> str:
    return lib().crisp_status_string(status).decode()


# ------------------------------------------------------------------ parameters and results

@dataclass
class CrispParams:
    """Selection parameters; defaults are the acceptance configuration (tau 0.3,
    alpha 1, gamma 0.95, 128-token sink and recency windows)."""
    block: int = BLOCK
    sink: int = 128
    local: int = 128
    tau: float = 0.3
    alpha: float = 1.0
    gamma: float = 0.95
    min_blocks: int = 0
    dense_below_n: int = 0
    flags: int = 0

    def c(self) -> CrispParamsC:
        return CrispParamsC(self.block, self.sink, self.local, self.tau, self.alpha, self.gamma,
                            self.min_blocks, self.dense_below_n, self.flags)


@dataclass
class Selection:
    route: torch.Tensor           # [hq] int32: 1 VS, 0 PE, -1 dense path
    c_struct: torch.Tensor        # [hq] float32
    row_ptr: torch.Tensor         # [hq*nb + 1] int32
    col_idx: torch.Tensor         # [capacity] int32
    pv: torch.Tensor | None = None
    ps: torch.Tensor | None = None
    sv: torch.Tensor | None = None
    nv: torch.Tensor | None = None
    ss: torch.Tensor | None = None
    ns: torch.Tensor | None = None
    pe_prob: torch.Tensor | None = None
    jsd: torch.Tensor | None = None   # [hq] float64, written with FLAG_ROUTE_JSD
    abar: torch.Tensor | None = None  # [hq*nb] float32 pooled estimate, written with FLAG_ROUTE_JSD
    extra: dict = field(default_factory=dict)

    def c(self) -> CrispSelectionC:
        p = lambda t: t.data_ptr() if t is not None else None
        return CrispSelectionC(p(self.route), p(self.c_struct), p(self.row_ptr), p(self.col_idx),
                               self.col_idx.numel(), p(self.pv), p(self.ps), p(self.sv), p(self.nv), p(self.ss),
                               p(self.ns), p(self.pe_prob), p(self.jsd), p(self.abar))


# ------------------------------------------------------------------ marshalling

def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(t: torch.Tensor, name: str, dtype) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() != 3 or t.stride(2) != 1:
        raise ValueError(f"{name} must be [heads, n, d] with a contiguous last axis")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")


def make_shape(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor | None = None,
               o: torch.Tensor | None = None) -> CrispShape:
    _check(q, "q", q.dtype)
    _check(k, "k", q.dtype)
    v_ = v if v is not None else k
    o_ = o if o is not None else q
    _check(v_, "v", q.dtype)
    _check(o_, "o", q.dtype)
    hq, n, d = q.shape
    hkv = k.shape[0]
    if k.shape[1] != n or k.shape[2] != d or v_.shape != k.shape or o_.shape != q.shape:
        raise ValueError("inconsistent q / k / v / o shapes")
    return CrispShape(n, hq, hkv, d, _dtype_code(q), q.stride(0), q.stride(1), k.stride(0), k.stride(1),
                      v_.stride(0), v_.stride(1), o_.stride(0), o_.stride(1))


def _stream() -> C.c_void_p:
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _workspace(nbytes: int, device, ws: torch.Tensor | None) -> torch.Tensor:
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def select_workspace_bytes(shape: CrispShape, params: CrispParams) -> int:
    return int(lib().crisp_select_workspace_bytes(C.byref(shape), C.byref(params.c())))


def attn_workspace_bytes(shape: CrispShape) -> int:
    return int(lib().crisp_attn_workspace_bytes(C.byref(shape)))


def workspace_bytes(shape: CrispShape, params: CrispParams) -> int:
    return int(lib().crisp_workspace_bytes(C.byref(shape), C.byref(params.c())))


def col_capacity(shape: CrispShape) -> int:
    return int(lib().crisp_col_capacity(C.byref(shape)))


def new_selection(q: torch.Tensor, k: torch.Tensor, diagnostics: bool = True, pe_prob: bool = False) -> Selection:
    shape = make_shape(q, k)
    hq, n = q.shape[0], q.shape[1]
    nb = n // BLOCK
    dev = q.device
    i32 = dict(dtype=torch.int32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    cap = col_capacity(shape)
    sel = Selection(torch.empty(hq, **i32), torch.empty(hq, **f32), torch.empty(hq * nb + 1, **i32),
                    torch.empty(max(cap, 1), **i32))
    if diagnostics:
        sel.pv, sel.ps = torch.empty(hq * nb, **f32), torch.empty(hq * nb, **f32)
        sel.sv, sel.ss = torch.empty(hq * nb, **i32), torch.empty(hq * nb, **i32)
        sel.nv, sel.ns = torch.empty(hq, **i32), torch.empty(hq, **i32)
        sel.jsd = torch.zeros(hq, dtype=torch.float64, device=dev)
        sel.abar = torch.zeros(hq * nb, **f32)
    if pe_prob:
        sel.pe_prob = torch.empty(hq * nb * (nb + 1) // 2, **f32)
    return sel


# ------------------------------------------------------------------ entry points

def crisp_select(q, k, params: CrispParams | None = None, sel: Selection | None = None, ws=None,
                 diagnostics: bool = True, pe_prob: bool = False) -> Selection:
    params = params or CrispParams()
    shape = make_shape(q, k)
    sel = sel or new_selection(q, k, diagnostics, pe_prob)
    ws = _workspace(select_workspace_bytes(shape, params), q.device, ws)
    c_sel = sel.c()
    st = lib().crisp_select(C.byref(shape), q.data_ptr(), k.data_ptr(), C.byref(params.c()), C.byref(c_sel),
                            ws.data_ptr(), ws.numel(), _stream())
    if st:
        raise CrispError(st, "crisp_select")
    return sel


def crisp_sparse_attn(q, k, v, sel: Selection, o=None, ws=None) -> torch.Tensor:
    o = torch.empty_like(q) if o is None else o
    shape = make_shape(q, k, v, o)
    ws = _workspace(attn_workspace_bytes(shape), q.device, ws)
    c_sel = sel.c()
    st = lib().crisp_sparse_attn(C.byref(shape), q.data_ptr(), k.data_ptr(), v.data_ptr(), C.byref(c_sel),
                                 o.data_ptr(), ws.data_ptr(), ws.numel(), _stream())
    if st:
        raise CrispError(st, "crisp_sparse_attn")
    return o


def crisp_dense_attn(q, k, v, o=None, ws=None) -> torch.Tensor:
    o = torch.empty_like(q) if o is None else o
    shape = make_shape(q, k, v, o)
    ws = _workspace(attn_workspace_bytes(shape), q.device, ws)
    st = lib().crisp_dense_attn(C.byref(shape), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                ws.data_ptr(), ws.numel(), _stream())
    if st:
        raise CrispError(st, "crisp_dense_attn")
    return o


def crisp_prefill(q, k, v, params: CrispParams | None = None, sel: Selection | None = None, o=None, ws=None,
                  diagnostics: bool = True, pe_prob: bool = False):
    params = params or CrispParams()
    o = torch.empty_like(q) if o is None else o
    shape = make_shape(q, k, v, o)
    sel = sel or new_selection(q, k, diagnostics, pe_prob)
    ws = _workspace(workspace_bytes(shape, params), q.device, ws)
    c_sel = sel.c()
    st = lib().crisp_prefill(C.byref(shape), q.data_ptr(), k.data_ptr(), v.data_ptr(), C.byref(params.c()),
                             C.byref(c_sel), o.data_ptr(), ws.data_ptr(), ws.numel(), _stream())
    if st:
        raise CrispError(st, "crisp_prefill")
    return o, sel


def noalloc_scratch_bytes() -> int:
    """Size of the fixed scratch array behind crisp_prefill_noalloc."""
    return int(lib().crisp_noalloc_scratch_bytes())


def crisp_prefill_noalloc(q, k, v, params: CrispParams, sel: Selection, o: torch.Tensor):
    """crisp_prefill with the library's fixed scratch as workspace: the caller
    passes the outputs (sel from new_selection, o like q) and nothing is
    allocated.  Raises CrispError with status CRISP_E_TOO_LARGE (-5) when the
    problem needs more than noalloc_scratch_bytes()."""
    shape = make_shape(q, k, v, o)
    c_sel = sel.c()
    st = lib().crisp_prefill_noalloc(C.byref(shape), q.data_ptr(), k.data_ptr(), v.data_ptr(), C.byref(params.c()),
                                     C.byref(c_sel), o.data_ptr(), _stream())
    if st:
        raise CrispError(st, "crisp_prefill_noalloc")
    return o, sel


# ------------------------------------------------------------------ packed batches (varlen)

def _cu(cu_seqlens):
    cu = [int(x) for x in cu_seqlens]
    return (C.c_int64 * len(cu))(*cu), len(cu) - 1


def varlen_col_capacity(shape: CrispShape, cu_seqlens) -> int:
    arr, nseq = _cu(cu_seqlens)
    return int(lib().crisp_varlen_col_capacity(C.byref(shape), nseq, arr))


def varlen_workspace_bytes(shape: CrispShape, cu_seqlens, params: CrispParams) -> int:
    arr, nseq = _cu(cu_seqlens)
    return int(lib().crisp_varlen_workspace_bytes(C.byref(shape), nseq, arr, C.byref(params.c())))


def new_varlen_selection(q: torch.Tensor, k: torch.Tensor, cu_seqlens, diagnostics: bool = True,
                         pe_prob: bool = False) -> Selection:
    """Buffers for crisp_prefill_varlen: sequence-major (see include/crisp.h)."""
    shape = make_shape(q, k)
    hq = q.shape[0]
    nbs = [(int(b) - int(a)) // BLOCK for a, b in zip(cu_seqlens[:-1], cu_seqlens[1:])]
    nseq = len(nbs)
    rows = hq * sum(nbs)
    dev = q.device
    i32 = dict(dtype=torch.int32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    cap = varlen_col_capacity(shape, cu_seqlens)
    sel = Selection(torch.empty(nseq * hq, **i32), torch.empty(nseq * hq, **f32), torch.empty(rows + nseq, **i32),
                    torch.empty(max(cap, 1), **i32))
    if diagnostics:
        sel.pv, sel.ps = torch.empty(rows, **f32), torch.empty(rows, **f32)
        sel.sv, sel.ss = torch.empty(rows, **i32), torch.empty(rows, **i32)
        sel.nv, sel.ns = torch.empty(nseq * hq, **i32), torch.empty(nseq * hq, **i32)
        sel.jsd = torch.zeros(nseq * hq, dtype=torch.float64, device=dev)
        sel.abar = torch.zeros(rows, **f32)
    if pe_prob:
        sel.pe_prob = torch.empty(max(cap, 1), **f32)
    sel.extra["cu_seqlens"] = [int(x) for x in cu_seqlens]
    return sel


def crisp_prefill_varlen(q, k, v, cu_seqlens, params: CrispParams | None = None, sel: Selection | None = None,
                         o=None, ws=None, diagnostics: bool = True, pe_prob: bool = False):
    """Several sequences packed along the token axis (cu_seqlens: host offsets,
    multiples of 128); each is routed and selected on its own, attention is one
    launch.  Returns (o, sel)."""
    params = params or CrispParams()
    o = torch.empty_like(q) if o is None else o
    shape = make_shape(q, k, v, o)
    sel = sel or new_varlen_selection(q, k, cu_seqlens, diagnostics, pe_prob)
    arr, nseq = _cu(cu_seqlens)
    ws = _workspace(varlen_workspace_bytes(shape, cu_seqlens, params), q.device, ws)
    c_sel = sel.c()
    st = lib().crisp_prefill_varlen(C.byref(shape), nseq, arr, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                    C.byref(params.c()), C.byref(c_sel), o.data_ptr(), ws.data_ptr(), ws.numel(),
                                    _stream())
    if st:
        raise CrispError(st, "crisp_prefill_varlen")
    return o, sel
