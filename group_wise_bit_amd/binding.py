"""Python binding of libgwb.so — group-wise low-bit weight quantization on MI355X.

Thin Python binding of libgwb.so (C ABI in include/gwb.h). This module only
marshals arguments: torch tensors provide device memory and the current HIP stream,
every step of the method runs in the library's HIP kernels. There is no fallback: if
the library is missing, importing this package raises.

Formats ("fmt"): "gptq_sym", "gptq_asym", "mxfp4", "uintx", "mxfp4_page_ties" (MXFP4 with the
page code's own tie rule; same stored layout), "gptq_sym_act" / "gptq_asym_act" (GPTQ with
act-order groups: quantize takes the channel order `perm`, g_idx names each channel's group),
"gptq_sym_grouped" / "gptq_asym_grouped" (the same weight in group order, made by group_order()
for the decode GEMV; g_idx holds the channel permutation).
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import torch  # must come first: libgwb then binds to the HIP runtime torch loaded

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgwb.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m group_wise_bit_amd._build` "
                      "(or __graft_entry__.build()) first")
lib = ctypes.CDLL(LIB_PATH)

OK, E_ARG, E_SHAPE, E_UNSUPPORTED, E_SIZE, E_HIP = 0, -1, -2, -3, -4, -5
FORMATS = {"gptq_sym": 1, "gptq_asym": 2, "mxfp4": 3, "uintx": 4, "mxfp4_page_ties": 5,
           "gptq_sym_act": 6, "gptq_asym_act": 7, "gptq_sym_grouped": 8, "gptq_asym_grouped": 9}
DEFAULT_GROUP = {"gptq_sym": 128, "gptq_asym": 128, "mxfp4": 32, "uintx": 64, "mxfp4_page_ties": 32,
                 "gptq_sym_act": 128, "gptq_asym_act": 128, "gptq_sym_grouped": 128, "gptq_asym_grouped": 128}
F32, BF16, F16 = 0, 1, 2
_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}


class QSpec(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("nbits", ctypes.c_int32),
                ("group", ctypes.c_int32), ("w_dtype", ctypes.c_int32)]


class QTensors(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("zeros", ctypes.c_void_p), ("g_idx", ctypes.c_void_p)]


class Fold(ctypes.Structure):
    _fields_ = [("col", ctypes.c_void_p), ("row", ctypes.c_void_p), ("col_op", ctypes.c_int32),
                ("row_op", ctypes.c_int32)]


FOLD_OPS = {"none": 0, "mul": 1, "div": 2}


class Sizes(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_size_t), ("scales", ctypes.c_size_t), ("zeros", ctypes.c_size_t),
                ("g_idx", ctypes.c_size_t), ("workspace", ctypes.c_size_t)]


_P, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_SIGS = {
    "gwb_query_sizes": [ctypes.POINTER(QSpec), _I64, _I64, ctypes.POINTER(Sizes)],
    "gwb_quantize": [ctypes.POINTER(QSpec), _P, _I64, _I64, _I64, ctypes.POINTER(QTensors), _P, _SZ, _P],
    "gwb_quantize_act_order": [ctypes.POINTER(QSpec), _P, _I64, _I64, _I64, _P, ctypes.POINTER(QTensors), _P, _SZ,
                               _P],
    "gwb_gptq_group_order": [ctypes.POINTER(QSpec), ctypes.POINTER(QTensors), _I64, _I64, _P, _P, _P, _P],
    "gwb_dequantize": [ctypes.POINTER(QSpec), ctypes.POINTER(QTensors), _I64, _I64, _P, _I32, _I64, _P, _SZ, _P],
    "gwb_snr": [ctypes.POINTER(QSpec), _P, _I64, _I64, _I64, ctypes.POINTER(QTensors), _P, _P, _SZ, _P],
    "gwb_quantize_snr": [ctypes.POINTER(QSpec), _P, _I64, _I64, _I64, ctypes.POINTER(QTensors), _P, _P, _SZ, _P],
    "gwb_quantize_snr_static": [ctypes.POINTER(QSpec), _P, _I64, _I64, _I64, ctypes.POINTER(QTensors), _P, _P],
    "gwb_awq_workspace": [_I64, _I64, _I32, _I64, ctypes.POINTER(_SZ)],
    "gwb_awq_search_mxfp4": [_P, _I32, _I64, _I64, _I64, _P, _P, _I32, _I64, _P, _P, _P, _P, _SZ, _P],
    "gwb_stream_bench": [_I32, _I32, _P, _P, _SZ, _P],
    "gwb_awq_scales_host": [_P, _I64, _P, _I32, _P],
    "gwb_fold_mxfp4": [_P, _I32, _I64, _I64, _I64, ctypes.POINTER(Fold), _P, _I64, ctypes.POINTER(QTensors), _P],
    "gwb_gemv_workspace": [ctypes.POINTER(QSpec), _I64, _I64, _I64, ctypes.POINTER(_SZ)],
    "gwb_gemv": [ctypes.POINTER(QSpec), ctypes.POINTER(QTensors), _I64, _I64, _P, _I64, _I64, _P, _I32, _I64, _P,
                 _SZ, _P],
    "gwb_gemm_workspace": [ctypes.POINTER(QSpec), _I64, _I64, _I64, ctypes.POINTER(_SZ)],
    "gwb_gemm": [ctypes.POINTER(QSpec), ctypes.POINTER(QTensors), _I64, _I64, _P, _I64, _I64, _P, _I32, _I64, _P,
                 _SZ, _P],
}
for _name, _args in _SIGS.items():
    _f = getattr(lib, _name)
    _f.argtypes = _args
    _f.restype = ctypes.c_int
lib.gwb_last_error.argtypes = []
lib.gwb_last_error.restype = ctypes.c_char_p

EXPORTS = tuple(_SIGS) + ("gwb_last_error",)


class GwbError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"gwb error {code}: {msg}")
        self.code = code


def _check(rc: int) -> None:
    if rc != OK:
        raise GwbError(rc, lib.gwb_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def make_spec(fmt: str, nbits: int = 4, group: Optional[int] = None, w_dtype=torch.bfloat16) -> QSpec:
    if fmt not in FORMATS:
        raise ValueError(f"unknown format {fmt!r}")
    return QSpec(FORMATS[fmt], nbits, DEFAULT_GROUP[fmt] if group is None else group,
                 _DT.get(w_dtype, -1) if isinstance(w_dtype, torch.dtype) else int(w_dtype))


def query_sizes(fmt: str, N: int, K: int, nbits: int = 4, group: Optional[int] = None,
                w_dtype=torch.bfloat16) -> Dict[str, int]:
    sp = make_spec(fmt, nbits, group, w_dtype)
    s = Sizes()
    _check(lib.gwb_query_sizes(ctypes.byref(sp), N, K, ctypes.byref(s)))
    return {f: getattr(s, f) for f, _ in Sizes._fields_}


def _alloc(nbytes: int, device) -> torch.Tensor:
    # 256-byte aligned by the caching allocator; at least 16 bytes so the pointer is real
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def _views(fmt: str, N: int, K: int, group: int, w_dtype, sz, codes, scales, zeros, gidx):
    """Typed views of the raw byte buffers (the layouts of gwb_qtensors)."""
    out = {}
    if fmt.startswith("gptq"):
        out["qweight"] = codes[:sz["codes"]].view(torch.int32).view(K // 8, N)
        out["scales"] = scales[:sz["scales"]].view(torch.float16).view(K // group, N)
        out["qzeros"] = zeros[:sz["zeros"]].view(torch.int32).view(K // group, N // 8)
        if gidx is not None:
            out["g_idx"] = gidx[:sz["g_idx"]].view(torch.int32)
    elif fmt.startswith("mxfp4"):
        out["packed"] = codes[:sz["codes"]].view(N, K // 2)
        out["e8m0"] = scales[:sz["scales"]].view(N, K // 32)
    else:
        out["packed"] = codes[:sz["codes"]]
        esize = 4 if w_dtype == torch.float32 else 2            # the scale has the weight dtype
        out["scale_bytes"] = scales[:sz["scales"]].view(N, esize * (K // group))
        out["zero_point"] = zeros[:sz["zeros"]].view(N, K // group)
    return out


class Quantized:
    """Raw buffers of one quantized weight plus typed views; pass it back to
    dequantize() and snr()."""

    def __init__(self, fmt, nbits, group, w_dtype, N, K, codes, scales, zeros, gidx, sizes):
        self.fmt, self.nbits, self.group, self.w_dtype, self.N, self.K = fmt, nbits, group, w_dtype, N, K
        self.codes, self.scales, self.zeros, self.gidx, self.sizes = codes, scales, zeros, gidx, sizes
        self.views = _views(fmt, N, K, group, w_dtype, sizes, codes, scales, zeros, gidx)

    def spec(self) -> QSpec:
        return make_spec(self.fmt, self.nbits, self.group, self.w_dtype)

    def qtensors(self) -> QTensors:
        return QTensors(_ptr(self.codes), _ptr(self.scales), _ptr(self.zeros), _ptr(self.gidx))

    def __getitem__(self, k):
        return self.views[k]


def _weight_args(W: torch.Tensor):
    if W.dim() != 2 or W.dtype not in _DT or not W.is_cuda:
        raise ValueError("W must be a 2-D float32, bfloat16 or float16 CUDA tensor")
    if W.stride(1) != 1:
        raise ValueError("W must have unit stride along K")
    return W.shape[0], W.shape[1], W.stride(0)


def quantize(W: torch.Tensor, fmt: str, nbits: int = 4, group: Optional[int] = None,
             with_g_idx: bool = True, out: Optional[Quantized] = None,
             workspace: Optional[torch.Tensor] = None, perm: Optional[torch.Tensor] = None) -> Quantized:
    """Quantize+pack W [N, K] into a new (or the given) Quantized. The act-order GPTQ
    formats take perm, the channel order (int32 [K] on the device)."""
    N, K, ldw = _weight_args(W)
    group = DEFAULT_GROUP[fmt] if group is None else group
    act = fmt.endswith("_act")
    if act and (perm is None or perm.dtype != torch.int32 or tuple(perm.shape) != (K,) or not perm.is_cuda):
        raise ValueError("act-order formats need perm: an int32 CUDA tensor [K]")
    sp = make_spec(fmt, nbits, group, W.dtype)
    sz = query_sizes(fmt, N, K, nbits, group, W.dtype)
    if out is None:
        dev = W.device
        gidx = _alloc(sz["g_idx"], dev) if (fmt.startswith("gptq") and (with_g_idx or act)) else None
        zeros = _alloc(sz["zeros"], dev) if not fmt.startswith("mxfp4") else None   # GPTQ and uintx carry zeros
        out = Quantized(fmt, nbits, group, W.dtype, N, K, _alloc(sz["codes"], dev), _alloc(sz["scales"], dev),
                        zeros, gidx, sz)
    if workspace is None and sz["workspace"]:
        workspace = _alloc(sz["workspace"], W.device)
    ws_b = 0 if workspace is None else workspace.numel() * workspace.element_size()
    qt = out.qtensors()
    if act:
        _check(lib.gwb_quantize_act_order(ctypes.byref(sp), _ptr(W), N, K, ldw, _ptr(perm.contiguous()),
                                          ctypes.byref(qt), _ptr(workspace), ws_b, _stream()))
    else:
        _check(lib.gwb_quantize(ctypes.byref(sp), _ptr(W), N, K, ldw, ctypes.byref(qt), _ptr(workspace), ws_b,
                                _stream()))
    return out


def group_order(q: Quantized) -> Quantized:
    """Act-order GPTQ into group order for the decode GEMV (gwb_gptq_group_order): a new
    Quantized of format gptq_{sym,asym}_grouped sharing q's scales and qzeros, with the
    rearranged qweight and the permutation in g_idx. Synchronizes to read the kernels'
    status; raises GwbError (E_SHAPE) when a group does not hold exactly G channels or a
    g_idx entry lies outside [0, K/G)."""
    if not q.fmt.endswith("_act"):
        raise ValueError("group_order takes act-order GPTQ (gptq_sym_act / gptq_asym_act)")
    dev = q.codes.device
    codes, perm = _alloc(q.sizes["codes"], dev), _alloc(q.sizes["g_idx"], dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    sp, qt = q.spec(), q.qtensors()
    _check(lib.gwb_gptq_group_order(ctypes.byref(sp), ctypes.byref(qt), q.N, q.K, _ptr(codes), _ptr(perm),
                                    _ptr(status), _stream()))
    st = int(status.item())
    if st:
        raise GwbError(E_SHAPE, "g_idx: a group without exactly G channels" if st == 1 else
                       "g_idx: an entry outside [0, K/G)")
    return Quantized(q.fmt.replace("_act", "_grouped"), q.nbits, q.group, q.w_dtype, q.N, q.K, codes, q.scales,
                     q.zeros, perm, q.sizes)


def dequantize(q: Quantized, out_dtype=None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Unpack+dequantize to [N, K] of out_dtype: float32 or bfloat16; uintx: float32 or
    the weight dtype. Default: bfloat16, uintx the weight dtype."""
    if out_dtype is None:
        out_dtype = q.w_dtype if q.fmt == "uintx" else torch.bfloat16
    if out is None:
        out = torch.empty(q.N, q.K, dtype=out_dtype, device=q.codes.device)
    if out.dtype not in _DT or out.stride(1) != 1:
        raise ValueError("out must be float32, bfloat16 or float16 with unit stride along K")
    sp, qt = q.spec(), q.qtensors()
    _check(lib.gwb_dequantize(ctypes.byref(sp), ctypes.byref(qt), q.N, q.K, _ptr(out), _DT[out.dtype],
                              out.stride(0), None, 0, _stream()))
    return out


def snr(W: torch.Tensor, q: Quantized, workspace: Optional[torch.Tensor] = None,
        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Fused dequant + squared error. Returns a device float64 tensor
    [sum w^2, sum (w - d)^2, SNR dB]."""
    N, K, ldw = _weight_args(W)
    if out is None:
        out = torch.empty(3, dtype=torch.float64, device=W.device)
    if workspace is None:
        workspace = _alloc(q.sizes["workspace"], W.device)
    sp, qt = q.spec(), q.qtensors()
    _check(lib.gwb_snr(ctypes.byref(sp), _ptr(W), N, K, ldw, ctypes.byref(qt), _ptr(out), _ptr(workspace),
                       workspace.numel(), _stream()))
    return out


def quantize_snr(W: torch.Tensor, fmt: str, nbits: int = 4, group: Optional[int] = None,
                 out: Optional[Quantized] = None, snr_out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None):
    """quantize and snr in one call (gwb_quantize_snr): returns (Quantized, device float64
    [sum w^2, sum (w - d)^2, SNR dB])."""
    N, K, ldw = _weight_args(W)
    group = DEFAULT_GROUP[fmt] if group is None else group
    if out is None:
        sz = query_sizes(fmt, N, K, nbits, group, W.dtype)
        dev = W.device
        gidx = _alloc(sz["g_idx"], dev) if fmt.startswith("gptq") else None
        zeros = _alloc(sz["zeros"], dev) if not fmt.startswith("mxfp4") else None
        out = Quantized(fmt, nbits, group, W.dtype, N, K, _alloc(sz["codes"], dev), _alloc(sz["scales"], dev),
                        zeros, gidx, sz)
    if snr_out is None:
        snr_out = torch.empty(3, dtype=torch.float64, device=W.device)
    if workspace is None:
        workspace = _alloc(max(out.sizes["workspace"], 16), W.device)
    sp, qt = out.spec(), out.qtensors()
    _check(lib.gwb_quantize_snr(ctypes.byref(sp), _ptr(W), N, K, ldw, ctypes.byref(qt), _ptr(snr_out),
                                _ptr(workspace), workspace.numel(), _stream()))
    return out, snr_out


def prepare_quantize_snr(W: torch.Tensor, q: Quantized, snr_out: torch.Tensor, workspace: torch.Tensor) -> Prepared:
    N, K, ldw = _weight_args(W)
    if (N, K, W.dtype) != (q.N, q.K, q.w_dtype):
        raise ValueError("W does not match the Quantized buffers")
    sp, qt = q.spec(), q.qtensors()
    return Prepared(lib.gwb_quantize_snr, (ctypes.byref(sp), _ptr(W), N, K, ldw, ctypes.byref(qt), _ptr(snr_out),
                                           _ptr(workspace), workspace.numel(), _stream()),
                    (sp, qt, W, q, snr_out, workspace))


DEFAULT_ALPHAS = tuple(i / 10 for i in range(11))


def awq_scales_host(a: torch.Tensor, alphas: Sequence[float] = DEFAULT_ALPHAS) -> torch.Tensor:
    """The AWQ scaling table [n_alpha, K] float32, computed on the host."""
    a = a.detach().to("cpu", torch.float32).contiguous()
    al = (ctypes.c_double * len(alphas))(*[float(x) for x in alphas])
    out = torch.empty(len(alphas), a.numel(), dtype=torch.float32)
    _check(lib.gwb_awq_scales_host(a.data_ptr(), a.numel(), ctypes.cast(al, _P), len(alphas), out.data_ptr()))
    return out


def awq_workspace_bytes(N: int, K: int, n_alpha: int, max_rows: int = 2048) -> int:
    b = ctypes.c_size_t()
    _check(lib.gwb_awq_workspace(N, K, n_alpha, max_rows, ctypes.byref(b)))
    return b.value




def awq_search(W: torch.Tensor, a: torch.Tensor, alphas: Optional[Sequence[float]] = DEFAULT_ALPHAS,
               max_rows: int = 2048, s_table: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """AWQ alpha search on MXFP4. With alphas=None, s_table [n_alpha, K] float32 is an
    input (the scalings to evaluate); otherwise it is computed (and returned).
    Returns device tensors: err float64 [n_alpha], best int32 [1], s_table."""
    N, K, ldw = _weight_args(W)
    if a.dtype != torch.float32 or a.numel() != K or not a.is_cuda:
        raise ValueError("a must be a float32 CUDA tensor of K elements")
    if alphas is None:
        if s_table is None:
            raise ValueError("alphas=None needs s_table")
        n_alpha = s_table.shape[0]
        host_alphas = None
    else:
        n_alpha = len(alphas)
        host_alphas = (ctypes.c_double * n_alpha)(*alphas)
        if s_table is None:
            s_table = torch.empty(n_alpha, K, dtype=torch.float32, device=W.device)
    err = torch.empty(n_alpha, dtype=torch.float64, device=W.device)
    best = torch.empty(1, dtype=torch.int32, device=W.device)
    if workspace is None:
        workspace = _alloc(awq_workspace_bytes(N, K, n_alpha, max_rows), W.device)
    _check(lib.gwb_awq_search_mxfp4(_ptr(W), _DT[W.dtype], N, K, ldw, _ptr(a.contiguous()),
                                    host_alphas, n_alpha, max_rows, _ptr(s_table), _ptr(err), _ptr(best),
                                    _ptr(workspace), workspace.numel(), _stream()))
    return {"err": err, "best": best, "s_table": s_table}


def _fold_args(W, col, col_op, row, row_op, folded, mx):
    N, K, ldw = _weight_args(W)
    if W.dtype != torch.bfloat16:
        raise ValueError("the fold takes bf16 weights")
    for v, n, what in ((col, K, "col"), (row, N, "row")):
        if v is not None and (v.dtype != torch.float32 or v.numel() != n or not v.is_cuda or not v.is_contiguous()):
            raise ValueError(f"{what} must be a contiguous float32 CUDA tensor of {n} elements")
    f = Fold(_ptr(col), _ptr(row), FOLD_OPS[col_op], FOLD_OPS[row_op])
    qt = None if mx is None else QTensors(_ptr(mx.codes), _ptr(mx.scales), None, None)
    ldo = 0 if folded is None else folded.stride(0)
    return (_ptr(W), BF16, N, K, ldw, ctypes.byref(f), _ptr(folded), ldo,
            None if qt is None else ctypes.byref(qt), _stream()), (f, qt)


def fold_mxfp4(W: torch.Tensor, col: Optional[torch.Tensor] = None, col_op: str = "none",
               row: Optional[torch.Tensor] = None, row_op: str = "none", want_folded: bool = True,
               want_mxfp4: bool = True, folded: Optional[torch.Tensor] = None,
               mx: Optional[Quantized] = None) -> Dict[str, object]:
    """Fold per-column / per-row AWQ scales into a bf16 W [N, K] (column step, then row
    step, each rounded to bf16) and/or quantize the folded weight to MXFP4, in one pass.
    Returns {"folded": bf16 [N, K] or None, "mxfp4": Quantized or None}."""
    N, K, _ = _weight_args(W)
    if want_folded and folded is None:
        folded = torch.empty(N, K, dtype=torch.bfloat16, device=W.device)
    if want_mxfp4 and mx is None:
        sz = query_sizes("mxfp4", N, K, 4, 32, W.dtype)
        mx = Quantized("mxfp4", 4, 32, W.dtype, N, K, _alloc(sz["codes"], W.device), _alloc(sz["scales"], W.device),
                       None, None, sz)
    args, keep = _fold_args(W, col, col_op, row, row_op, folded if want_folded else None,
                            mx if want_mxfp4 else None)
    _check(lib.gwb_fold_mxfp4(*args))
    return {"folded": folded if want_folded else None, "mxfp4": mx if want_mxfp4 else None}


def prepare_fold_mxfp4(W: torch.Tensor, col, col_op: str, row, row_op: str, folded: Optional[torch.Tensor],
                       mx: Optional[Quantized]) -> Prepared:
    args, keep = _fold_args(W, col, col_op, row, row_op, folded, mx)
    return Prepared(lib.gwb_fold_mxfp4, args, (keep, W, col, row, folded, mx))


def gemv_workspace_bytes(q: Quantized, B: int) -> int:
    sp, b = q.spec(), ctypes.c_size_t()
    _check(lib.gwb_gemv_workspace(ctypes.byref(sp), q.N, q.K, B, ctypes.byref(b)))
    return b.value


def _gemv_args(q, x, y, workspace):
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[1] != q.K or x.stride(1) != 1 or not x.is_cuda:
        raise ValueError("x must be a bf16 CUDA tensor [B, K] with unit stride along K")
    B = x.shape[0]
    if y.dtype not in _DT or tuple(y.shape) != (B, q.N) or y.stride(1) != 1:
        raise ValueError("y must be float32 or bf16 [B, N] with unit stride along N")
    sp, qt = q.spec(), q.qtensors()
    ws_b = 0 if workspace is None else workspace.numel()
    return (ctypes.byref(sp), ctypes.byref(qt), q.N, q.K, _ptr(x), B, x.stride(0), _ptr(y), _DT[y.dtype], y.stride(0),
            _ptr(workspace), ws_b, _stream()), (sp, qt)


def gemv(q: Quantized, x: torch.Tensor, y_dtype=torch.float32, out: Optional[torch.Tensor] = None,
         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = x @ dequantize(W)^T from the packed weight (GPTQ or MXFP4); x bf16 [B, K],
    B <= 8; returns y [B, N] of y_dtype."""
    if out is None:
        out = torch.empty(x.shape[0], q.N, dtype=y_dtype, device=x.device)
    if workspace is None:
        nb = gemv_workspace_bytes(q, x.shape[0])
        workspace = _alloc(nb, x.device) if nb else None
    args, _keep = _gemv_args(q, x, out, workspace)
    _check(lib.gwb_gemv(*args))
    return out


def prepare_gemv(q: Quantized, x: torch.Tensor, y: torch.Tensor, workspace: Optional[torch.Tensor]) -> Prepared:
    args, keep = _gemv_args(q, x, y, workspace)
    return Prepared(lib.gwb_gemv, args, (keep, q, x, y, workspace))


def gemm_workspace_bytes(q: Quantized, M: int) -> int:
    sp, b = q.spec(), ctypes.c_size_t()
    _check(lib.gwb_gemm_workspace(ctypes.byref(sp), q.N, q.K, M, ctypes.byref(b)))
    return b.value


def _gemm_args(q, x, y, workspace):
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[1] != q.K or x.stride(1) != 1 or not x.is_cuda:
        raise ValueError("x must be a bf16 CUDA tensor [M, K] with unit stride along K")
    M = x.shape[0]
    if y.dtype not in _DT or tuple(y.shape) != (M, q.N) or y.stride(1) != 1:
        raise ValueError("y must be float32 or bf16 [M, N] with unit stride along N")
    sp, qt = q.spec(), q.qtensors()
    ws_b = 0 if workspace is None else workspace.numel()
    return (ctypes.byref(sp), ctypes.byref(qt), q.N, q.K, _ptr(x), M, x.stride(0), _ptr(y), _DT[y.dtype], y.stride(0),
            _ptr(workspace), ws_b, _stream()), (sp, qt)


def gemm(q: Quantized, x: torch.Tensor, y_dtype=torch.float32, out: Optional[torch.Tensor] = None,
         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = x @ dequantize(W)^T on the matrix cores (GPTQ sym/asym or MXFP4); x bf16
    [M, K]; returns y [M, N] of y_dtype."""
    if out is None:
        out = torch.empty(x.shape[0], q.N, dtype=y_dtype, device=x.device)
    if workspace is None:
        nb = gemm_workspace_bytes(q, x.shape[0])
        workspace = _alloc(nb, x.device) if nb else None
    args, _keep = _gemm_args(q, x, out, workspace)
    _check(lib.gwb_gemm(*args))
    return out


def prepare_gemm(q: Quantized, x: torch.Tensor, y: torch.Tensor, workspace: Optional[torch.Tensor]) -> Prepared:
    args, keep = _gemm_args(q, x, y, workspace)
    return Prepared(lib.gwb_gemm, args, (keep, q, x, y, workspace))


STREAM_PATTERNS = {"copy": 0, "read": 1, "read4_write1": 2, "read1_write4": 3}


STREAM_STRIDED = 4


def stream_bench(pattern: str, dst: torch.Tensor, src: torch.Tensor, blocks: int = 1024,
                 strided: bool = False) -> None:
    """One launch of the streaming ceiling (gwb_stream_bench); both tensors hold the
    larger side's bytes."""
    n = min(src.numel() * src.element_size(), dst.numel() * dst.element_size())
    pat = STREAM_PATTERNS[pattern] | (STREAM_STRIDED if strided else 0)
    _check(lib.gwb_stream_bench(pat, blocks, _ptr(dst), _ptr(src), n, _stream()))


class Prepared:
    """One library call with its arguments marshalled once, for repeated launches
    (timing loops, serving): calling it makes exactly one C call, on the stream that
    was current when it was prepared. The tensors it refers to must stay alive."""

    def __init__(self, fn, args, keep):
        self._fn, self._args, self._keep = fn, tuple(args), keep

    def __call__(self) -> None:
        _check(self._fn(*self._args))


def prepare_quantize(W: torch.Tensor, q: Quantized, workspace: Optional[torch.Tensor] = None,
                     perm: Optional[torch.Tensor] = None) -> Prepared:
    N, K, ldw = _weight_args(W)
    if (N, K, W.dtype) != (q.N, q.K, q.w_dtype):
        raise ValueError("W does not match the Quantized buffers")
    if workspace is None and q.sizes["workspace"]:
        workspace = _alloc(q.sizes["workspace"], W.device)
    sp, qt = q.spec(), q.qtensors()
    ws_b = 0 if workspace is None else workspace.numel()
    if q.fmt.endswith("_act"):
        if perm is None or perm.dtype != torch.int32 or not perm.is_contiguous():
            raise ValueError("act-order formats need perm: a contiguous int32 CUDA tensor [K]")
        return Prepared(lib.gwb_quantize_act_order, (ctypes.byref(sp), _ptr(W), N, K, ldw, _ptr(perm),
                                                     ctypes.byref(qt), _ptr(workspace), ws_b, _stream()),
                        (sp, qt, W, q, workspace, perm))
    return Prepared(lib.gwb_quantize, (ctypes.byref(sp), _ptr(W), N, K, ldw, ctypes.byref(qt), _ptr(workspace),
                                       ws_b, _stream()), (sp, qt, W, q, workspace))


def prepare_dequantize(q: Quantized, out: torch.Tensor) -> Prepared:
    if out.dtype not in _DT or out.stride(1) != 1 or tuple(out.shape) != (q.N, q.K):
        raise ValueError("out must be [N, K] float32, bfloat16 or float16 with unit stride along K")
    sp, qt = q.spec(), q.qtensors()
    return Prepared(lib.gwb_dequantize, (ctypes.byref(sp), ctypes.byref(qt), q.N, q.K, _ptr(out), _DT[out.dtype],
                                         out.stride(0), None, 0, _stream()), (sp, qt, q, out))


def prepare_snr(W: torch.Tensor, q: Quantized, out: torch.Tensor, workspace: torch.Tensor) -> Prepared:
    N, K, ldw = _weight_args(W)
    sp, qt = q.spec(), q.qtensors()
    return Prepared(lib.gwb_snr, (ctypes.byref(sp), _ptr(W), N, K, ldw, ctypes.byref(qt), _ptr(out), _ptr(workspace),
                                  workspace.numel(), _stream()), (sp, qt, W, q, out, workspace))


def prepare_awq_search(W: torch.Tensor, a: torch.Tensor, alphas: Sequence[float], max_rows: int,
                       s_table: torch.Tensor, err: torch.Tensor, best: torch.Tensor,
                       workspace: torch.Tensor) -> Prepared:
    N, K, ldw = _weight_args(W)
    host_alphas = (ctypes.c_double * len(alphas))(*alphas)
    return Prepared(lib.gwb_awq_search_mxfp4, (_ptr(W), _DT[W.dtype], N, K, ldw, _ptr(a), host_alphas, len(alphas),
                                               max_rows, _ptr(s_table), _ptr(err), _ptr(best), _ptr(workspace),
                                               workspace.numel(), _stream()),
                    (W, a, host_alphas, s_table, err, best, workspace))
