"""Thin ctypes binding of libufp4.so.

Argument marshalling only: torch provides device memory (every output is a
torch tensor allocated here and handed to the library as a raw pointer) and
the current stream; every step of the computation runs in the library's HIP
kernels.  The binding fails loudly if the library is missing -- there is no
fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libufp4.so")

GRID_UNIFORM, GRID_E2M1, GRID_E2M1_MAX2 = 0, 1, 2
ROUND_RTNE, ROUND_SR = 0, 1
BLOCKS_ALONG_COLS, BLOCKS_ALONG_ROWS, BLOCKS_ALONG_ROWS_STACKED = 0, 1, 2
FPROP, DGRAD, WGRAD = 0, 1, 2

STATUS = {0: "UFP4_OK", -1: "UFP4_ERR_INVALID_ARG", -2: "UFP4_ERR_SHAPE",
          -3: "UFP4_ERR_MISMATCH", -4: "UFP4_ERR_UNSUPPORTED", -5: "UFP4_ERR_HIP"}

# Every symbol include/ufp4.h declares.
EXPORTS = ("ufp4_rht_quantize", "ufp4_rht_quantize_dual", "ufp4_dequantize", "ufp4_gemm_fprop",
           "ufp4_gemm_dgrad", "ufp4_gemm_wgrad", "ufp4_grouped_gemm", "ufp4_workspace_size",
           "ufp4_status_string", "ufp4_stats_workspace_size", "ufp4_quant_stats",
           "ufp4_output_stats", "ufp4_gemm_out", "ufp4_grouped_gemm_out",
           "ufp4_quant_stats_noalloc")


class UFP4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}")
        self.status = status


class QuantSide(ctypes.Structure):
    """Mirror of ufp4_quant_side."""
    _fields_ = [("rht", ctypes.c_int32), ("sign_mask", ctypes.c_uint32),
                ("stream_id", ctypes.c_uint32), ("reserved", ctypes.c_int32)]


class QTensorDesc(ctypes.Structure):
    """Mirror of ufp4_qtensor."""
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("k", ctypes.c_int64), ("kpad", ctypes.c_int64),
                ("grid", ctypes.c_int32), ("rht", ctypes.c_int32),
                ("sign_mask", ctypes.c_uint32), ("reserved", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libufp4.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m uniform_grid_fp4_amd.build` (no fallback exists)")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I64, I32, U32, U64 = ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint64
    Q = ctypes.POINTER(QTensorDesc)
    L.ufp4_rht_quantize.argtypes = [P, I64, I64, I64, I32, P, I32, I32, U32, I32, I32, U64, U32,
                                    Q, P]
    L.ufp4_rht_quantize_dual.argtypes = [P, I64, I64, I64, I32, P, I32, I32, I32, U64,
                                         ctypes.POINTER(QuantSide), ctypes.POINTER(QuantSide),
                                         Q, Q, P]
    L.ufp4_dequantize.argtypes = [Q, I32, P, I64, P]
    L.ufp4_gemm_fprop.argtypes = [Q, Q, P, I64, P]
    L.ufp4_gemm_dgrad.argtypes = [Q, Q, P, I64, P]
    L.ufp4_gemm_wgrad.argtypes = [Q, Q, P, I64, P, ctypes.c_size_t, P]
    L.ufp4_grouped_gemm.argtypes = [I32, I32, P, Q, Q, P, I64, P, ctypes.c_size_t, P]
    L.ufp4_gemm_out.argtypes = [I32, Q, Q, P, I32, I64, P]
    L.ufp4_grouped_gemm_out.argtypes = [I32, I32, P, Q, Q, P, I32, I64, P]
    L.ufp4_workspace_size.argtypes = [I32, I64, I64, I64, I32]
    L.ufp4_workspace_size.restype = ctypes.c_size_t
    L.ufp4_stats_workspace_size.argtypes = []
    L.ufp4_stats_workspace_size.restype = ctypes.c_size_t
    L.ufp4_quant_stats.argtypes = [P, I64, I64, I64, I32, Q, P, ctypes.c_size_t, P, P]
    L.ufp4_output_stats.argtypes = [P, I64, P, I64, I64, I64, P, ctypes.c_size_t, P, P]
    L.ufp4_quant_stats_noalloc.argtypes = [P, I64, I64, I64, I32, Q, P, P]
    L.ufp4_status_string.argtypes = [I32]
    L.ufp4_status_string.restype = ctypes.c_char_p
    for f in ("ufp4_quant_stats", "ufp4_quant_stats_noalloc", "ufp4_output_stats",
              "ufp4_rht_quantize",
              "ufp4_rht_quantize_dual", "ufp4_dequantize", "ufp4_gemm_fprop", "ufp4_gemm_dgrad",
              "ufp4_gemm_wgrad", "ufp4_grouped_gemm", "ufp4_gemm_out", "ufp4_grouped_gemm_out"):
        getattr(L, f).restype = ctypes.c_int32
    _lib = L
    return L


def _check(status: int, where: str):
    if status != 0:
        raise UFP4Error(status, where)


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


@dataclass
class Quantized:
    """A quantized operand: codes [rows, kpad/2] uint8 and scales [rows,
    kpad/16] float32 on the GPU, plus what the GEMMs need to check."""
    codes: torch.Tensor
    scales: torch.Tensor
    rows: int
    k: int
    kpad: int
    grid: int
    rht: int
    sign_mask: int

    def desc(self) -> QTensorDesc:
        return QTensorDesc(self.codes.data_ptr(), self.scales.data_ptr(), self.rows, self.k,
                           self.kpad, self.grid, self.rht, self.sign_mask, 0)


def padded_k_capacity(n_rows: int, n_groups: int) -> int:
    """The kpad the binding gives a grouped ALONG_ROWS quantization: the
    smallest the call accepts, roundup16(n_rows + 15 * n_groups), rounded up
    to a multiple of 512 so that every output row's codes (kpad/2 bytes) and
    scales (kpad/4 bytes) start on a 128-byte boundary.  Rows that do not
    (e.g. kpad = 524768 for the MoE-124B tokens) made the column-wise kernel's
    128-byte code pieces straddle two lines: 1.67x slower."""
    return (n_rows + 15 * n_groups + 511) // 512 * 512


def _quant_shape(x: torch.Tensor, axis: int, group_offsets: Optional[torch.Tensor],
                 kpad: Optional[int], n_groups: int):
    """(rows, kpad, n_groups) of the quantized output of x along `axis`."""
    assert x.dim() == 2 and x.dtype == torch.bfloat16 and x.is_cuda and x.stride(1) == 1
    n_rows, n_cols = x.shape
    if axis != BLOCKS_ALONG_ROWS_STACKED:
        n_groups = 0
    if axis == BLOCKS_ALONG_COLS:
        return n_rows, (n_cols + 15) // 16 * 16, 0
    if axis == BLOCKS_ALONG_ROWS_STACKED:
        assert n_groups >= 1 and n_rows % n_groups == 0
        return n_cols * n_groups, (n_rows // n_groups + 15) // 16 * 16, n_groups
    if group_offsets is not None:
        assert group_offsets.dtype == torch.int64 and group_offsets.is_cuda
        n_groups = group_offsets.numel() - 1
        kp = kpad if kpad is not None else padded_k_capacity(n_rows, n_groups)
        return n_cols, kp, n_groups
    return n_cols, (n_rows + 15) // 16 * 16, 0


def _out_desc(out: Optional[Quantized], rows: int, kp: int, device):
    if out is not None:
        assert out.rows == rows and out.kpad == kp
        codes, scales = out.codes, out.scales
    else:
        codes = torch.empty((rows, kp // 2), dtype=torch.uint8, device=device)
        scales = torch.empty((rows, kp // 16), dtype=torch.float32, device=device)
    return codes, scales, QTensorDesc(codes.data_ptr(), scales.data_ptr(), rows, 0, kp, 0, 0, 0, 0)


def ufp4_rht_quantize(x: torch.Tensor, axis: int = BLOCKS_ALONG_COLS, rht: bool = True,
                      sign_mask: int = 0, grid: int = GRID_UNIFORM, rnd: int = ROUND_RTNE,
                      seed: int = 0, stream_id: int = 0,
                      group_offsets: Optional[torch.Tensor] = None,
                      kpad: Optional[int] = None, out: Optional[Quantized] = None,
                      n_groups: int = 0) -> Quantized:
    """Quantize a 2-D bf16 CUDA tensor (any row stride, unit column stride).
    `out` reuses the buffers of an earlier result of the same shape;
    `n_groups` is the number of equal row groups for BLOCKS_ALONG_ROWS_STACKED."""
    rows, kp, n_groups = _quant_shape(x, axis, group_offsets, kpad, n_groups)
    codes, scales, d = _out_desc(out, rows, kp, x.device)
    n_rows, n_cols = x.shape
    st = lib().ufp4_rht_quantize(_ptr(x), n_rows, n_cols, x.stride(0), axis,
                                 _ptr(group_offsets), n_groups, int(rht), sign_mask, grid, rnd,
                                 seed, stream_id, ctypes.byref(d), _stream(x.device))
    _check(st, "ufp4_rht_quantize")
    return Quantized(codes, scales, rows, d.k, kp, d.grid, d.rht, d.sign_mask)


def ufp4_rht_quantize_dual(x: torch.Tensor, rowwise: Tuple[bool, int, int],
                           colwise: Tuple[bool, int, int], col_axis: int = BLOCKS_ALONG_ROWS,
                           grid: int = GRID_UNIFORM, rnd: int = ROUND_RTNE, seed: int = 0,
                           group_offsets: Optional[torch.Tensor] = None,
                           kpad: Optional[int] = None, n_groups: int = 0,
                           out_rows: Optional[Quantized] = None,
                           out_cols: Optional[Quantized] = None) -> Tuple[Quantized, Quantized]:
    """Both operands of x from one read: (row-wise, column-wise).  `rowwise`
    and `colwise` are (rht, sign_mask, stream_id) of each output; the
    column-wise output follows `col_axis`, `group_offsets`, `kpad` and
    `n_groups` exactly as ufp4_rht_quantize does."""
    rr, kr, _ = _quant_shape(x, BLOCKS_ALONG_COLS, None, None, 0)
    rc, kc, n_groups = _quant_shape(x, col_axis, group_offsets, kpad, n_groups)
    codes_r, scales_r, dr = _out_desc(out_rows, rr, kr, x.device)
    codes_c, scales_c, dc = _out_desc(out_cols, rc, kc, x.device)
    sr = QuantSide(int(rowwise[0]), rowwise[1], rowwise[2], 0)
    sc = QuantSide(int(colwise[0]), colwise[1], colwise[2], 0)
    n_rows, n_cols = x.shape
    st = lib().ufp4_rht_quantize_dual(_ptr(x), n_rows, n_cols, x.stride(0), col_axis,
                                      _ptr(group_offsets), n_groups, grid, rnd, seed,
                                      ctypes.byref(sr), ctypes.byref(sc), ctypes.byref(dr),
                                      ctypes.byref(dc), _stream(x.device))
    _check(st, "ufp4_rht_quantize_dual")
    return (Quantized(codes_r, scales_r, rr, dr.k, kr, dr.grid, dr.rht, dr.sign_mask),
            Quantized(codes_c, scales_c, rc, dc.k, kc, dc.grid, dc.rht, dc.sign_mask))


STATS_SUMS = ("sum_x2", "sum_err2", "sum_x_xhat", "sum_abs_x", "sum_abs_xhat")
STATS_COUNTS = ("n_elems", "n_nonzero", "n_underflow")


def ufp4_stats_workspace_size() -> int:
    return int(lib().ufp4_stats_workspace_size())


def _stats_buffers(device, workspace: Optional[torch.Tensor]):
    nbytes = ufp4_stats_workspace_size()
    if workspace is None:
        workspace = torch.empty(nbytes // 8, dtype=torch.int64, device=device)
    out = torch.empty(24, dtype=torch.int64, device=device)   # one ufp4_stats
    return workspace, workspace.numel() * workspace.element_size(), out


def _stats_dict(out: torch.Tensor) -> dict:
    h = out.cpu()
    sums = h[:5].view(torch.float64).tolist()
    d = dict(zip(STATS_SUMS, sums))
    d.update(zip(STATS_COUNTS, (int(v) for v in h[5:8])))
    d["hist"] = [int(v) for v in h[8:24]]
    return d


def ufp4_quant_stats(x: torch.Tensor, q: Quantized, axis: int = BLOCKS_ALONG_COLS,
                     workspace: Optional[torch.Tensor] = None) -> dict:
    """Sums and counts comparing x with its quantization q (see ufp4_stats in
    include/ufp4.h); waits for the result."""
    assert x.dim() == 2 and x.dtype == torch.bfloat16 and x.is_cuda and x.stride(1) == 1
    ws, nbytes, out = _stats_buffers(x.device, workspace)
    d = q.desc()
    st = lib().ufp4_quant_stats(_ptr(x), x.shape[0], x.shape[1], x.stride(0), axis,
                                ctypes.byref(d), _ptr(ws), nbytes, _ptr(out), _stream(x.device))
    _check(st, "ufp4_quant_stats")
    return _stats_dict(out)


def ufp4_quant_stats_noalloc(x: torch.Tensor, q: Quantized, axis: int = BLOCKS_ALONG_COLS,
                             out: Optional[torch.Tensor] = None) -> dict:
    """ufp4_quant_stats with the partial sums in the library's own scratch
    array (the C call takes no workspace and allocates nothing); `out`, an
    int64 tensor of 24 elements, receives the ufp4_stats record.  Waits for
    the result."""
    assert x.dim() == 2 and x.dtype == torch.bfloat16 and x.is_cuda and x.stride(1) == 1
    if out is None:
        out = torch.empty(24, dtype=torch.int64, device=x.device)
    assert out.dtype == torch.int64 and out.numel() == 24 and out.is_contiguous()
    d = q.desc()
    st = lib().ufp4_quant_stats_noalloc(_ptr(x), x.shape[0], x.shape[1], x.stride(0), axis,
                                        ctypes.byref(d), _ptr(out), _stream(x.device))
    _check(st, "ufp4_quant_stats_noalloc")
    return _stats_dict(out)


def ufp4_output_stats(ref: torch.Tensor, test: torch.Tensor,
                      workspace: Optional[torch.Tensor] = None) -> dict:
    """The same sums for a GEMM output `test` against `ref` (FP32, 2-D)."""
    assert ref.shape == test.shape and ref.dim() == 2
    assert ref.dtype == test.dtype == torch.float32 and ref.stride(1) == test.stride(1) == 1
    ws, nbytes, out = _stats_buffers(ref.device, workspace)
    st = lib().ufp4_output_stats(_ptr(ref), ref.stride(0), _ptr(test), test.stride(0),
                                 ref.shape[0], ref.shape[1], _ptr(ws), nbytes, _ptr(out),
                                 _stream(ref.device))
    _check(st, "ufp4_output_stats")
    return _stats_dict(out)


def ufp4_dequantize(q: Quantized, inverse_rht: bool = False) -> torch.Tensor:
    out = torch.empty((q.rows, q.kpad), dtype=torch.float32, device=q.codes.device)
    d = q.desc()
    st = lib().ufp4_dequantize(ctypes.byref(d), int(inverse_rht), _ptr(out), q.kpad,
                               _stream(out.device))
    _check(st, "ufp4_dequantize")
    return out


def _dense(fn, name, a: Quantized, b: Quantized, out: Optional[torch.Tensor], *extra):
    if out is None:
        out = torch.empty((a.rows, b.rows), dtype=torch.float32, device=a.codes.device)
    da, db = a.desc(), b.desc()
    st = fn(ctypes.byref(da), ctypes.byref(db), _ptr(out), out.stride(0), *extra,
            _stream(out.device))
    _check(st, name)
    return out


def ufp4_gemm_fprop(xq: Quantized, wq: Quantized, out: Optional[torch.Tensor] = None):
    """Y = X_hat W_hat^T, [T, F] FP32."""
    return _dense(lib().ufp4_gemm_fprop, "ufp4_gemm_fprop", xq, wq, out)


def ufp4_gemm_dgrad(dyq: Quantized, wtq: Quantized, out: Optional[torch.Tensor] = None):
    """dX = dY_hat (W^T)_hat^T, [T, H] FP32."""
    return _dense(lib().ufp4_gemm_dgrad, "ufp4_gemm_dgrad", dyq, wtq, out)


def ufp4_gemm_wgrad(dytq: Quantized, xtq: Quantized, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None):
    """dW = (dY^T)_hat (X^T)_hat^T, [F, H] FP32."""
    ws = _ptr(workspace)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return _dense(lib().ufp4_gemm_wgrad, "ufp4_gemm_wgrad", dytq, xtq, out, ws, nbytes)


def ufp4_grouped_gemm(kind: int, group_offsets: torch.Tensor, a: Quantized, b: Quantized,
                      out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None):
    """Expert-grouped GEMM; see include/ufp4.h for the three kinds."""
    n_groups = group_offsets.numel() - 1
    if kind == WGRAD:
        shape = (n_groups, a.rows, b.rows)
        ldc = b.rows
    else:
        n = b.rows // n_groups
        shape = (a.rows, n)
        ldc = n
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=a.codes.device)
    da, db = a.desc(), b.desc()
    ws = _ptr(workspace)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().ufp4_grouped_gemm(kind, n_groups, _ptr(group_offsets), ctypes.byref(da),
                                 ctypes.byref(db), _ptr(out), ldc, ws, nbytes,
                                 _stream(out.device))
    _check(st, "ufp4_grouped_gemm")
    return out


OUT_F32, OUT_BF16 = 0, 1
_OUT_CODE = {torch.float32: OUT_F32, torch.bfloat16: OUT_BF16}


def ufp4_gemm_out(kind: int, a: Quantized, b: Quantized, dtype=torch.bfloat16,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """FPROP / DGRAD / WGRAD (kind 0 / 1 / 2) with a float32 or bfloat16
    output written by the GEMM's epilogue."""
    if out is None:
        out = torch.empty((a.rows, b.rows), dtype=dtype, device=a.codes.device)
    assert out.dtype in _OUT_CODE and out.stride(1) == 1
    da, db = a.desc(), b.desc()
    st = lib().ufp4_gemm_out(kind, ctypes.byref(da), ctypes.byref(db), _ptr(out),
                             _OUT_CODE[out.dtype], out.stride(0), _stream(out.device))
    _check(st, "ufp4_gemm_out")
    return out


def ufp4_grouped_gemm_out(kind: int, group_offsets: torch.Tensor, a: Quantized, b: Quantized,
                          dtype=torch.bfloat16, out: Optional[torch.Tensor] = None):
    """ufp4_grouped_gemm with a float32 or bfloat16 output."""
    n_groups = group_offsets.numel() - 1
    if kind == WGRAD:
        shape, ldc = (n_groups, a.rows, b.rows), b.rows
    else:
        shape, ldc = (a.rows, b.rows // n_groups), b.rows // n_groups
    if out is None:
        out = torch.empty(shape, dtype=dtype, device=a.codes.device)
    assert out.dtype in _OUT_CODE and out.is_contiguous()
    da, db = a.desc(), b.desc()
    st = lib().ufp4_grouped_gemm_out(kind, n_groups, _ptr(group_offsets), ctypes.byref(da),
                                     ctypes.byref(db), _ptr(out), _OUT_CODE[out.dtype], ldc,
                                     _stream(out.device))
    _check(st, "ufp4_grouped_gemm_out")
    return out


def ufp4_workspace_size(kind: int, m: int, n: int, kpad: int, n_groups: int = 1) -> int:
    return int(lib().ufp4_workspace_size(kind, m, n, kpad, n_groups))


def ufp4_status_string(status: int) -> str:
    return lib().ufp4_status_string(status).decode()
