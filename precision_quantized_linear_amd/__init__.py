"""Quantized-linear hot path for AMD MI355X (gfx950): Python binding of libpql.

Argument marshalling only: every step of quantize / dequantize / qgemm /
qlinear runs in the HIP kernels of ``libpql.so`` (declared in
``include/pql.h``).  torch supplies device memory and the current stream.
There is no CPU fallback: if the library is missing, every call raises.

    import precision_quantized_linear_amd as pql
    wq = pql.quantize(w, "mxfp8", "weight")      # once, at load
    y = pql.qlinear(x, wq)                        # every call: quantize x, GEMM
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpql.so")

# MX exponent bytes per packed chunk (one chunk = 128 bytes of codes along K).
MX_CHUNK = {"mxfp8": 4, "mxfp4": 8}

SCHEMES = {"fp8_tensor": 0, "fp8_row": 1, "fp8_block128": 2, "mxfp8": 3, "mxfp4": 4,
           "w4a16_asym": 5, "w4a16_sym": 6, "int8_row": 7, "mxfp4_dual": 8}
STATIC_SCHEMES = ("fp8_tensor", "fp8_block128")
ROLES = {"activation": 0, "weight": 1}
OPS = {"quantize": 0, "dequantize": 1, "qgemm": 2, "qlinear": 3}

PQL_OK, PQL_ERR_INVALID_ARGUMENT, PQL_ERR_UNSUPPORTED, PQL_ERR_WORKSPACE, PQL_ERR_HIP = range(5)

_lib = None


class PqlError(RuntimeError):
    """A HIP runtime failure reported by libpql."""


def lib() -> ctypes.CDLL:
    """Load libpql.so (built in-tree by ``precision_quantized_linear_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; run `python -m precision_quantized_linear_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i64, sz, vp, ci = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int
        L.pql_version.restype = ci
        L.pql_last_error.restype = ctypes.c_char_p
        L.pql_kernel_name.restype = ctypes.c_char_p
        L.pql_kernel_name.argtypes = [ci, ci, ci, i64, i64, i64]
        L.pql_quantized_sizes.argtypes = [ci, ci, i64, i64, ctypes.POINTER(sz), ctypes.POINTER(sz), ctypes.POINTER(sz)]
        L.pql_workspace_size.argtypes = [ci, ci, ci, i64, i64, i64, ctypes.POINTER(sz)]
        L.pql_quantize.argtypes = [ci, ci, vp, i64, i64, i64, vp, vp, vp, vp, sz, vp]
        L.pql_dequantize.argtypes = [ci, ci, vp, vp, vp, i64, i64, vp, i64, vp]
        L.pql_qgemm.argtypes = [ci, vp, vp, vp, vp, vp, i64, i64, i64, vp, i64, vp]
        L.pql_qlinear.argtypes = [ci, vp, i64, i64, i64, vp, vp, vp, i64, vp, i64, vp, sz, vp]
        f32 = ctypes.c_float
        L.pql_quantize_static.argtypes = [ci, ci, vp, i64, i64, i64, vp, vp, vp]
        L.pql_qgemm_ex.argtypes = [ci, vp, vp, vp, vp, vp, i64, i64, i64, f32, vp, vp, i64, vp]
        L.pql_qlinear_ex.argtypes = [ci, vp, i64, i64, i64, vp, vp, vp, vp, i64, f32, vp, vp, i64, vp, sz, vp]
        L.pql_layout_sizes.argtypes = [ci, ci, ci, i64, i64, ctypes.POINTER(sz), ctypes.POINTER(sz), ctypes.POINTER(sz)]
        L.pql_repack.argtypes = [ci, ci, ci, ci, vp, vp, vp, vp, i64, i64, vp]
        L.pql_qlinear_noalloc.argtypes = [ci, vp, i64, i64, i64, vp, vp, vp, vp, i64, f32, vp, vp, i64, vp]
        L.pql_noalloc_scratch_bytes.restype = sz
        for f in ("pql_quantized_sizes", "pql_workspace_size", "pql_quantize", "pql_dequantize",
                  "pql_qgemm", "pql_qlinear", "pql_quantize_static", "pql_qgemm_ex", "pql_qlinear_ex",
                  "pql_qlinear_noalloc", "pql_layout_sizes", "pql_repack"):
            getattr(L, f).restype = ci
        _lib = L
    return _lib


def _check(status: int, what: str) -> None:
    if status == PQL_OK:
        return
    msg = f"{what}: {lib().pql_last_error().decode()}"
    if status in (PQL_ERR_INVALID_ARGUMENT, PQL_ERR_WORKSPACE):
        raise ValueError(msg)
    if status == PQL_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise PqlError(msg)


def _scheme(s) -> int:
    if isinstance(s, int):
        return s
    if s not in SCHEMES:
        raise ValueError(f"unknown scheme {s!r}; supported: {sorted(SCHEMES)}")
    return SCHEMES[s]


def _role(r) -> int:
    if isinstance(r, int):
        return r
    if r not in ROLES:
        raise ValueError(f"unknown role {r!r}")
    return ROLES[r]


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


@dataclass
class QTensor:
    """A quantized [rows, cols] tensor in the canonical layout of include/pql.h."""
    scheme: str
    role: str
    rows: int
    cols: int
    codes: torch.Tensor
    scales: torch.Tensor
    zeros: torch.Tensor | None = None

    @property
    def device(self):
        return self.codes.device


def quantized_sizes(scheme, role, rows: int, cols: int):
    c, s, z = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().pql_quantized_sizes(_scheme(scheme), _role(role), rows, cols,
                                     ctypes.byref(c), ctypes.byref(s), ctypes.byref(z)), "quantized_sizes")
    return c.value, s.value, z.value


def workspace_size(op, scheme, role="activation", M=0, N=0, K=0) -> int:
    b = ctypes.c_size_t()
    _check(lib().pql_workspace_size(OPS[op] if isinstance(op, str) else op, _scheme(scheme), _role(role),
                                    M, N, K, ctypes.byref(b)), "workspace_size")
    return b.value


def kernel_name(op, scheme, role="activation", M=0, N=0, K=0) -> str:
    return lib().pql_kernel_name(OPS[op] if isinstance(op, str) else op, _scheme(scheme), _role(role),
                                 M, N, K).decode()


def _alloc_q(scheme: str, role: str, rows: int, cols: int, device) -> QTensor:
    cb, sb, zb = quantized_sizes(scheme, role, rows, cols)
    if scheme.startswith("w4a16"):
        codes = torch.empty((rows, cols // 8), dtype=torch.int32, device=device)
        scales = torch.empty((cols // 128, rows), dtype=torch.bfloat16, device=device)   # group-major
        zeros = torch.empty((cols // 128, rows), dtype=torch.uint8, device=device)
    elif scheme == "int8_row":
        codes = torch.empty((rows, cols), dtype=torch.int8, device=device)
        scales = torch.empty((rows,), dtype=torch.float32, device=device)
        zeros = None
    elif scheme == "mxfp4_dual":   # fine exponents, then coarse fp32 scales, in one byte buffer
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=device)
        scales = torch.empty((sb,), dtype=torch.uint8, device=device)
        zeros = None
    else:
        codes = torch.empty((rows, cols if scheme != "mxfp4" else cols // 2), dtype=torch.uint8, device=device)
        if scheme in ("mxfp8", "mxfp4"):
            c = MX_CHUNK[scheme]
            scales = torch.empty((-(-cols // (32 * c)), rows, c), dtype=torch.uint8, device=device)
        elif scheme == "fp8_tensor":
            scales = torch.empty((1,), dtype=torch.float32, device=device)
        elif scheme == "fp8_row":
            scales = torch.empty((rows,), dtype=torch.float32, device=device)
        elif role == "activation":
            scales = torch.empty((rows, cols // 128), dtype=torch.float32, device=device)
        else:
            scales = torch.empty((rows // 128, cols // 128), dtype=torch.float32, device=device)
        zeros = None
    assert codes.numel() * codes.element_size() == cb and scales.numel() * scales.element_size() == sb
    return QTensor(scheme, role, rows, cols, codes, scales, zeros)


def _as_2d_bf16(x: torch.Tensor) -> torch.Tensor:
    if x.dtype != torch.bfloat16:
        raise ValueError("expected a bfloat16 tensor")
    if not x.is_cuda:
        raise ValueError("expected a tensor on a HIP device")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit stride along K")
    return x


def quantize(x: torch.Tensor, scheme: str, role: str = "activation", workspace: torch.Tensor | None = None,
             out: QTensor | None = None) -> QTensor:
    """Quantize a bf16 [rows, K] tensor (activation: rows = tokens; weight: rows = out channels).
    ``out`` reuses the buffers of an earlier result of the same scheme, role and shape."""
    x = _as_2d_bf16(x)
    rows, cols = x.shape
    if out is not None:
        _check_qtensor(out, "out")
        if (out.scheme, out.role, out.rows, out.cols) != (scheme, role, rows, cols):
            raise ValueError("out does not match the scheme, role and shape")
        if out.device != x.device:
            raise ValueError(f"out is on {out.device}, x on {x.device}")
        q = out
    else:
        q = _alloc_q(scheme, role, rows, cols, x.device)
    wsb = workspace_size("quantize", scheme, role)
    if wsb and workspace is None:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=x.device)
    _check(lib().pql_quantize(_scheme(scheme), _role(role), x.data_ptr(), rows, cols, x.stride(0),
                              q.codes.data_ptr(), q.scales.data_ptr(), _ptr(q.zeros), _ptr(workspace),
                              0 if workspace is None else workspace.numel() * workspace.element_size(),
                              _stream(x.device)), "quantize")
    return q


def quantize_static(x: torch.Tensor, scheme: str, role: str, scales: torch.Tensor,
                    out: QTensor | None = None) -> QTensor:
    """FP8 quantization with supplied (static, calibrated) fp32 scales in the scheme's
    canonical scale layout (fp8_tensor: [1]; fp8_block128: [rows, K/128] activations,
    [rows/128, K/128] weights).  The result holds ``scales`` itself."""
    if scheme not in STATIC_SCHEMES:
        raise NotImplementedError(f"static scales are defined for {STATIC_SCHEMES} only, not {scheme!r}")
    x = _as_2d_bf16(x)
    rows, cols = x.shape
    if scales.dtype != torch.float32 or not scales.is_contiguous() or scales.device != x.device:
        raise ValueError("scales must be a contiguous float32 tensor on the input's device")
    q = out if out is not None else _alloc_q(scheme, role, rows, cols, x.device)
    if scales.numel() != q.scales.numel():
        raise ValueError(f"expected {q.scales.numel()} scales, got {scales.numel()}")
    _check(lib().pql_quantize_static(_scheme(scheme), _role(role), x.data_ptr(), rows, cols, x.stride(0),
                                     scales.data_ptr(), q.codes.data_ptr(), _stream(x.device)), "quantize_static")
    return QTensor(scheme, role, rows, cols, q.codes, scales.reshape(q.scales.shape), None)


def _bias_ptr(bias, n: int, device):
    if bias is None:
        return None
    if bias.dtype != torch.bfloat16 or bias.shape != (n,) or not bias.is_contiguous() or bias.device != device:
        raise ValueError(f"bias must be a contiguous bfloat16 [{n}] tensor on the weight's device")
    return bias.data_ptr()


def _check_out(out: torch.Tensor, rows: int, cols: int, device, what: str = "out") -> None:
    """The C ABI sees only a pointer and a row stride, so the binding checks the rest:
    a bf16 [rows, cols] view on ``device`` with unit column stride and a row stride of
    at least ``cols`` (a view into a wider buffer is fine)."""
    if not isinstance(out, torch.Tensor):
        raise ValueError(f"{what} must be a torch tensor")
    if out.dtype != torch.bfloat16:
        raise ValueError(f"{what} must be bfloat16, not {out.dtype}")
    if out.dim() != 2 or tuple(out.shape) != (rows, cols):
        raise ValueError(f"{what} must have shape ({rows}, {cols}), not {tuple(out.shape)}")
    if rows and (out.stride(1) != 1 or out.stride(0) < cols):
        raise ValueError(f"{what} needs unit column stride and a row stride >= {cols} "
                         f"(strides {tuple(out.stride())})")
    if out.device != torch.device(device):
        raise ValueError(f"{what} is on {out.device}, the operands on {device}")


def _check_qtensor(q: QTensor, what: str) -> None:
    if not isinstance(q, QTensor):
        raise ValueError(f"{what} must be a QTensor")
    bufs = [q.codes, q.scales] + ([q.zeros] if q.zeros is not None else [])
    if any(b.device != q.codes.device for b in bufs):
        raise ValueError(f"{what}: codes, scales and zero-points must be on one device")


def _on_device(device) -> None:
    if torch.device(device).type != "cuda":
        raise ValueError(f"operands must be on a HIP device, not {device}")


def dequantize(q: QTensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 [rows, cols] = bf16(decode(code) * scale)."""
    _check_qtensor(q, "q")
    if out is None:
        out = torch.empty((q.rows, q.cols), dtype=torch.bfloat16, device=q.device)
    _check_out(out, q.rows, q.cols, q.device)
    _on_device(q.device)
    _check(lib().pql_dequantize(_scheme(q.scheme), _role(q.role), q.codes.data_ptr(), q.scales.data_ptr(),
                                _ptr(q.zeros), q.rows, q.cols, out.data_ptr(), out.stride(0),
                                _stream(q.device)), "dequantize")
    return out


def qgemm(a, w: QTensor, out: torch.Tensor | None = None, alpha: float = 1.0,
          bias: torch.Tensor | None = None) -> torch.Tensor:
    """C[M, N] = alpha * (A_hat * W_hat^T) + bias on quantized operands (W4A16: ``a`` is the
    bf16 activation).  ``alpha`` and ``bias`` (bf16 [N]) are the fused epilogue of the FP8
    and int8 schemes."""
    _check_qtensor(w, "w")
    if w.role != "weight":
        raise ValueError("the second operand must be a quantized weight")
    if isinstance(a, QTensor):
        _check_qtensor(a, "a")
        if a.role != "activation":
            raise ValueError("the first operand must be a quantized activation")
        if a.scheme != w.scheme:
            raise ValueError("activation and weight schemes differ")
        if w.scheme.startswith("w4a16"):
            raise ValueError("W4A16 takes the bf16 activation itself, not a quantized one")
        if a.device != w.device:
            raise ValueError(f"activation on {a.device}, weight on {w.device}")
        M, K = a.rows, a.cols
        a_ptr, as_ptr = a.codes.data_ptr(), a.scales.data_ptr()
    else:
        if not w.scheme.startswith("w4a16"):
            raise ValueError(f"{w.scheme} needs a quantized activation (pql.quantize(x, scheme, 'activation'))")
        a = _as_2d_bf16(a)
        if a.device != w.device:
            raise ValueError(f"activation on {a.device}, weight on {w.device}")
        if a.stride(0) != a.shape[1]:
            a = a.contiguous()
        M, K = a.shape
        a_ptr, as_ptr = a.data_ptr(), None
    if K != w.cols:
        raise ValueError(f"K mismatch: {K} vs {w.cols}")
    if out is None:
        out = torch.empty((M, w.rows), dtype=torch.bfloat16, device=w.device)
    _check_out(out, M, w.rows, w.device)
    _on_device(w.device)
    _check(lib().pql_qgemm_ex(_scheme(w.scheme), a_ptr, as_ptr, w.codes.data_ptr(), w.scales.data_ptr(),
                              _ptr(w.zeros), M, w.rows, K, float(alpha), _bias_ptr(bias, w.rows, w.device),
                              out.data_ptr(), out.stride(0), _stream(w.device)), "qgemm")
    return out


def qlinear(x: torch.Tensor, w: QTensor, out: torch.Tensor | None = None,
            workspace: torch.Tensor | None = None, alpha: float = 1.0, bias: torch.Tensor | None = None,
            act_scales: torch.Tensor | None = None) -> torch.Tensor:
    """The quantized linear layer's forward: flatten x[..., K] to 2-D, quantize it with the
    weight's scheme (activation rule), GEMM against ``w``, restore the leading shape.
    ``out``, if given, is the 2-D [M, N] bf16 output (a view with a wider row stride is
    accepted).
    ``alpha`` / ``bias`` are the fused epilogue; ``act_scales`` (fp32, the scheme's
    activation scale layout) makes the activation scales static (fp8_tensor and
    fp8_block128)."""
    _check_qtensor(w, "w")
    if w.role != "weight":
        raise ValueError("w must be a quantized weight")
    lead = x.shape[:-1]
    x2 = x.reshape(-1, x.shape[-1])
    if x2.stride(-1) != 1 or (w.scheme.startswith("w4a16") and x2.stride(0) != x2.shape[1]):
        x2 = x2.contiguous()
    x2 = _as_2d_bf16(x2)
    M, K = x2.shape
    if K != w.cols:
        raise ValueError(f"K mismatch: {K} vs {w.cols}")
    if x2.device != w.device:
        raise ValueError(f"input on {x2.device}, weight on {w.device}")
    if out is None:
        out = torch.empty((M, w.rows), dtype=torch.bfloat16, device=x.device)
    _check_out(out, M, w.rows, w.device)
    if act_scales is not None:
        if w.scheme not in STATIC_SCHEMES:
            raise NotImplementedError(f"static activation scales are defined for {STATIC_SCHEMES} only")
        want = 1 if w.scheme == "fp8_tensor" else M * (K // 128)
        if (act_scales.dtype != torch.float32 or not act_scales.is_contiguous()
                or act_scales.device != x2.device):
            raise ValueError("act_scales must be a contiguous float32 tensor on the input's device")
        if act_scales.numel() != want:
            raise ValueError(f"{w.scheme} takes {want} activation scales, got {act_scales.numel()}")
    wsb = workspace_size("qlinear", w.scheme, "activation", M, w.rows, K)
    if wsb and workspace is None:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=x.device)
    if workspace is not None and (workspace.device != x2.device or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on the input's device")
    _on_device(w.device)
    _check(lib().pql_qlinear_ex(_scheme(w.scheme), x2.data_ptr(), M, K, x2.stride(0), _ptr(act_scales),
                                w.codes.data_ptr(), w.scales.data_ptr(), _ptr(w.zeros), w.rows, float(alpha),
                                _bias_ptr(bias, w.rows, x.device), out.data_ptr(), out.stride(0),
                                _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
                                _stream(x.device)), "qlinear")
    return out.reshape(*lead, w.rows)


LAYOUTS = {"canonical": 0, "packed": 1}


def layout_sizes(scheme, role, layout, rows: int, cols: int):
    c, s, z = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().pql_layout_sizes(_scheme(scheme), _role(role), LAYOUTS[layout], rows, cols,
                                  ctypes.byref(c), ctypes.byref(s), ctypes.byref(z)), "layout_sizes")
    return c.value, s.value, z.value


def _dual_coarse_offset(rows, cols):
    return (rows * (cols // 32) + 255) // 256 * 256


def _canonical_shapes(scheme, role, rows, cols):
    """(scales dtype, scales shape, zeros shape or None) of the canonical layout."""
    if scheme == "mxfp4_dual":
        return torch.uint8, (_dual_coarse_offset(rows, cols) + 4 * rows * (cols // 512),), None
    if scheme in MX_CHUNK:
        return torch.uint8, (rows, cols // 32), None
    if scheme.startswith("w4a16"):
        return torch.bfloat16, (rows, cols // 128), (rows, cols // 128)
    return None, None, None     # the same bytes as the packed layout


def _repack(scheme, role, rows, cols, frm, to, scales_in, zeros_in, scales_out, zeros_out, device):
    _check(lib().pql_repack(_scheme(scheme), _role(role), LAYOUTS[frm], LAYOUTS[to], scales_in.data_ptr(),
                            _ptr(zeros_in), scales_out.data_ptr(), _ptr(zeros_out), rows, cols, _stream(device)),
           "repack")


def to_canonical(q: QTensor):
    """(codes, scales, zeros) of ``q`` in the canonical layout, as device tensors; the
    scales (and W4A16 zero-points) are rearranged on the device by pql_repack."""
    _check_qtensor(q, "q")
    _on_device(q.device)
    dt, shape, zshape = _canonical_shapes(q.scheme, q.role, q.rows, q.cols)
    if dt is None:
        return q.codes, q.scales, q.zeros
    scales = torch.empty(shape, dtype=dt, device=q.device)
    zeros = torch.empty(zshape, dtype=torch.uint8, device=q.device) if zshape else None
    _repack(q.scheme, q.role, q.rows, q.cols, "packed", "canonical", q.scales, q.zeros, scales, zeros, q.device)
    return q.codes, scales, zeros


def from_canonical(scheme: str, role: str, rows: int, cols: int, codes: torch.Tensor, scales: torch.Tensor,
                   zeros: torch.Tensor | None = None) -> QTensor:
    """A QTensor (packed layout) from device tensors in the canonical layout; codes are
    used as they are, scales (and W4A16 zero-points) are rearranged on the device."""
    _on_device(codes.device)
    q = _alloc_q(scheme, role, rows, cols, codes.device)
    cb, sb, zb = layout_sizes(scheme, role, "canonical", rows, cols)
    for t, nb, what in ((codes, cb, "codes"), (scales, sb, "scales"), (zeros, zb, "zeros")):
        if t is None:
            if nb:
                raise ValueError(f"{scheme} needs {what}")
            continue
        if t.device != codes.device or not t.is_contiguous() or t.numel() * t.element_size() != nb:
            raise ValueError(f"{what} must be a contiguous tensor of {nb} bytes on {codes.device}")
    q.codes = codes.view(q.codes.dtype).reshape(q.codes.shape)
    _repack(scheme, role, rows, cols, "canonical", "packed", scales, zeros, q.scales, q.zeros, codes.device)
    return q


def from_numpy(q: dict, device) -> QTensor:
    """Upload a quantized tensor given as NumPy arrays in the canonical layout (MX
    exponents [rows, cols / 32], W4A16 scales and zero-points [rows, cols / 128]); the
    arrays go up as they are and pql_repack rearranges them into the packed layout on
    the device."""
    import numpy as np
    scheme = q["scheme"]

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    codes = up(np.asarray(q["codes"]).view(np.uint8))
    if scheme == "mxfp4_dual":      # one canonical buffer: fine [rows, cols/32], then coarse [rows, cols/512]
        off = _dual_coarse_offset(q["rows"], q["cols"])
        buf = np.zeros(off + 4 * q["rows"] * (q["cols"] // 512), np.uint8)
        fine = np.ascontiguousarray(q["scales"], np.uint8).reshape(-1)
        buf[:fine.size] = fine
        buf[off:] = np.ascontiguousarray(q["coarse"], np.float32).reshape(-1).view(np.uint8)
        scales = up(buf)
    else:
        scales = up(np.asarray(q["scales"]).view(np.uint8))
    zeros = up(np.asarray(q["zeros"]).view(np.uint8)) if q.get("zeros") is not None else None
    return from_canonical(scheme, q["role"], q["rows"], q["cols"], codes, scales, zeros)


def to_numpy(q: QTensor) -> dict:
    """Download a quantized tensor into NumPy arrays in the canonical layout: pql_repack
    rearranges the scales (and W4A16 zero-points) on the device, then the bytes come down
    as they are.  The packed device bytes of MX exponents are also returned, under
    "scales_packed"."""
    import numpy as np
    codes, scales, zeros = to_canonical(q)
    np_dtype = {torch.uint8: np.uint8, torch.int8: np.int8, torch.int32: np.uint32, torch.float32: np.float32,
                torch.bfloat16: np.uint16}

    def down(t):
        return t.contiguous().view(torch.uint8).cpu().numpy().view(np_dtype[t.dtype]).reshape(t.shape)

    out = {"scheme": q.scheme, "role": q.role, "rows": q.rows, "cols": q.cols,
           "codes": down(codes), "scales": down(scales), "zeros": None if zeros is None else down(zeros)}
    if q.scheme in MX_CHUNK:
        out["scales_packed"] = down(q.scales)
    if q.scheme == "mxfp4_dual":    # split the canonical buffer into its two levels
        buf, off = out["scales"], _dual_coarse_offset(q.rows, q.cols)
        out["scales"] = buf[:q.rows * (q.cols // 32)].reshape(q.rows, q.cols // 32).copy()
        out["coarse"] = buf[off:].view(np.float32).reshape(q.rows, q.cols // 512).copy()
        out["scales_packed"] = down(q.scales)
    return out


def qlinear_noalloc(x: torch.Tensor, w: QTensor, out: torch.Tensor, alpha: float = 1.0,
                    bias: torch.Tensor | None = None, act_scales: torch.Tensor | None = None) -> torch.Tensor:
    """``qlinear`` that allocates nothing, for code under HIP graph capture or loops that must
    not allocate: x is a 2-D bf16 [M, K] tensor (W4A16: contiguous), ``out`` the caller's bf16
    [M, N] output.  The activation's codes and scales live in the library's static device
    buffer (``noalloc_scratch_bytes()``); calls overlapping in time on one device race."""
    _check_qtensor(w, "w")
    if w.role != "weight":
        raise ValueError("w must be a quantized weight")
    x = _as_2d_bf16(x)
    M, K = x.shape
    if K != w.cols:
        raise ValueError(f"K mismatch: {K} vs {w.cols}")
    if x.device != w.device:
        raise ValueError(f"input on {x.device}, weight on {w.device}")
    _check_out(out, M, w.rows, w.device)
    if act_scales is not None:
        if w.scheme not in STATIC_SCHEMES:
            raise NotImplementedError(f"static activation scales are defined for {STATIC_SCHEMES} only")
        want = 1 if w.scheme == "fp8_tensor" else M * (K // 128)
        if act_scales.dtype != torch.float32 or not act_scales.is_contiguous() or act_scales.device != x.device \
                or act_scales.numel() != want:
            raise ValueError(f"act_scales must be {want} contiguous float32 values on the input's device")
    _check(lib().pql_qlinear_noalloc(_scheme(w.scheme), x.data_ptr(), M, K, x.stride(0), _ptr(act_scales),
                                     w.codes.data_ptr(), w.scales.data_ptr(), _ptr(w.zeros), w.rows, float(alpha),
                                     _bias_ptr(bias, w.rows, x.device), out.data_ptr(), out.stride(0),
                                     _stream(x.device)), "qlinear_noalloc")
    return out


def noalloc_scratch_bytes() -> int:
    return int(lib().pql_noalloc_scratch_bytes())
