"""Thin ctypes binding of libhq.so (C ABI in include/hq.h).

The functions keep the C names.  They only marshal arguments: they check
tensor placement, dtype, contiguity and shape, allocate outputs with torch
when the caller passes none, pass raw device pointers plus torch's current
HIP stream, and turn a non-OK status into an exception.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.  If the
library is missing the first call raises.

Pages cited: [RQ] "旋转量化：大模型低比特量化中的离群值克星" sections 2.1-2.2;
[QT] "手把手教你用QuaRot实现LLM的4位量化：从原理到代码实践" section 2.1.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libhq.so")

HQ_OK, HQ_EINVAL, HQ_EUNSUPPORTED, HQ_EHIP = 0, 1, 2, 3
HQ_F32, HQ_BF16, HQ_F16 = 0, 1, 2

_TORCH_TO_HQ = {torch.float32: HQ_F32, torch.bfloat16: HQ_BF16, torch.float16: HQ_F16}
_HQ_TO_TORCH = {v: k for k, v in _TORCH_TO_HQ.items()}

EXPORTS = ("hq_rotate_quant", "hq_dequant_rotate_inv", "hq_rotate_quant_grouped",
           "hq_dequant_rotate_inv_grouped", "hq_rotate_quant_append", "hq_decode_attention",
           "hq_decode_attention_workspace", "hq_decode_attention_noalloc", "hq_rotate",
           "hq_status_str", "hq_last_hip_error", "hq_max_n", "hq_version")

# Bytes of the library's own decode-attention workspace on each GPU
# (HQ_NOALLOC_WORKSPACE_BYTES in include/hq.h).
NOALLOC_WORKSPACE_BYTES = 4 * 1024 * 1024

_lock = threading.Lock()
_lib = None


class HQError(RuntimeError):
    """A libhq call returned a status other than HQ_OK."""

    def __init__(self, status: int, fn: str, detail: str = ""):
        self.status = status
        msg = f"{fn}: {status_str(status)}"
        if detail:
            msg += f" ({detail})"
        super().__init__(msg)


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libhq.so (once) and declare its signatures."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(
                f"libhq.so not found at {p}: build it first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        lib = ctypes.CDLL(p)
        P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.hq_rotate_quant.argtypes = [P, I32, I64, I32, I32, P, I32, P, P, I32, P]
        lib.hq_rotate_quant.restype = I32
        lib.hq_dequant_rotate_inv.argtypes = [P, P, I32, I64, I32, I32, P, I32, P, I32, P]
        lib.hq_dequant_rotate_inv.restype = I32
        lib.hq_rotate_quant_grouped.argtypes = [P, I32, I64, I32, I32, P, I32, I32, P, P, I32, P]
        lib.hq_rotate_quant_grouped.restype = I32
        lib.hq_dequant_rotate_inv_grouped.argtypes = [P, P, I32, I64, I32, I32, P, I32, I32, P,
                                                      I32, P]
        lib.hq_dequant_rotate_inv_grouped.restype = I32
        lib.hq_rotate_quant_append.argtypes = [P, I32, I64, I32, I32, P, I32, P, P, P, I32, I64, P]
        lib.hq_rotate_quant_append.restype = I32
        lib.hq_decode_attention_workspace.argtypes = [I32, I32, I64]
        lib.hq_decode_attention_workspace.restype = I64
        lib.hq_decode_attention.argtypes = [P, I32, I32, I32, I32, I32, P, I64, I32, P, P, P, P,
                                            I32, P, P, I64, P]
        lib.hq_decode_attention.restype = I32
        lib.hq_decode_attention_noalloc.argtypes = [P, I32, I32, I32, I32, I32, P, I64, I32, P, P,
                                                    P, P, I32, P, P]
        lib.hq_decode_attention_noalloc.restype = I32
        lib.hq_rotate.argtypes = [P, I32, I64, I32, I32, P, P, P]
        lib.hq_rotate.restype = I32
        lib.hq_status_str.argtypes = [I32]
        lib.hq_status_str.restype = ctypes.c_char_p
        lib.hq_last_hip_error.argtypes = []
        lib.hq_last_hip_error.restype = ctypes.c_char_p
        lib.hq_max_n.argtypes = []
        lib.hq_max_n.restype = I32
        lib.hq_version.argtypes = []
        lib.hq_version.restype = I32
        _lib = lib
        return lib


def status_str(status: int) -> str:
    return load().hq_status_str(int(status)).decode()


def hq_version() -> int:
    return int(load().hq_version())


def hq_max_n() -> int:
    return int(load().hq_max_n())


def _raise(status: int, fn: str):
    if status == HQ_OK:
        return
    detail = load().hq_last_hip_error().decode()
    if status == HQ_EINVAL:
        raise ValueError(f"{fn}: {status_str(status)}")
    if status == HQ_EUNSUPPORTED:
        raise NotImplementedError(f"{fn}: {status_str(status)}")
    raise HQError(status, fn, detail)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check_dev(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _rows_n(x: torch.Tensor, name: str):
    if x.dim() != 2:
        raise ValueError(f"{name} must be 2-D [rows, n]")
    return x.shape[0], x.shape[1]


def hq_rotate_quant(x: torch.Tensor, s: torch.Tensor, b: int, bits: int = 4,
                    scale_dtype: torch.dtype = torch.float32,
                    codes: torch.Tensor | None = None,
                    scales: torch.Tensor | None = None, stream=None):
    """Rotate + quantise rows of x.  Returns (codes, scales): codes uint8
    [rows, n/2] (bits 4) or int8 [rows, n] (bits 8); scales [rows]."""
    return _rotate_quant(x, s, b, bits, None, scale_dtype, codes, scales, stream)


def hq_rotate_quant_grouped(x: torch.Tensor, s: torch.Tensor, b: int, group: int,
                            bits: int = 4, scale_dtype: torch.dtype = torch.float32,
                            codes: torch.Tensor | None = None,
                            scales: torch.Tensor | None = None, stream=None):
    """Rotate + quantise with one scale per `group` consecutive rotated
    elements.  Returns (codes, scales) with scales [rows, n/group]."""
    return _rotate_quant(x, s, b, bits, int(group), scale_dtype, codes, scales, stream)


def _rotate_quant(x, s, b, bits, group, scale_dtype, codes, scales, stream):
    _check_dev(x, "x")
    if x.dtype not in _TORCH_TO_HQ:
        raise ValueError(f"x dtype {x.dtype} unsupported")
    rows, n = _rows_n(x, "x")
    _check_dev(s, "s", torch.int8, (n,))
    if scale_dtype not in (torch.float32, torch.float16):
        raise ValueError("scale_dtype must be float32 or float16")
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    cshape = (rows, n // 2) if bits == 4 else (rows, n)
    cdtype = torch.uint8 if bits == 4 else torch.int8
    if codes is None:
        codes = torch.empty(cshape, dtype=cdtype, device=x.device)
    _check_dev(codes, "codes", cdtype, cshape)
    sshape = (rows,) if group is None else (rows, n // group if group > 0 else 0)
    if scales is None:
        scales = torch.empty(sshape, dtype=scale_dtype, device=x.device)
    _check_dev(scales, "scales", scale_dtype, sshape)
    if group is None:
        st = load().hq_rotate_quant(x.data_ptr(), _TORCH_TO_HQ[x.dtype], rows, n, int(b),
                                    s.data_ptr(), int(bits), codes.data_ptr(),
                                    scales.data_ptr(), _TORCH_TO_HQ[scale_dtype],
                                    _stream(stream))
        _raise(st, "hq_rotate_quant")
    else:
        st = load().hq_rotate_quant_grouped(x.data_ptr(), _TORCH_TO_HQ[x.dtype], rows, n,
                                            int(b), s.data_ptr(), int(bits), group,
                                            codes.data_ptr(), scales.data_ptr(),
                                            _TORCH_TO_HQ[scale_dtype], _stream(stream))
        _raise(st, "hq_rotate_quant_grouped")
    return codes, scales


def hq_rotate_quant_append(x: torch.Tensor, s: torch.Tensor, b: int, dst_rows: torch.Tensor,
                           codes: torch.Tensor, scales: torch.Tensor, bits: int = 4,
                           stream=None):
    """Rotate + quantise the rows of x into an existing cache: row r's codes
    and scale go to cache row dst_rows[r] (int64, on the GPU).  codes is the
    cache's [cache_rows, n/2] uint8 (bits 4) or [cache_rows, n] int8, scales
    its [cache_rows] float32 or float16.  Rows whose index is outside the
    cache are skipped.  Returns (codes, scales)."""
    _check_dev(x, "x")
    if x.dtype not in _TORCH_TO_HQ:
        raise ValueError(f"x dtype {x.dtype} unsupported")
    rows, n = _rows_n(x, "x")
    _check_dev(s, "s", torch.int8, (n,))
    _check_dev(dst_rows, "dst_rows", torch.int64, (rows,))
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    _check_dev(codes, "codes")
    if codes.dim() != 2:
        raise ValueError("codes must be 2-D [cache_rows, n/2] or [cache_rows, n]")
    cache_rows = codes.shape[0]
    cshape = (cache_rows, n // 2) if bits == 4 else (cache_rows, n)
    cdtype = torch.uint8 if bits == 4 else torch.int8
    _check_dev(codes, "codes", cdtype, cshape)
    _check_dev(scales, "scales", None, (cache_rows,))
    if scales.dtype not in (torch.float32, torch.float16):
        raise ValueError("scales must be float32 or float16")
    st = load().hq_rotate_quant_append(x.data_ptr(), _TORCH_TO_HQ[x.dtype], rows, n, int(b),
                                       s.data_ptr(), int(bits), dst_rows.data_ptr(),
                                       codes.data_ptr(), scales.data_ptr(),
                                       _TORCH_TO_HQ[scales.dtype], cache_rows, _stream(stream))
    _raise(st, "hq_rotate_quant_append")
    return codes, scales


def hq_decode_attention_workspace(q_heads: int, kv_heads: int, tokens: int) -> int:
    """Bytes of workspace hq_decode_attention needs."""
    return int(load().hq_decode_attention_workspace(int(q_heads), int(kv_heads), int(tokens)))


def _attention_args(q, s, k_codes, k_scales, v_codes, v_scales, bits, out):
    """Checks of hq_decode_attention's tensors; returns (q_heads, n, tokens,
    kv_heads, out)."""
    # shapes first (the library reads tokens * kv_heads rows of n/2 code
    # bytes from each code tensor, so a narrower one would be read past its
    # end), then placement and types
    q_heads, n = _rows_n(q, "q")
    for name, t in (("k_codes", k_codes), ("v_codes", v_codes)):
        if not isinstance(t, torch.Tensor) or t.dim() != 3:
            raise ValueError(f"{name} must be a 3-D tensor [tokens, kv_heads, n/2]")
    tokens, kv_heads, _ = k_codes.shape
    width = n // 2 if bits == 4 else n
    for name, t in (("k_codes", k_codes), ("v_codes", v_codes)):
        if tuple(t.shape) != (tokens, kv_heads, width):
            raise ValueError(f"{name} must have shape {(tokens, kv_heads, width)} for "
                             f"n={n}, bits={bits}; got {tuple(t.shape)}")
    _check_dev(q, "q")
    if q.dtype not in _TORCH_TO_HQ:
        raise ValueError(f"q dtype {q.dtype} unsupported")
    _check_dev(s, "s", torch.int8, (n,))
    for name, t in (("k_codes", k_codes), ("v_codes", v_codes)):
        _check_dev(t, name, torch.uint8)
    if k_scales.dtype not in (torch.float32, torch.float16):
        raise ValueError("scales must be float32 or float16")
    _check_dev(k_scales, "k_scales", None, (tokens, kv_heads))
    _check_dev(v_scales, "v_scales", k_scales.dtype, (tokens, kv_heads))
    if out is None:
        out = torch.empty((q_heads, n), dtype=torch.float32, device=q.device)
    _check_dev(out, "out", torch.float32, (q_heads, n))
    return q_heads, n, tokens, kv_heads, out


def hq_decode_attention(q: torch.Tensor, s: torch.Tensor, b: int, k_codes: torch.Tensor,
                        k_scales: torch.Tensor, v_codes: torch.Tensor, v_scales: torch.Tensor,
                        bits: int = 4, out: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Attention of one query token per head (q [q_heads, n], not rotated)
    over a rotated, quantised K/V cache: codes [tokens, kv_heads, n/2] uint8,
    scales [tokens, kv_heads].  Returns out [q_heads, n] float32 in the
    query's space.  The workspace is allocated with torch when not given."""
    q_heads, n, tokens, kv_heads, out = _attention_args(q, s, k_codes, k_scales, v_codes,
                                                        v_scales, bits, out)
    need = hq_decode_attention_workspace(q_heads, kv_heads, tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_dev(workspace, "workspace")
    st = load().hq_decode_attention(q.data_ptr(), _TORCH_TO_HQ[q.dtype], q_heads, kv_heads, n,
                                    int(b), s.data_ptr(), tokens, int(bits), k_codes.data_ptr(),
                                    k_scales.data_ptr(), v_codes.data_ptr(), v_scales.data_ptr(),
                                    _TORCH_TO_HQ[k_scales.dtype], out.data_ptr(),
                                    workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                    _stream(stream))
    _raise(st, "hq_decode_attention")
    return out


def hq_decode_attention_noalloc(q: torch.Tensor, s: torch.Tensor, b: int,
                                k_codes: torch.Tensor, k_scales: torch.Tensor,
                                v_codes: torch.Tensor, v_scales: torch.Tensor, bits: int = 4,
                                out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """hq_decode_attention with the library's own per-GPU workspace (no
    allocation inside the library; pass `out` to allocate nothing here
    either).  Calls that overlap on one GPU race."""
    q_heads, n, tokens, kv_heads, out = _attention_args(q, s, k_codes, k_scales, v_codes,
                                                        v_scales, bits, out)
    st = load().hq_decode_attention_noalloc(q.data_ptr(), _TORCH_TO_HQ[q.dtype], q_heads,
                                            kv_heads, n, int(b), s.data_ptr(), tokens, int(bits),
                                            k_codes.data_ptr(), k_scales.data_ptr(),
                                            v_codes.data_ptr(), v_scales.data_ptr(),
                                            _TORCH_TO_HQ[k_scales.dtype], out.data_ptr(),
                                            _stream(stream))
    _raise(st, "hq_decode_attention_noalloc")
    return out


def hq_dequant_rotate_inv(codes: torch.Tensor, scales: torch.Tensor, s: torch.Tensor,
                          b: int, bits: int = 4, out_dtype: torch.dtype = torch.float32,
                          y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Dequantise codes with their row scales and rotate back: y [rows, n]."""
    return _dequant_inv(codes, scales, s, b, bits, None, out_dtype, y, stream)


def hq_dequant_rotate_inv_grouped(codes: torch.Tensor, scales: torch.Tensor, s: torch.Tensor,
                                  b: int, group: int, bits: int = 4,
                                  out_dtype: torch.dtype = torch.float32,
                                  y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Dequantise codes with their group scales [rows, n/group] and rotate
    back: y [rows, n]."""
    return _dequant_inv(codes, scales, s, b, bits, int(group), out_dtype, y, stream)


def _dequant_inv(codes, scales, s, b, bits, group, out_dtype, y, stream):
    _check_dev(codes, "codes")
    rows, w = _rows_n(codes, "codes")
    n = w * 2 if bits == 4 else w
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    if codes.dtype not in ((torch.uint8,) if bits == 4 else (torch.int8, torch.uint8)):
        raise ValueError(f"codes dtype {codes.dtype} does not match bits={bits}")
    sshape = (rows,) if group is None else (rows, n // group if group > 0 else 0)
    _check_dev(scales, "scales", None, sshape)
    if scales.dtype not in (torch.float32, torch.float16):
        raise ValueError("scales must be float32 or float16")
    _check_dev(s, "s", torch.int8, (n,))
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be float32 or bfloat16")
    if y is None:
        y = torch.empty((rows, n), dtype=out_dtype, device=codes.device)
    _check_dev(y, "y", out_dtype, (rows, n))
    if group is None:
        st = load().hq_dequant_rotate_inv(codes.data_ptr(), scales.data_ptr(),
                                          _TORCH_TO_HQ[scales.dtype], rows, n, int(b),
                                          s.data_ptr(), int(bits), y.data_ptr(),
                                          _TORCH_TO_HQ[out_dtype], _stream(stream))
        _raise(st, "hq_dequant_rotate_inv")
    else:
        st = load().hq_dequant_rotate_inv_grouped(codes.data_ptr(), scales.data_ptr(),
                                                  _TORCH_TO_HQ[scales.dtype], rows, n, int(b),
                                                  s.data_ptr(), int(bits), group, y.data_ptr(),
                                                  _TORCH_TO_HQ[out_dtype], _stream(stream))
        _raise(st, "hq_dequant_rotate_inv_grouped")
    return y


def hq_rotate(x: torch.Tensor, s: torch.Tensor, b: int, y: torch.Tensor | None = None,
              stream=None) -> torch.Tensor:
    """Rotation only: fp32 [rows, n] rotated rows."""
    _check_dev(x, "x")
    if x.dtype not in _TORCH_TO_HQ:
        raise ValueError(f"x dtype {x.dtype} unsupported")
    rows, n = _rows_n(x, "x")
    _check_dev(s, "s", torch.int8, (n,))
    if y is None:
        y = torch.empty((rows, n), dtype=torch.float32, device=x.device)
    _check_dev(y, "y", torch.float32, (rows, n))
    st = load().hq_rotate(x.data_ptr(), _TORCH_TO_HQ[x.dtype], rows, n, int(b),
                          s.data_ptr(), y.data_ptr(), _stream(stream))
    _raise(st, "hq_rotate")
    return y
