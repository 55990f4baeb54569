"""ctypes front-end of the CPU oracle in ``hq_oracle.c``.

TEST INFRASTRUCTURE ONLY: imported by the test suite, by the smoke check and
by the CPU-baseline leg of the benchmark, never by the product package.  It
shares no code with the HIP path; inputs reach it as host numpy arrays.

Pages cited (see the C file for the definitions it follows):
  [RQ] "旋转量化：大模型低比特量化中的离群值克星", sections 2.1 and 2.2.
  [QT] "手把手教你用QuaRot实现LLM的4位量化：从原理到代码实践", section 2.1.

Every function here is pinned by ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

# element types, the oracle's own numbering
F32, BF16, F16 = 0, 1, 2

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile hq_oracle.c into oracle/liboracle.so with gcc (plain -O2, no
    fast-math, so fp64 arithmetic is IEEE)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-Wall", "-fPIC", "-shared", "-pthread",
             _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        P, I, L = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        lib.hqo_hadamard.argtypes = [I, P]
        lib.hqo_paley.argtypes = [I, P]
        lib.hqo_hadamard_split.argtypes = [I, P, P]
        lib.hqo_decode.argtypes = [P, I, L, P]
        lib.hqo_rotate.argtypes = [P, L, I, I, P, P, I]
        lib.hqo_rotate_quant.argtypes = [P, I, L, I, I, P, I, P, P, I, P, P, P, I]
        lib.hqo_rotate_quant_g.argtypes = [P, I, L, I, I, P, I, I, P, P, I, P, P, P, I]
        lib.hqo_dequant_rotate_inv.argtypes = [P, P, I, L, I, I, P, I, P, I]
        lib.hqo_dequant_rotate_inv_g.argtypes = [P, P, I, L, I, I, P, I, I, P, I]
        lib.hqo_decode_attention.argtypes = [P, I, I, I, I, I, P, L, I, P, P, P, P, I, P]
        lib.hqo_f64_to_f16.argtypes = [ctypes.c_double]
        lib.hqo_f64_to_f16.restype = ctypes.c_uint16
        lib.hqo_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.hqo_f16_to_f64.restype = ctypes.c_double
        lib.hqo_default_threads.restype = ctypes.c_int
        for f in (lib.hqo_hadamard, lib.hqo_paley, lib.hqo_hadamard_split, lib.hqo_decode, lib.hqo_rotate,
                  lib.hqo_rotate_quant, lib.hqo_rotate_quant_g,
                  lib.hqo_dequant_rotate_inv, lib.hqo_dequant_rotate_inv_g,
                  lib.hqo_decode_attention):
            f.restype = ctypes.c_int
        _lib = lib
        return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def default_threads() -> int:
    return int(_load().hqo_default_threads())


def dtype_code(raw: np.ndarray, name: str | None = None) -> int:
    """Element type of a raw input array: float32 -> F32, float16 -> F16,
    uint16/int16 bit patterns -> BF16 unless name says 'f16'."""
    if raw.dtype == np.float32:
        return F32
    if raw.dtype == np.float16:
        return F16
    if raw.dtype in (np.uint16, np.int16):
        return F16 if name == "f16" else BF16
    raise TypeError(f"unsupported raw dtype {raw.dtype}")


def hadamard(b: int) -> np.ndarray:
    """The Hadamard matrix of order b the library rotates with, entries
    +1/-1: Sylvester for a power of two ([RQ] 2.1), else the Kronecker
    product of a Paley matrix and a Sylvester matrix (hadamard_split)."""
    H = np.empty((b, b), dtype=np.int8)
    _check(_load().hqo_hadamard(int(b), _ptr(H)), "hadamard")
    return H


def paley(k: int) -> np.ndarray:
    """Paley's first construction of order k (k - 1 a prime power = 3 mod 4,
    at most a cube), entries +1/-1."""
    H = np.empty((k, k), dtype=np.int8)
    _check(_load().hqo_paley(int(k), _ptr(H)), "paley")
    return H


def hadamard_split(n: int) -> tuple[int, int] | None:
    """(k, m2) with n = k * m2, m2 a power of two and k the Paley order the
    library uses (k = 1 when n is a power of two), or None."""
    k, m2 = ctypes.c_int(0), ctypes.c_int(0)
    rc = _load().hqo_hadamard_split(int(n), ctypes.byref(k), ctypes.byref(m2))
    return None if rc != 0 else (k.value, m2.value)


def decode(raw: np.ndarray, dtype: int) -> np.ndarray:
    """Exact widening of f32 / bf16 / f16 storage to float64."""
    raw = np.ascontiguousarray(raw)
    out = np.empty(raw.shape, dtype=np.float64)
    _check(_load().hqo_decode(_ptr(raw), int(dtype), raw.size, _ptr(out)), "decode")
    return out


def rotate(x: np.ndarray, s: np.ndarray, b: int, threads: int = 0) -> np.ndarray:
    """x' = blockwise (x*s).H_b/sqrt(b) of float64 rows [rows, n]."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    s = np.ascontiguousarray(s, dtype=np.int8)
    rows, n = x.shape
    out = np.empty_like(x)
    _check(_load().hqo_rotate(_ptr(x), rows, n, int(b), _ptr(s), _ptr(out), threads),
           "rotate")
    return out


def rotate_quant(raw: np.ndarray, x_dtype: int, b: int, s: np.ndarray, bits: int,
                 scale_dtype: int, threads: int = 0, want_xr: bool = False,
                 want_preround: bool = True, group: int | None = None) -> dict:
    """Rotation + symmetric quantisation of raw rows [rows, n], one scale per
    row (group None) or per run of `group` consecutive rotated elements.

    Returns a dict with
      codes        uint8 [rows, n/2] (bits 4) or [rows, n] (bits 8)
      scales       stored scales: float32, or float16 when scale_dtype is F16;
                   [rows] per row, [rows, n/group] per group
      scale_exact  float64, same shape: absmax/qmax before storage rounding
      preround     float64 [rows, n], x'/scale_exact (if want_preround)
      xr           float64 [rows, n], the rotated row (if want_xr)
    """
    raw = np.ascontiguousarray(raw)
    s = np.ascontiguousarray(s, dtype=np.int8)
    rows, n = raw.shape
    g = n if group is None else int(group)
    sshape = (rows,) if group is None else (rows, n // g if g > 0 else 0)
    codes = np.empty((rows, n // 2 if bits == 4 else n), dtype=np.uint8)
    scales = np.empty(sshape, dtype=np.float32 if scale_dtype == F32 else np.uint16)
    scale_exact = np.empty(sshape, dtype=np.float64)
    pre = np.empty((rows, n), dtype=np.float64) if want_preround else None
    xr = np.empty((rows, n), dtype=np.float64) if want_xr else None
    rc = _load().hqo_rotate_quant_g(
        _ptr(raw), int(x_dtype), rows, n, int(b), _ptr(s), int(bits), g, _ptr(codes),
        _ptr(scales), int(scale_dtype), _ptr(scale_exact),
        _ptr(pre) if pre is not None else None,
        _ptr(xr) if xr is not None else None, threads)
    _check(rc, "rotate_quant")
    if scale_dtype == F16:
        scales = scales.view(np.float16)
    return {"codes": codes, "scales": scales, "scale_exact": scale_exact,
            "preround": pre, "xr": xr}


def dequant_rotate_inv(codes: np.ndarray, scales: np.ndarray, scale_dtype: int,
                       b: int, s: np.ndarray, bits: int, n: int,
                       threads: int = 0, group: int | None = None) -> np.ndarray:
    """y = ((q*scale_stored).H_b/sqrt(b)) * s, float64 [rows, n]; scales per
    row (group None) or [rows, n/group] per group."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales)
    if scale_dtype == F16:
        scales = scales.view(np.uint16)
    s = np.ascontiguousarray(s, dtype=np.int8)
    rows = codes.shape[0]
    g = int(n) if group is None else int(group)
    y = np.empty((rows, n), dtype=np.float64)
    rc = _load().hqo_dequant_rotate_inv_g(_ptr(codes), _ptr(scales), int(scale_dtype),
                                          rows, int(n), int(b), _ptr(s), int(bits), g,
                                          _ptr(y), threads)
    _check(rc, "dequant_rotate_inv")
    return y


def decode_attention(q_raw: np.ndarray, q_dtype: int, kv_heads: int, b: int, s: np.ndarray,
                     k_codes: np.ndarray, k_scales: np.ndarray, v_codes: np.ndarray,
                     v_scales: np.ndarray, scale_dtype: int, bits: int) -> np.ndarray:
    """Decode attention of one query token per head over a rotated,
    quantised K/V cache (hqo_decode_attention): q_raw [q_heads, n] raw values,
    codes [tokens * kv_heads, n/2 or n] (row = token * kv_heads + head),
    scales [tokens * kv_heads].  Returns float64 [q_heads, n] in the query's
    (unrotated) space."""
    q_raw = np.ascontiguousarray(q_raw)
    q_heads, n = q_raw.shape
    s = np.ascontiguousarray(s, dtype=np.int8)
    k_codes = np.ascontiguousarray(k_codes, dtype=np.uint8)
    v_codes = np.ascontiguousarray(v_codes, dtype=np.uint8)
    k_scales = np.ascontiguousarray(k_scales)
    v_scales = np.ascontiguousarray(v_scales)
    if scale_dtype == F16:
        k_scales = k_scales.view(np.uint16)
        v_scales = v_scales.view(np.uint16)
    tokens = k_codes.shape[0] // kv_heads
    out = np.empty((q_heads, n), dtype=np.float64)
    rc = _load().hqo_decode_attention(_ptr(q_raw), int(q_dtype), q_heads, int(kv_heads), n,
                                      int(b), _ptr(s), tokens, int(bits), _ptr(k_codes),
                                      _ptr(k_scales), _ptr(v_codes), _ptr(v_scales),
                                      int(scale_dtype), _ptr(out))
    _check(rc, "decode_attention")
    return out


def f64_to_f16_bits(v: float) -> int:
    return int(_load().hqo_f64_to_f16(float(v)))


def f16_bits_to_f64(h: int) -> float:
    return float(_load().hqo_f16_to_f64(int(h)))


def unpack_codes(codes: np.ndarray, bits: int, n: int) -> np.ndarray:
    """Signed integer codes [rows, n] from the packed storage (element 2j in
    the low nibble, 4-bit two's complement)."""
    codes = np.asarray(codes, dtype=np.uint8)
    if bits == 8:
        return codes.view(np.int8).astype(np.int32)
    lo = (codes & 0xF).astype(np.int32)
    hi = (codes >> 4).astype(np.int32)
    out = np.empty((codes.shape[0], n), dtype=np.int32)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return np.where(out >= 8, out - 16, out)
