"""Parity rules between the GPU path and the CPU oracle.

TEST INFRASTRUCTURE ONLY (imported by tests/, the smoke check and the
benchmark's CPU-baseline leg).  All expected values come from the oracle;
the GPU outputs are only ever the values under test.

Tolerances (floating point; integer work is bit-exact):
  rotated values   |gpu - oracle| <= 1e-5 * max|oracle row|  (relative to the
                   row's absmax: element-wise relative error is meaningless for
                   coordinates that cancel to nearly zero)
  fp32 scales      |gpu - exact| <= 1e-5 * exact + 2^-149 (the second term is
                   one step of binary32 below its normal range, where the
                   format itself cannot hold 1e-5 relative: a scale there is
                   stored to within half of that step)
  fp16 scales      bit-equal to the oracle's single rounding of the exact
                   scale, except one fp16 step where the exact scale lies
                   within 1e-5 (relative) of the midpoint between the two
  codes            bit-exact, except +-1 where the oracle's pre-rounding value
                   r = x'/scale lies within a window of a .5 boundary:
                   INT4: 1e-5 (absolute, in code units);
                   INT8: 1e-5 * max(1, |r|).  The GPU forms r = y * (qmax/m)
                   in binary32 from y carried in binary32 through up to 12
                   butterfly stages, so |r_gpu - r| is about 2^-23 * |r| plus
                   qmax times the relative error of y against the row maximum
                   (measured below 2.5e-7): under 2e-6 code units for INT4,
                   but up to about 3e-5 at |r| ~ 127 for INT8, which an
                   absolute 1e-5 cannot hold (a 128-element INT8 group case
                   landed 1.14e-5 from a tie).
  inverse (fp32)   |gpu - oracle| <= 1e-5 * max|oracle row|
  inverse (bf16)   |gpu - oracle| <= 2^-8 |oracle| + 1e-5 * max|oracle row|
                   (one round-to-nearest-even step of an fp32 value that is
                   itself within 1e-5 of the row max)
"""
from __future__ import annotations

import numpy as np

from . import oracle as O

ROT_TOL = 1e-5
SCALE_TOL = 1e-5
TIE_WINDOW = 1e-5
FP32_SUBNORMAL_STEP = 2.0 ** -149


class ParityError(AssertionError):
    pass


def _fail(what, detail):
    raise ParityError(f"{what}: {detail}")


def check_rotated(gpu: np.ndarray, xr: np.ndarray, what: str = "rotated") -> dict:
    gpu = np.asarray(gpu, dtype=np.float64)
    rowmax = np.abs(xr).max(axis=1, keepdims=True)
    err = np.abs(gpu - xr)
    lim = ROT_TOL * np.maximum(rowmax, np.finfo(np.float64).tiny)
    bad = err > lim
    if bad.any():
        r, c = np.argwhere(bad)[0]
        _fail(what, f"{bad.sum()} elements out of tolerance; first at row {r} col {c}: "
                    f"gpu {gpu[r, c]!r} oracle {xr[r, c]!r} rowmax {rowmax[r, 0]!r}")
    rel = float((err / np.maximum(rowmax, 1e-300)).max()) if err.size else 0.0
    return {"max_err_rel_rowmax": rel}


def check_scales(gpu: np.ndarray, ref: dict, scale_dtype: int, what: str = "scales") -> dict:
    """Per-row scales [rows] or group-wise scales [rows, n/group] (compared
    flat, one entry per scale)."""
    exact = np.ravel(ref["scale_exact"])
    gpu = np.ravel(np.asarray(gpu))
    if scale_dtype == O.F32:
        g = np.asarray(gpu, dtype=np.float64)
        err = np.abs(g - exact)
        bad = err > SCALE_TOL * exact + FP32_SUBNORMAL_STEP
        bad |= (exact == 0) & (g != 0)
        if bad.any():
            i = int(np.argmax(bad))
            _fail(what, f"{bad.sum()} rows out of tolerance; row {i}: gpu {g[i]!r} exact {exact[i]!r}")
        rel = float((err / np.where(exact > 0, exact, 1)).max()) if err.size else 0.0
        return {"max_rel": rel, "fp16_step_rows": 0}
    g16 = np.asarray(gpu).view(np.uint16) if np.asarray(gpu).dtype != np.uint16 else np.asarray(gpu)
    o16 = np.ravel(np.asarray(ref["scales"])).view(np.uint16)
    diff = g16 != o16
    steps = 0
    if diff.any():
        gv = g16.view(np.float16).astype(np.float64)
        ov = o16.view(np.float16).astype(np.float64)
        one_step = np.abs(g16.astype(np.int64) - o16.astype(np.int64)) == 1
        mid = (gv + ov) / 2
        near_mid = np.abs(exact - mid) <= SCALE_TOL * exact
        ok = one_step & near_mid
        bad = diff & ~ok
        if bad.any():
            i = int(np.argmax(bad))
            _fail(what, f"{bad.sum()} fp16 scales differ; row {i}: gpu {gv[i]!r} oracle {ov[i]!r} "
                        f"exact {exact[i]!r}")
        steps = int(diff.sum())
    return {"max_rel": 0.0, "fp16_step_rows": steps}


def check_codes(gpu_codes: np.ndarray, ref: dict, bits: int, n: int,
                what: str = "codes", exact: bool = False) -> dict:
    """exact=True: no tie window at all (inputs built so that every step of
    the GPU's arithmetic is exact)."""
    g = O.unpack_codes(np.asarray(gpu_codes).view(np.uint8), bits, n)
    o = O.unpack_codes(ref["codes"], bits, n)
    diff = g != o
    if exact and diff.any():
        r, c = np.argwhere(diff)[0]
        _fail(what, f"{diff.sum()} codes differ with no tie window allowed; first row {r} "
                    f"col {c}: gpu {g[r, c]} oracle {o[r, c]}")
    ties = 0
    if diff.any():
        pre = ref["preround"]
        if pre is None:
            _fail(what, "codes differ and no pre-rounding values were kept")
        frac = np.abs(pre - np.floor(pre))
        window = TIE_WINDOW if bits == 4 else TIE_WINDOW * np.maximum(1.0, np.abs(pre))
        near_tie = np.abs(frac - 0.5) <= window
        ok = (np.abs(g - o) == 1) & near_tie
        bad = diff & ~ok
        if bad.any():
            r, c = np.argwhere(bad)[0]
            _fail(what, f"{bad.sum()} codes differ outside the tie window; first row {r} col {c}: "
                        f"gpu {g[r, c]} oracle {o[r, c]} pre-round {pre[r, c]!r}")
        ties = int(diff.sum())
    return {"tie_flips": ties, "elements": int(g.size)}


def check_inverse(gpu: np.ndarray, y: np.ndarray, bf16: bool, what: str = "inverse") -> dict:
    g = np.asarray(gpu, dtype=np.float64)
    rowmax = np.abs(y).max(axis=1, keepdims=True)
    lim = ROT_TOL * rowmax
    if bf16:
        lim = lim + np.abs(y) * 2.0 ** -8
    err = np.abs(g - y)
    bad = err > lim
    if bad.any():
        r, c = np.argwhere(bad)[0]
        _fail(what, f"{bad.sum()} elements out of tolerance; first row {r} col {c}: gpu {g[r, c]!r} "
                    f"oracle {y[r, c]!r}")
    return {"max_err_rel_rowmax": float((err / np.maximum(rowmax, 1e-300)).max()) if err.size else 0.0}


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return O.decode(np.asarray(bits).view(np.uint16), O.BF16)
