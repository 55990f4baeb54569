"""GPU parity at the workloads' full sizes, every row compared with the oracle.

The five workloads stand in for the pages' LLM tensors: hidden width 4096 and
head dimension 128 ("旋转量化：大模型低比特量化中的离群值克星" section 2.1), a
width that is not a power of two rotated in 128-blocks (same section), and
the 4-bit online K/V cache ("手把手教你用QuaRot实现LLM的4位量化：从原理到代码实践"
section 2.2).  Each test runs the whole tensor through the launch the
benchmark times (so the kernel instances a full-size launch selects are the
ones compared) and checks, for every row:
  codes and scales                         all five workloads
  the fp32 rotation itself (hq_rotate)     the INT8 case, Q/K, hidden 4096, FFN 11008
  the fp32 inverse of the oracle's codes   Q/K, hidden 4096, FFN 11008, K/V
  the bf16 inverse as well                 FFN 11008
plus the 11008-wide rows with one scale per 128-block (forward, fp32 and
bf16 inverse) and the 4096-wide rows with 128-element groups.  Tolerances are those of
oracle/parity.py.  The oracle runs on every host core; the largest case
(16384 x 4096) is 2.7e11 multiply-adds, seconds on a 16-thread host.
"""
from __future__ import annotations

import numpy as np
import pytest

from hadamard_rotation_amd import workloads as W
from oracle import oracle as O
from oracle import parity as P
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

ROTATE = ("tiny_int8", "qk_heads", "hidden_4096", "ffn_11008")
INVERSE = ("qk_heads", "hidden_4096", "ffn_11008", "kv_cache")
INVERSE_BF16 = ("ffn_11008",)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    G.require_gpu()


@pytest.mark.parametrize("name", W.ORDER)
def test_full_size_every_row(name):
    w = W.WORKLOADS[name]
    data = W.generate(name, seed=42)
    s = data["s"]
    for t in w.tensors:
        raw = data[t]
        tag = f"{name}/{t} full"
        print(f"[full] {tag} rows={raw.shape[0]} forward", flush=True)
        codes, scales = G.gpu_rotate_quant(raw, w.x_dtype, s, w.b, w.bits, w.scale_dtype)
        ref = O.rotate_quant(raw, w.x_dtype, w.b, s, w.bits, w.scale_dtype,
                             want_xr=name in ROTATE)
        st = P.check_codes(codes, ref, w.bits, w.n, what=f"{tag} codes")
        P.check_scales(scales, ref, w.scale_dtype, what=f"{tag} scales")
        print(f"[full] {tag} codes ok ({st['tie_flips']} tie flips of {st['elements']})",
              flush=True)
        if name in ROTATE:
            y = G.gpu_rotate(raw, w.x_dtype, s, w.b)
            P.check_rotated(y, ref["xr"], what=f"{tag} rotated")
            del y
        ref.pop("xr", None)
        ref.pop("preround", None)
        if name in INVERSE:
            print(f"[full] {tag} inverse", flush=True)
            y_ref = O.dequant_rotate_inv(ref["codes"], ref["scales"], w.scale_dtype, w.b, s,
                                         w.bits, w.n)
            y = G.gpu_dequant_inv(ref["codes"], ref["scales"], s, w.b, w.bits)
            P.check_inverse(y, y_ref, bf16=False, what=f"{tag} inverse f32")
            del y
            if name in INVERSE_BF16:
                yb = G.gpu_dequant_inv(ref["codes"], ref["scales"], s, w.b, w.bits,
                                       out_bf16=True)
                P.check_inverse(P.bf16_bits_to_f64(yb), y_ref, bf16=True,
                                what=f"{tag} inverse bf16")
                del yb
            del y_ref
        if name == "kv_cache":
            # GPU forward -> GPU inverse stays within the orthogonality bound
            # of the input, row by row
            y = G.gpu_dequant_inv(codes, scales, s, w.b, w.bits)
            x = O.decode(raw, w.x_dtype)
            err = np.linalg.norm(y - x, axis=1)
            sc = ref["scales"].astype(np.float64)
            bound = np.sqrt(w.n) / 2 * ref["scale_exact"] * (1 + 1e-3) + \
                np.sqrt(w.n) * 7 * np.abs(sc - ref["scale_exact"]) + 1e-6
            assert np.all(err <= bound), f"{tag} round trip"
            del y, x


@pytest.mark.parametrize("name,group", [("ffn_11008", 128), ("hidden_4096", 128)])
def test_full_size_grouped_every_row(name, group):
    # 16384 x 11008 with one scale per 128-block: the forward runs one
    # workgroup per row on the matrix core, the inverse rows of one block;
    # 16384 x 4096 with 128-element groups takes the sub-tile group reduction
    w = W.WORKLOADS[name]
    data = W.generate(name, seed=42)
    raw, s = data["x"], data["s"]
    tag = f"{name} g={group} full"
    print(f"[full] {tag} forward", flush=True)
    codes, scales = G.gpu_rotate_quant_grouped(raw, w.x_dtype, s, w.b, group, w.bits,
                                               w.scale_dtype)
    ref = O.rotate_quant(raw, w.x_dtype, w.b, s, w.bits, w.scale_dtype, group=group)
    P.check_codes(codes, ref, w.bits, w.n, what=f"{tag} codes")
    P.check_scales(scales, ref, w.scale_dtype, what=f"{tag} scales")
    ref.pop("preround", None)
    print(f"[full] {tag} inverse", flush=True)
    y_ref = O.dequant_rotate_inv(ref["codes"], ref["scales"], w.scale_dtype, w.b, s, w.bits,
                                 w.n, group=group)
    y = G.gpu_dequant_inv_grouped(ref["codes"], ref["scales"], s, w.b, group, w.bits)
    P.check_inverse(y, y_ref, bf16=False, what=f"{tag} inverse f32")
    del y
    yb = G.gpu_dequant_inv_grouped(ref["codes"], ref["scales"], s, w.b, group, w.bits,
                                   out_bf16=True)
    P.check_inverse(P.bf16_bits_to_f64(yb), y_ref, bf16=True, what=f"{tag} inverse bf16")
