"""GPU codes at exact .5 ties: round half to even, with no tie window.

The pages round with numpy's and torch's round, i.e. half to even
("旋转量化：大模型低比特量化中的离群值克星" section 2.2, the quantisation-error
snippet; "哈特曼旋转，轻量级QAT，流式注意力" section 1).  The rows come from
tests/ties.py: small integers whose rotated values make x'/scale = y/4 exact
in every step of the GPU's fp32 arithmetic, with a large share of them on a
.5 boundary.  The codes must then equal the oracle's bit for bit
(check_codes(exact=True)), which the normal +-1 tie window would not catch
for a kernel that rounded ties away from zero or truncated them.

One case per kernel family: the matrix-core kernels (16-bit input, full and
128-blocks, per-row, whole-tile and sub-tile groups, 128-block rows of wider
rows, long rows with one scale per row, cache append), the butterfly kernel
(fp32 input, long rows), the generic kernel, and the Paley kernels (generic
for 96, block-circulant for 11008, dense for 10624).
"""
from __future__ import annotations

import numpy as np
import pytest

from hadamard_rotation_amd import workloads as W
from oracle import oracle as O
from oracle import parity as P
from tests import gpu_util as G
from tests.ties import exact_ties, tie_rows, to_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    G.require_gpu()


def _case(n, b, dtype, bits, rows, seed, group=None):
    rng = np.random.default_rng(seed)
    s = np.where(rng.integers(0, 2, n) == 1, 1, -1).astype(np.int8)
    H = O.hadamard(b)
    x = tie_rows(H, rows, n, s, bits, rng)
    return to_dtype(x, dtype), s


# (n, b, input dtype, rows, group or None)
CASES = [
    (64, 64, W.BF16, 67, None),        # matrix core, rows of 64
    (64, 64, W.F16, 67, None),
    (128, 128, W.BF16, 131, None),     # matrix core, b = 128 (sqrt(b) irrational)
    (256, 256, W.F16, 41, None),
    (512, 128, W.BF16, 37, None),      # matrix core, 128-blocks of a 512 row
    (1024, 1024, W.F16, 9, None),
    (4096, 4096, W.BF16, 5, None),     # matrix core, the headline shape
    (4096, 128, W.BF16, 5, 128),       # matrix core, sub-tile groups (transposed)
    (4096, 128, W.BF16, 5, 512),       # matrix core, whole-tile groups
    (11008, 128, W.BF16, 3, 128),      # matrix core, one workgroup per long row, block scales
    (640, 128, W.F16, 9, 128),         # the same, a partial last tile
    (16512, 128, W.BF16, 2, 128),      # matrix core, 128-block rows of wide rows
    (128, 128, W.F32, 67, None),       # butterfly kernel
    (4096, 4096, W.F32, 5, None),
    (11008, 128, W.F32, 3, None),      # butterfly kernel, long rows
    (11008, 128, W.BF16, 3, None),     # matrix core, one workgroup per long row
    (640, 128, W.F16, 9, None),        # the same, a partial last tile
    (32768, 4096, W.F32, 2, None),     # generic kernel
    (96, 96, W.F32, 33, None),         # Paley 12 x 8, generic kernel
    (11008, 11008, W.BF16, 3, None),   # Paley 344 x 32, block-circulant kernel
    (10624, 10624, W.BF16, 2, None),   # Paley 332 x 32, dense kernel
]


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("n,b,dtype,rows,group", CASES)
def test_exact_ties_round_half_to_even(n, b, dtype, rows, group, bits):
    tag = f"ties n={n} b={b} dt={dtype} g={group} bits={bits}"
    print(f"[ties] {tag}", flush=True)
    x, s = _case(n, b, dtype, bits, rows, seed=7 * n + b + bits)
    ref = O.rotate_quant(x, dtype, b, s, bits, W.F32, group=group)
    assert exact_ties(ref["preround"]) > x.size // 8
    if group is None:
        codes, scales = G.gpu_rotate_quant(x, dtype, s, b, bits, W.F32)
    else:
        codes, scales = G.gpu_rotate_quant_grouped(x, dtype, s, b, group, bits, W.F32)
    P.check_codes(codes, ref, bits, n, what=tag, exact=True)
    P.check_scales(scales, ref, W.F32, what=tag)


def test_exact_ties_cache_append():
    # the append mode of the matrix-core kernel writes the same codes
    import torch
    import hadamard_rotation_amd as hq
    n, rows, cache_rows = 128, 64, 1000
    x, s = _case(n, n, W.BF16, 4, rows, seed=11)
    ref = O.rotate_quant(x, W.BF16, n, s, 4, W.F16)
    dst = np.random.default_rng(3).choice(cache_rows, rows, replace=False).astype(np.int64)
    codes = torch.zeros((cache_rows, n // 2), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((cache_rows,), dtype=torch.float16, device="cuda")
    hq.hq_rotate_quant_append(G.to_dev(x, W.BF16), G.s_dev(s), n,
                              torch.from_numpy(dst).cuda(), codes, scales, 4)
    torch.cuda.synchronize()
    got = codes.cpu().numpy()[dst]
    P.check_codes(got, ref, 4, n, what="ties append", exact=True)
