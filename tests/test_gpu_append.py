"""GPU parity of hq_rotate_quant_append: rotate + quantise a few new rows into
a preallocated cache at given rows (the online K/V rotation into a 4-bit
cache of "手把手教你用QuaRot实现LLM的4位量化：从原理到代码实践" section 2.2,
one decode step at a time).

Expected values come from the oracle only: each appended row must equal the
oracle's codes and scale of its input row (the tolerances of oracle/parity.py);
every other cache row must keep its sentinel bytes; rows whose index lies
outside the cache write nothing.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import hadamard_rotation_amd as hq
from hadamard_rotation_amd import workloads as W
from oracle import oracle as O
from oracle import parity as P
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

SENTINEL = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    G.require_gpu()


def _append_case(n, b, x_dtype, bits, sd, cache_rows, rows, seed, bad=()):
    tag = f"n={n} b={b} dt={x_dtype} bits={bits} sd={sd} rows={rows}"
    print(f"[append] {tag}", flush=True)
    raw, s = W.random_rows(seed, rows, n, x_dtype, outliers=2)
    rng = np.random.default_rng(seed + 1)
    dst = rng.choice(cache_rows, size=rows, replace=False).astype(np.int64)
    for i, v in bad:  # indices outside the cache: skipped
        dst[i] = v
    cw = n // 2 if bits == 4 else n
    codes = torch.full((cache_rows, cw), SENTINEL, dtype=torch.uint8, device="cuda")
    if bits == 8:
        codes = codes.view(torch.int8)
    st = torch.float32 if sd == W.F32 else torch.float16
    scales = torch.full((cache_rows,), -3.0, dtype=st, device="cuda")
    hq.hq_rotate_quant_append(G.to_dev(raw, x_dtype), G.s_dev(s), b,
                              torch.from_numpy(dst).cuda(), codes, scales, bits)
    torch.cuda.synchronize()
    c = codes.cpu().numpy().view(np.uint8)
    sc = scales.cpu().numpy()
    live = (dst >= 0) & (dst < cache_rows)
    ref = O.rotate_quant(raw[live], x_dtype, b, s, bits, sd)
    rows_w = dst[live]
    P.check_codes(c[rows_w], ref, bits, n, what=f"{tag} codes")
    P.check_scales(sc[rows_w], ref, sd, what=f"{tag} scales")
    untouched = np.ones(cache_rows, dtype=bool)
    untouched[rows_w] = False
    assert np.all(c[untouched] == SENTINEL), tag
    assert np.all(sc[untouched] == -3.0), tag
    return raw, s, dst, live, c, sc


CASES = [  # (n, b, x_dtype): matrix-core append and the generic kernel
    (128, 128, W.BF16), (128, 128, W.F16), (256, 128, W.BF16), (512, 512, W.BF16),
    (1024, 1024, W.BF16), (4096, 4096, W.BF16), (4096, 128, W.BF16),
    (128, 128, W.F32), (11008, 128, W.BF16), (48, 16, W.BF16),
]


@pytest.mark.parametrize("n,b,x_dtype", CASES)
def test_append_shapes(n, b, x_dtype):
    cache_rows = 4096 if n <= 512 else 300
    for rows in (1, 7, 64, 133):
        for bits, sd in ((4, W.F16), (8, W.F32)):
            _append_case(n, b, x_dtype, bits, sd, cache_rows, min(rows, cache_rows // 2),
                         seed=n + rows + bits)


def test_append_skips_rows_outside_the_cache():
    for n, b in ((128, 128), (4096, 4096), (11008, 128)):
        cache_rows = 512 if n == 128 else 64
        _append_case(n, b, W.BF16, 4, W.F16, cache_rows, 21, seed=5,
                     bad=((0, -1), (3, cache_rows), (9, 2 ** 40), (20, -(2 ** 62))))


def test_append_decode_step_round_trip():
    # a decode step of a 8-head K cache: 40 sequences append one token each at
    # their own positions; dequantising the cache rows gives back the rows
    heads, n = 8, 128
    positions = 2048
    cache_rows = positions * heads
    raw, s = W.random_rows(11, 40 * heads, n, W.BF16, outliers=1)
    rng = np.random.default_rng(12)
    pos = rng.choice(positions, size=40, replace=False)
    dst = (pos[:, None] * heads + np.arange(heads)[None, :]).reshape(-1).astype(np.int64)
    codes = torch.full((cache_rows, n // 2), SENTINEL, dtype=torch.uint8, device="cuda")
    scales = torch.zeros((cache_rows,), dtype=torch.float16, device="cuda")
    hq.hq_rotate_quant_append(G.to_dev(raw, W.BF16), G.s_dev(s), n,
                              torch.from_numpy(dst).cuda(), codes, scales, 4)
    y = hq.hq_dequant_rotate_inv(codes[torch.from_numpy(dst).cuda()].contiguous(),
                                 scales[torch.from_numpy(dst).cuda()].contiguous(),
                                 G.s_dev(s), n, 4)
    torch.cuda.synchronize()
    ref = O.rotate_quant(raw, W.BF16, n, s, 4, W.F16)
    y_ref = O.dequant_rotate_inv(ref["codes"], ref["scales"], W.F16, n, s, 4, n)
    same = np.all(O.unpack_codes(codes.cpu().numpy()[dst], 4, n) ==
                  O.unpack_codes(ref["codes"], 4, n), axis=1)
    assert same.mean() > 0.9
    P.check_inverse(y.cpu().numpy()[same], y_ref[same], bf16=False, what="append round trip")
