"""GPU parity of full-width rotations whose width is not a power of two:
H_n = H_k (x) H_(n/k), H_k from Paley's first construction (the Kronecker
route of [RQ] "旋转量化：大模型低比特量化中的离群值克星" section 2.1, for the full-width
block size of the [MS] "QuaRot：基于旋转的离群值抑制算法说明" YAML table).

Widths: 48 = 12 x 4, 96 = 12 x 8, 160 = 20 x 8, 688 = 344 x 2, the FFN
width 11008 = 344 x 32 (Paley over GF(7^3): the matrix-core kernels, the
forward on a dense chunk layout with a helper wave, rotation only and the
inverse in block-circulant form) and 10624 = 332 x 32, 11136 = 348 x 32 (prime fields: the dense
matrix-core kernel).  Inputs are seeded Gaussians
with outlier channels; expected values come from the oracle only, with the
tolerances of oracle/parity.py.
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    G.require_gpu()


def _input(seed, rows, n, x_dtype, outliers=3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, n), dtype=np.float32)
    cols = rng.choice(n, size=outliers, replace=False)
    x[:, cols] *= np.float32(50.0)
    s = np.where(rng.integers(0, 2, n) == 1, 1, -1).astype(np.int8)
    if x_dtype == W.F32:
        return x, s
    if x_dtype == W.BF16:
        return W.to_bf16_bits(x), s
    return x.astype(np.float16).view(np.uint16), s


CASES = [
    (48, 37, W.BF16, 4, W.F16),
    (96, 64, W.F32, 8, W.F32),
    (96, 130, W.F16, 4, W.F32),
    (160, 33, W.BF16, 8, W.F16),
    (688, 19, W.BF16, 4, W.F32),
    (11008, 6, W.BF16, 4, W.F32),
    (11008, 3, W.F32, 8, W.F16),
    (10624, 5, W.BF16, 4, W.F32),
    (11136, 4, W.F16, 8, W.F32),
]


@pytest.mark.parametrize("n,rows,x_dtype,bits,sd", CASES)
def test_rotate_quant_and_inverse(n, rows, x_dtype, bits, sd):
    print(f"[paley] n={n} rows={rows} x={x_dtype} bits={bits} sd={sd}", flush=True)
    raw, s = _input(n + rows, rows, n, x_dtype)
    ref = O.rotate_quant(raw, x_dtype, n, s, bits, sd)
    codes, scales = G.gpu_rotate_quant(raw, x_dtype, s, n, bits, sd)
    P.check_codes(codes, ref, bits, n, what=f"n={n} codes")
    P.check_scales(scales, ref, sd, what=f"n={n} scales")
    y_ref = O.dequant_rotate_inv(ref["codes"], ref["scales"], sd, n, s, bits, n)
    y = G.gpu_dequant_inv(ref["codes"], ref["scales"], s, n, bits)
    P.check_inverse(y, y_ref, bf16=False, what=f"n={n} inverse f32")
    yb = G.gpu_dequant_inv(ref["codes"], ref["scales"], s, n, bits, out_bf16=True)
    P.check_inverse(P.bf16_bits_to_f64(yb), y_ref, bf16=True, what=f"n={n} inverse bf16")


@pytest.mark.parametrize("n,rows,x_dtype", [(96, 33, W.BF16), (688, 9, W.F32), (11008, 4, W.BF16)])
def test_rotate_only(n, rows, x_dtype):
    print(f"[paley] rotate n={n} rows={rows}", flush=True)
    raw, s = _input(7 * n + rows, rows, n, x_dtype)
    xr = O.rotate(O.decode(raw, x_dtype), s, n)
    P.check_rotated(G.gpu_rotate(raw, x_dtype, s, n), xr, what=f"n={n} rotated")


@pytest.mark.parametrize("n,rows,group,bits", [(96, 20, 32, 4), (688, 7, 16, 8), (11008, 3, 128, 4)])
def test_grouped(n, rows, group, bits):
    print(f"[paley] grouped n={n} group={group}", flush=True)
    raw, s = _input(3 * n + group, rows, n, W.BF16)
    ref = O.rotate_quant(raw, W.BF16, n, s, bits, W.F32, group=group)
    codes, scales = G.gpu_rotate_quant_grouped(raw, W.BF16, s, n, group, bits, W.F32)
    P.check_codes(codes, ref, bits, n, what=f"n={n} g={group} codes")
    P.check_scales(scales, ref, W.F32, what=f"n={n} g={group} scales")
    y_ref = O.dequant_rotate_inv(ref["codes"], ref["scales"], W.F32, n, s, bits, n, group=group)
    y = G.gpu_dequant_inv_grouped(ref["codes"], ref["scales"], s, n, group, bits)
    P.check_inverse(y, y_ref, bf16=False, what=f"n={n} g={group} inverse")


def test_append_into_cache():
    n, rows, cache_rows = 688, 5, 40
    print(f"[paley] append n={n}", flush=True)
    raw, s = _input(99, rows, n, W.BF16)
    ref = O.rotate_quant(raw, W.BF16, n, s, 4, W.F16)
    dst = np.array([3, 39, 0, 17, 40], dtype=np.int64)  # the last one lies outside
    codes = torch.zeros((cache_rows, n // 2), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((cache_rows,), dtype=torch.float16, device="cuda")
    hq.hq_rotate_quant_append(G.to_dev(raw, W.BF16), G.s_dev(s), n, torch.from_numpy(dst).cuda(),
                              codes, scales, 4)
    torch.cuda.synchronize()
    c = codes.cpu().numpy()
    sc = scales.cpu().numpy()
    for r, d in enumerate(dst):
        if d >= cache_rows:
            continue
        one = {k: (v[r:r + 1] if isinstance(v, np.ndarray) and v.ndim >= 1 and len(v) == rows else v)
               for k, v in ref.items()}
        P.check_codes(c[d:d + 1], one, 4, n, what=f"append row {r}")
        P.check_scales(sc[d:d + 1], one, W.F16, what=f"append row {r}")
    untouched = np.setdiff1d(np.arange(cache_rows), dst)
    assert not c[untouched].any() and not sc[untouched].view(np.uint16).any()


@pytest.mark.parametrize("x_dtype,bits", [(W.BF16, 4), (W.F16, 8), (W.BF16, 8)])
def test_11008_many_rows_sampled(x_dtype, bits):
    # more rows than workgroups: every workgroup walks several rows; the
    # oracle checks a sample of them (rows are independent)
    n, rows = 11008, 600
    print(f"[paley] 11008 x {rows} x={x_dtype} bits={bits}", flush=True)
    raw, s = _input(1234 + bits, rows, n, x_dtype, outliers=11)
    codes, scales = G.gpu_rotate_quant(raw, x_dtype, s, n, bits, W.F32)
    pick = np.array([0, 1, 127, 255, 256, 257, 300, 511, 512, 513, 599])
    ref = O.rotate_quant(raw[pick], x_dtype, n, s, bits, W.F32)
    P.check_codes(codes[pick], ref, bits, n, what=f"11008 sampled codes")
    P.check_scales(scales[pick], ref, W.F32, what=f"11008 sampled scales")


def test_ffn_11008_full_at_full_size_first_and_last_rows():
    # the benchmarked call: 16384 x 11008 from the workload's own generator,
    # in the launch configuration bench.py times (512 workgroups, workgroup
    # b taking rows b, b + 512, ...).  The oracle checks rows 0 .. 1023 and
    # 15360 .. 16383: the first two and the last two rows of every
    # workgroup, i.e. each one's pipeline start and end, 2048 rows in all
    # (every row would cost the oracle minutes).  Then the inverse of the
    # oracle's codes for the same rows at the benchmarked size (fp32 out).
    w = W.WORKLOADS["ffn_11008_full"]
    data = W.generate("ffn_11008_full", seed=42)
    raw, s = data["x"], data["s"]
    pick = np.r_[0:1024, raw.shape[0] - 1024:raw.shape[0]]
    print(f"[paley] ffn_11008_full {raw.shape} forward", flush=True)
    codes, scales = G.gpu_rotate_quant(raw, w.x_dtype, s, w.b, w.bits, w.scale_dtype)
    ref = O.rotate_quant(raw[pick], w.x_dtype, w.b, s, w.bits, w.scale_dtype)
    st = P.check_codes(codes[pick], ref, w.bits, w.n, what="ffn_11008_full codes")
    P.check_scales(scales[pick], ref, w.scale_dtype, what="ffn_11008_full scales")
    print(f"[paley] ffn_11008_full codes ok ({st['tie_flips']} tie flips of {st['elements']})", flush=True)
    # the inverse at the benchmarked size: the oracle's codes for the picked
    # rows, the GPU's own codes elsewhere (the launch shape is the same)
    all_codes = codes.copy()
    all_codes[pick] = ref["codes"]
    all_scales = scales.copy()
    all_scales[pick] = ref["scales"]
    del codes, scales, raw
    print("[paley] ffn_11008_full inverse", flush=True)
    y = G.gpu_dequant_inv(all_codes, all_scales, s, w.n, w.bits)
    y_ref = O.dequant_rotate_inv(ref["codes"], ref["scales"], w.scale_dtype, w.n, s, w.bits, w.n)
    P.check_inverse(y[pick], y_ref, bf16=False, what="ffn_11008_full inverse f32")


@pytest.mark.parametrize("bits,sd", [(4, W.F32), (8, W.F16)])
def test_11008_inverse_many_rows_sampled(bits, sd):
    # the inverse over more rows than workgroups (each walks several rows
    # through its two staging buffers); seeded codes in [-qmax, qmax] and
    # positive scales as inputs, the oracle on a sample of rows
    n, rows = 11008, 600
    print(f"[paley] inverse 11008 x {rows} bits={bits}", flush=True)
    rng = np.random.default_rng(77 + bits)
    qmax = (1 << (bits - 1)) - 1
    q = rng.integers(-qmax, qmax + 1, size=(rows, n))
    if bits == 4:
        codes = ((q[:, 0::2] & 15) | ((q[:, 1::2] & 15) << 4)).astype(np.uint8)
    else:
        codes = q.astype(np.int8).view(np.uint8)
    scales = (rng.random(rows) * 0.5 + 0.01).astype(np.float32)
    if sd == W.F16:
        scales = scales.astype(np.float16)
    s = np.where(rng.integers(0, 2, n) == 1, 1, -1).astype(np.int8)
    pick = np.array([0, 1, 127, 255, 256, 257, 300, 511, 512, 513, 599])
    y_ref = O.dequant_rotate_inv(codes[pick], scales[pick], sd, n, s, bits, n)
    y = G.gpu_dequant_inv(codes, scales, s, n, bits)
    P.check_inverse(y[pick], y_ref, bf16=False, what=f"11008 inverse bits={bits} f32")
    yb = G.gpu_dequant_inv(codes, scales, s, n, bits, out_bf16=True)
    P.check_inverse(P.bf16_bits_to_f64(yb[pick]), y_ref, bf16=True, what=f"11008 inverse bits={bits} bf16")


def test_11008_rotate_many_rows_sampled():
    # rotation only over more rows than workgroups; the oracle on a sample
    n, rows = 11008, 600
    print(f"[paley] rotate 11008 x {rows}", flush=True)
    raw, s = _input(4321, rows, n, W.BF16, outliers=11)
    y = G.gpu_rotate(raw, W.BF16, s, n)
    pick = np.array([0, 1, 255, 256, 257, 511, 512, 599])
    xr = O.rotate(O.decode(raw[pick], W.BF16), s, n)
    P.check_rotated(y[pick], xr, what="11008 rotated, sampled rows")


def test_11008_tiny_and_zero_rows_across_the_pipeline():
    # Rows far below binary32's range for qmax / max (down to subnormal
    # inputs) and zero rows, mixed with ordinary rows over enough rows that
    # every workgroup of the 11008-wide forward codes several of them: the
    # codes of a row are written one row later, a third by the product waves
    # and the rest by the helper wave, each with its own magnification path.
    n, rows = 11008, 1100
    rng = np.random.default_rng(11008)
    raw = rng.standard_normal((rows, n), dtype=np.float32)
    raw[::7] = 0.0
    tiny = raw[3::7]
    tiny[:] = 0.0
    tiny[0::3, 5] = 1.5 * 2.0 ** -127                    # subnormal
    tiny[1::3, :] = 2.0 ** -110
    tiny[2::3, 3] = 2.0 ** -133                          # subnormal
    tiny[2::3, n // 2] = -3 * 2.0 ** -133
    raw[3::7] = tiny
    raw[5::7] = 0.0
    raw[5::7, 1::97] = 2.0 ** -126 * (1 + np.arange(len(range(1, n, 97))) % 64)
    x = (raw.view(np.uint32) >> 16).astype(np.uint16)  # exact in bf16
    s = np.where(np.arange(n) % 5 == 0, -1, 1).astype(np.int8)
    for bits in (4, 8):
        tag = f"11008 tiny/zero rows bits={bits}"
        print(f"[paley] {tag}", flush=True)
        codes, scales = G.gpu_rotate_quant(x, W.BF16, s, n, bits, W.F32)
        ref = O.rotate_quant(x, W.BF16, n, s, bits, W.F32)
        P.check_codes(codes, ref, bits, n, what=tag)
        P.check_scales(scales, ref, W.F32, what=tag)
