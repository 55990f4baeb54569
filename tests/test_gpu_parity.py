"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Inputs come from the seeded generators only; expected values come from the
oracle only.  Reduced sizes span many workgroups and end on a ragged tail
(the full sizes, every row, are in test_gpu_full_size.py).  Tolerances are
the ones in oracle/parity.py.
"""
from __future__ import annotations

import numpy as np
import pytest

from hadamard_rotation_amd import workloads as W
from oracle import oracle as O
from oracle import parity as P
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

SEEDS = (42, 0, 1)

# reduced sizes: (workload, token count) -- chosen so that the row count is
# not a multiple of any launch granularity
REDUCED = {
    "tiny_int8": 64,
    "qk_heads": 133,      # 32 * 133 = 4256 rows
    "hidden_4096": 259,
    "ffn_11008": 37,
    "kv_cache": 517,      # 8 * 517 = 4136 rows
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    G.require_gpu()


def _tensors(name, seed, tokens):
    w = W.WORKLOADS[name]
    data = W.generate(name, seed=seed, tokens=tokens)
    return w, data


def _check_forward(w, raw, s, tag):
    ref = O.rotate_quant(raw, w.x_dtype, w.b, s, w.bits, w.scale_dtype, want_xr=True)
    codes, scales = G.gpu_rotate_quant(raw, w.x_dtype, s, w.b, w.bits, w.scale_dtype)
    st = P.check_codes(codes, ref, w.bits, w.n, what=f"{tag} codes")
    P.check_scales(scales, ref, w.scale_dtype, what=f"{tag} scales")
    y = G.gpu_rotate(raw, w.x_dtype, s, w.b)
    P.check_rotated(y, ref["xr"], what=f"{tag} rotated")
    return ref, codes, scales, st


@pytest.mark.parametrize("seed", SEEDS)
@pytest.mark.parametrize("name", W.ORDER)
def test_workload_reduced(name, seed):
    w, data = _tensors(name, seed, REDUCED[name])
    for t in w.tensors:
        print(f"[parity] {name} seed={seed} tensor={t} rows={data[t].shape[0]}", flush=True)
        ref, codes, scales, _ = _check_forward(w, data[t], data["s"], f"{name}/{t}/seed{seed}")
        # inverse on the oracle's own codes and scales
        y_ref = O.dequant_rotate_inv(ref["codes"], ref["scales"], w.scale_dtype, w.b,
                                     data["s"], w.bits, w.n)
        y = G.gpu_dequant_inv(ref["codes"], ref["scales"], data["s"], w.b, w.bits)
        P.check_inverse(y, y_ref, bf16=False, what=f"{name}/{t} inverse f32")
        yb = G.gpu_dequant_inv(ref["codes"], ref["scales"], data["s"], w.b, w.bits, out_bf16=True)
        P.check_inverse(P.bf16_bits_to_f64(yb), y_ref, bf16=True, what=f"{name}/{t} inverse bf16")


def test_qk_inner_products_preserved():
    w, data = _tensors("qk_heads", 42, 257)
    q = G.gpu_rotate(data["q"], W.BF16, data["s"], 128).reshape(32, 257, 128)
    k = G.gpu_rotate(data["k"], W.BF16, data["s"], 128).reshape(32, 257, 128)
    q0 = O.decode(data["q"], O.BF16).reshape(32, 257, 128)
    k0 = O.decode(data["k"], O.BF16).reshape(32, 257, 128)
    for h in range(32):
        ref = q0[h] @ k0[h].T
        got = q[h].astype(np.float64) @ k[h].astype(np.float64).T
        norms = np.linalg.norm(q0[h], axis=1)[:, None] * np.linalg.norm(k0[h], axis=1)[None, :]
        assert np.all(np.abs(got - ref) <= 1e-5 * norms)


# ----------------------------------------------------------------- shapes

SHAPES = [  # (n, b): generic, butterfly and matrix-core paths, blockwise and full
    (16, 1), (16, 2), (16, 16), (32, 4), (32, 32), (64, 8), (64, 64), (128, 32),
    (128, 128), (256, 128), (256, 256), (512, 64), (512, 128), (512, 512), (1024, 128),
    (1024, 1024), (2048, 128), (2048, 2048), (4096, 64), (4096, 128), (4096, 256),
    (4096, 1024), (4096, 4096), (8192, 4096), (11008, 16), (11008, 128), (11008, 256),
    (16384, 4096),
    # 128-blocks of rows that are not whole 512-element tiles or wider than
    # 4096 (one workgroup per row on the matrix core): 3, 5, 24 and 128 blocks
    (384, 128), (640, 128), (3072, 128), (16384, 128),
]


@pytest.mark.parametrize("n,b", SHAPES)
@pytest.mark.parametrize("x_dtype", [W.BF16, W.F32, W.F16])
def test_shapes_and_dtypes(n, b, x_dtype):
    rows = 37 if n * b <= 4096 * 1024 else 9
    raw, s = W.random_rows(n + b + x_dtype, rows, n, x_dtype, outliers=2)
    for bits, sd in ((4, W.F32), (8, W.F16)):
        tag = f"n={n} b={b} dt={x_dtype} bits={bits}"
        print(f"[shape] {tag}", flush=True)
        ref = O.rotate_quant(raw, x_dtype, b, s, bits, sd, want_xr=True)
        codes, scales = G.gpu_rotate_quant(raw, x_dtype, s, b, bits, sd)
        P.check_codes(codes, ref, bits, n, what=tag)
        P.check_scales(scales, ref, sd, what=tag)
        if x_dtype == W.BF16:
            # inverse on the oracle's own codes and scales, both output types
            y_ref = O.dequant_rotate_inv(ref["codes"], ref["scales"], sd, b, s, bits, n)
            y = G.gpu_dequant_inv(ref["codes"], ref["scales"], s, b, bits)
            P.check_inverse(y, y_ref, bf16=False, what=f"{tag} inverse f32")
            yb = G.gpu_dequant_inv(ref["codes"], ref["scales"], s, b, bits, out_bf16=True)
            P.check_inverse(P.bf16_bits_to_f64(yb), y_ref, bf16=True, what=f"{tag} inverse bf16")
    y = G.gpu_rotate(raw, x_dtype, s, b)
    P.check_rotated(y, ref["xr"], what=f"n={n} b={b} rotate")


@pytest.mark.parametrize("rows", [1, 2, 3, 5, 15, 17, 63, 65, 255, 257, 1023, 1025])
def test_ragged_row_counts(rows):
    for n, b in ((128, 128), (4096, 4096), (11008, 128), (1024, 1024), (256, 128)):
        if (rows > 300 and n > 128) or (rows > 65 and n >= 1024):
            continue
        raw, s = W.random_rows(rows * 7 + n, rows, n, W.BF16, outliers=1)
        ref = O.rotate_quant(raw, W.BF16, b, s, 4, W.F16)
        codes, scales = G.gpu_rotate_quant(raw, W.BF16, s, b, 4, W.F16)
        P.check_codes(codes, ref, 4, n, what=f"rows={rows} n={n}")
        P.check_scales(scales, ref, W.F16, what=f"rows={rows} n={n}")
        y_ref = O.dequant_rotate_inv(ref["codes"], ref["scales"], W.F16, b, s, 4, n)
        for out_bf16 in (False, True):
            y = G.gpu_dequant_inv(ref["codes"], ref["scales"], s, b, 4, out_bf16=out_bf16)
            if out_bf16:
                y = P.bf16_bits_to_f64(y)
            P.check_inverse(y, y_ref, bf16=out_bf16, what=f"rows={rows} n={n} inverse")


@pytest.mark.parametrize("n,b,rows", [
    (128, 128, 32768 + 37),   # just past the grid form's threshold, ragged last group
    (256, 128, 16384 + 3),
    (512, 512, 8192 + 5),
    (1024, 1024, 32768 + 5),  # 8-tile groups of wide rows
    (2048, 128, 16384 + 1),
    (11008, 128, 3101),       # 128-block rows of 11008-wide rows, a partial last group
])
def test_grid_form_ragged_tails(n, b, rows):
    # Launches this large take the grid form of the matrix-core kernel (one
    # group of tiles per single-wave workgroup); the reduced-size tests above
    # take its persistent form.  Every row against the oracle: rotation
    # alone, rotation + quantisation, and the inverse.
    raw, s = W.random_rows(rows + n, rows, n, W.BF16, outliers=1)
    tag = f"grid n={n} b={b} rows={rows}"
    print(f"[grid] {tag}", flush=True)
    ref = O.rotate_quant(raw, W.BF16, b, s, 4, W.F16, want_xr=True)
    P.check_rotated(G.gpu_rotate(raw, W.BF16, s, b), ref.pop("xr"), what=f"{tag} rotate")
    codes, scales = G.gpu_rotate_quant(raw, W.BF16, s, b, 4, W.F16)
    P.check_codes(codes, ref, 4, n, what=tag)
    P.check_scales(scales, ref, W.F16, what=tag)
    ref.pop("preround")
    y_ref = O.dequant_rotate_inv(ref["codes"], ref["scales"], W.F16, b, s, 4, n)
    y = G.gpu_dequant_inv(ref["codes"], ref["scales"], s, b, 4)
    P.check_inverse(y, y_ref, bf16=False, what=f"{tag} inverse")


def test_zero_rows_and_spikes():
    for n, b in ((128, 128), (4096, 4096), (11008, 128)):
        raw = np.zeros((6, n), dtype=np.float32)
        raw[1, 3] = 30.0
        raw[2, n - 1] = -30.0
        raw[4, :] = 1.0
        raw[5, n // 2] = 1e-30
        s = np.where(np.arange(n) % 3 == 0, -1, 1).astype(np.int8)
        ref = O.rotate_quant(raw, W.F32, b, s, 4, W.F32, want_xr=True)
        codes, scales = G.gpu_rotate_quant(raw, W.F32, s, b, 4, W.F32)
        P.check_codes(codes, ref, 4, n, what=f"special n={n}")
        P.check_scales(scales, ref, W.F32, what=f"special n={n}")
        assert scales[0] == 0 and np.all(codes[0] == 0)
        y = G.gpu_dequant_inv(codes, scales, s, b, 4)
        assert np.all(y[0] == 0)
        # spike rows are on the grid: the round trip is exact
        assert np.allclose(y[1], raw[1], atol=1e-6)


def test_tiny_rows_follow_the_oracle():
    # Rows whose maximum lies far below the range where qmax / max fits
    # binary32, down to subnormal inputs, get the oracle's codes and scales
    # like any other row.  (32768, 4096) takes the generic LDS kernel, the
    # fp32 rows the butterfly kernel, the 16-bit rows the matrix core (and
    # the long-row butterfly kernel for 11008).
    for n, b in ((128, 128), (4096, 4096), (11008, 128), (32768, 4096), (512, 128)):
        raw = np.zeros((6, n), dtype=np.float32)
        raw[0, 5] = 1.5 * 2.0 ** -127                   # subnormal
        raw[1, n - 3] = -2.0 ** -119
        raw[2, :] = 2.0 ** -110
        raw[3, 7] = 1.0
        raw[4, 3] = 2.0 ** -133                          # subnormal
        raw[4, n // 2] = -3 * 2.0 ** -133
        raw[5, 1::97] = 2.0 ** -126 * (1 + np.arange(len(raw[5, 1::97])) % 64)
        s = np.where(np.arange(n) % 5 == 0, -1, 1).astype(np.int8)
        for dt in (W.F32, W.BF16):
            # bf16 holds the same exponent range; these values are exact in it
            x = raw if dt == W.F32 else \
                (raw.view(np.uint32) >> 16).astype(np.uint16)
            if dt == W.BF16:
                assert np.array_equal(O.decode(x, W.BF16), raw.astype(np.float64))
            for bits in (4, 8):
                tag = f"tiny n={n} b={b} dt={dt} bits={bits}"
                print(f"[tiny] {tag}", flush=True)
                codes, scales = G.gpu_rotate_quant(x, dt, s, b, bits, W.F32)
                ref = O.rotate_quant(x, dt, b, s, bits, W.F32)
                P.check_codes(codes, ref, bits, n, what=tag)
                P.check_scales(scales, ref, W.F32, what=tag)
                codes16, scales16 = G.gpu_rotate_quant(x, dt, s, b, bits, W.F16)
                ref16 = O.rotate_quant(x, dt, b, s, bits, W.F16)
                assert np.array_equal(codes16, codes)
                P.check_scales(scales16, ref16, W.F16, what=tag + " f16 scales")


def test_rows_zero_is_noop():
    import torch
    import hadamard_rotation_amd as hq
    x = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    s = torch.ones(128, dtype=torch.int8, device="cuda")
    codes, scales = hq.hq_rotate_quant(x, s, 128)
    assert codes.shape == (0, 64) and scales.shape == (0,)


def test_deterministic_and_stream():
    import torch
    import hadamard_rotation_amd as hq
    w, data = _tensors("hidden_4096", 1, 300)
    x = G.to_dev(data["x"], W.BF16)
    s = G.s_dev(data["s"])
    c1, s1 = hq.hq_rotate_quant(x, s, 4096)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        c2, s2 = hq.hq_rotate_quant(x, s, 4096, stream=st)
    st.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(s1, s2)


def test_max_n():
    import hadamard_rotation_amd as hq
    n = hq.hq_max_n()
    assert n >= 16384
    b = min(n & -n, 4096)
    raw, s = W.random_rows(3, 2, n, W.BF16, outliers=1)
    ref = O.rotate_quant(raw, W.BF16, b, s, 4, W.F32)
    codes, scales = G.gpu_rotate_quant(raw, W.BF16, s, b, 4, W.F32)
    P.check_codes(codes, ref, 4, n, what="max n")
    with pytest.raises(NotImplementedError):
        raw2, s2 = W.random_rows(3, 1, n + 16 * 256, W.BF16)
        G.gpu_rotate_quant(raw2, W.BF16, s2, 16, 4, W.F32)
