"""Seeded synthetic workloads for the rotation + quantisation path.

This module only draws random numbers and stores them; it holds none of the
method's arithmetic.  The test suite, the benchmark and the CPU oracle all
take their inputs from here, so the GPU and the oracle always see the same
bytes.  No public dataset is involved: every tensor is synthetic, with the
shapes and value statistics of the LLM workloads the pages discuss
(hidden width 4096 and head dimension 128 in "旋转量化：大模型低比特量化中的
离群值克星" section 2.1; a small share of channels about 100x larger than the
rest in "哈特曼旋转，轻量级QAT，流式注意力" section 1; the 4-bit K/V cache of
"手把手教你用QuaRot实现LLM的4位量化：从原理到代码实践" section 2.2).

Generator: ``numpy.random.default_rng(seed)`` (PCG64); the house seed is 42
(the rotation-quantization blog's section 6.2 recommends fixing it there).
Draw order inside every workload is fixed and documented per function.
Values are drawn in float32 (float64 for Student-t) and rounded to bfloat16
with round-to-nearest-even by torch's CPU cast.  The sign vector is
``where(rng.integers(0, 2, period) == 1, +1, -1)``, tiled to the row width.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

F32, BF16, F16 = 0, 1, 2  # same numbering as the C ABI's hq_dtype
DTYPE_NAMES = {F32: "f32", BF16: "bf16", F16: "f16"}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: a set of row tensors with a shared sign vector."""
    name: str
    description: str
    rows: int            # rows per tensor at the full size
    n: int               # row width
    b: int               # Hadamard block size (b == n: full rotation)
    x_dtype: int         # F32 or BF16
    bits: int            # 4 or 8
    scale_dtype: int     # F32 or F16
    tensors: tuple       # names of the tensors (e.g. ("q", "k"))
    unit: int            # rows per "token unit" (heads per token etc.)

    def bytes_per_call(self, rows: int | None = None, group: int | None = None) -> int:
        """Algorithmic HBM bytes of one rotate+quantise call: input + codes +
        scales, one per row (group None) or per `group` elements (the sign
        vector, n bytes, is negligible and not counted)."""
        r = self.rows if rows is None else rows
        in_b = 4 if self.x_dtype == F32 else 2
        code_b = self.n // 2 if self.bits == 4 else self.n
        sc_b = (4 if self.scale_dtype == F32 else 2) * (1 if group is None else self.n // group)
        return r * (self.n * in_b + code_b + sc_b)


def sign_vector(rng: np.random.Generator, period: int, n: int) -> np.ndarray:
    """+1/-1 int8 vector of length n: `period` fresh signs tiled n/period times."""
    base = np.where(rng.integers(0, 2, size=period) == 1, 1, -1).astype(np.int8)
    return np.tile(base, n // period)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32/float64 to bfloat16 (nearest-even, via torch) and return
    the raw 16-bit patterns as uint16."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


WORKLOADS = {
    "tiny_int8": Workload(
        "tiny_int8",
        "64 rows x 128 fp32, N(0,1) with one +-100 outlier per row at a random "
        "channel; full 128-point rotation; INT8, fp32 scales",
        64, 128, 128, F32, 8, F32, ("x",), 1),
    "qk_heads": Workload(
        "qk_heads",
        "Q and K of batch 1 x 32 heads x 4096 tokens x head_dim 128, bf16, "
        "N(0,1) with one fixed channel per head x100; per-head-vector "
        "128-point rotation; INT4, fp16 scales",
        32 * 4096, 128, 128, BF16, 4, F16, ("q", "k"), 32),
    "hidden_4096": Workload(
        "hidden_4096",
        "16384 tokens x 4096 bf16, Student-t(4)/sqrt(2) with 4 fixed outlier "
        "channels x50; full 4096-point rotation; per-token INT4, fp32 scales",
        16384, 4096, 4096, BF16, 4, F32, ("x",), 1),
    "ffn_11008": Workload(
        "ffn_11008",
        "16384 tokens x 11008 bf16, N(0,1) with 11 fixed channels x100; "
        "86 blocks of 128 with one shared 128-sign vector; per-token INT4, "
        "fp32 scales",
        16384, 11008, 128, BF16, 4, F32, ("x",), 1),
    "ffn_11008_full": Workload(
        "ffn_11008_full",
        "16384 tokens x 11008 bf16, N(0,1) with 11 fixed channels x100; "
        "full 11008-point rotation H_344 (x) H_32 (Paley over GF(7^3)) with an "
        "11008-sign vector; per-token INT4, fp32 scales",
        16384, 11008, 11008, BF16, 4, F32, ("x",), 1),
    "kv_cache": Workload(
        "kv_cache",
        "K and V of 131072 tokens x 8 KV heads x head_dim 128, bf16, N(0,1); "
        "K has one fixed channel per head x30; 128-point rotation per head "
        "vector; INT4, fp16 scales; dequant + inverse round trip",
        131072 * 8, 128, 128, BF16, 4, F16, ("k", "v"), 8),
}

# Order used when a list of workloads is wanted.
ORDER = ("tiny_int8", "qk_heads", "hidden_4096", "ffn_11008", "kv_cache")


def generate(name: str, seed: int = 42, tokens: int | None = None) -> dict:
    """Draw the inputs of workload `name`.

    `tokens` scales the workload down (rows = tokens * unit); None = full size.
    Returns {"s": int8 [n], <tensor>: raw rows [rows, n], "channels": ...}
    where raw rows are float32 for fp32 workloads and uint16 bf16 bit
    patterns otherwise.

    Draw order per workload:
      tiny_int8   : s(128); x N(0,1) [rows,128] f32; outlier channel per row;
                    outlier sign per row
      qk_heads    : s(128); outlier channel per head (32); Q N(0,1) f32; K N(0,1)
      hidden_4096 : s(4096); 4 distinct outlier channels; x Student-t(4) f64
      ffn_11008   : s(128) tiled x86; 11 distinct outlier channels; x N(0,1)
      ffn_11008_full: s(11008); 11 distinct outlier channels; x N(0,1)
      kv_cache    : s(128); outlier channel per KV head (8); K N(0,1); V N(0,1)
    """
    w = WORKLOADS[name]
    rng = np.random.default_rng(seed)
    out: dict = {}
    if name == "tiny_int8":
        rows = w.rows if tokens is None else tokens
        out["s"] = sign_vector(rng, 128, 128)
        x = rng.standard_normal((rows, 128), dtype=np.float32)
        ch = rng.integers(0, 128, size=rows)
        sg = np.where(rng.integers(0, 2, size=rows) == 1, 100.0, -100.0)
        x[np.arange(rows), ch] = sg.astype(np.float32)
        out["x"] = x
        out["channels"] = ch
    elif name == "qk_heads":
        seq = 4096 if tokens is None else tokens
        heads = 32
        out["s"] = sign_vector(rng, 128, 128)
        ch = rng.integers(0, 128, size=heads)
        for t in ("q", "k"):
            v = rng.standard_normal((heads, seq, 128), dtype=np.float32)
            v[np.arange(heads), :, ch] *= 100.0
            out[t] = to_bf16_bits(v.reshape(heads * seq, 128))
        out["channels"] = ch
    elif name == "hidden_4096":
        rows = w.rows if tokens is None else tokens
        out["s"] = sign_vector(rng, 4096, 4096)
        ch = rng.choice(4096, size=4, replace=False)
        x = rng.standard_t(4, size=(rows, 4096)) / math.sqrt(2.0)
        x[:, ch] *= 50.0
        out["x"] = to_bf16_bits(x)
        out["channels"] = ch
    elif name == "ffn_11008":
        rows = w.rows if tokens is None else tokens
        out["s"] = sign_vector(rng, 128, 11008)
        ch = rng.choice(11008, size=11, replace=False)
        x = rng.standard_normal((rows, 11008), dtype=np.float32)
        x[:, ch] *= 100.0
        out["x"] = to_bf16_bits(x)
        out["channels"] = ch
    elif name == "ffn_11008_full":
        rows = w.rows if tokens is None else tokens
        out["s"] = sign_vector(rng, 11008, 11008)
        ch = rng.choice(11008, size=11, replace=False)
        x = rng.standard_normal((rows, 11008), dtype=np.float32)
        x[:, ch] *= 100.0
        out["x"] = to_bf16_bits(x)
        out["channels"] = ch
    elif name == "kv_cache":
        toks = 131072 if tokens is None else tokens
        heads = 8
        out["s"] = sign_vector(rng, 128, 128)
        ch = rng.integers(0, 128, size=heads)
        k = rng.standard_normal((toks, heads, 128), dtype=np.float32)
        k[:, np.arange(heads), ch] *= 30.0
        out["k"] = to_bf16_bits(k.reshape(toks * heads, 128))
        v = rng.standard_normal((toks * heads, 128), dtype=np.float32)
        out["v"] = to_bf16_bits(v)
        out["channels"] = ch
    else:  # pragma: no cover
        raise KeyError(name)
    return out


def random_rows(seed: int, rows: int, n: int, dtype: int = BF16,
                scale: float = 1.0, outliers: int = 0,
                outlier_gain: float = 100.0) -> tuple:
    """Generic seeded rows for edge-case tests: N(0,1)*scale with `outliers`
    fixed channels multiplied by `outlier_gain`.  Draw order: s(n); outlier
    channels; values.  Returns (raw rows, s)."""
    rng = np.random.default_rng(seed)
    s = sign_vector(rng, n, n)
    ch = rng.choice(n, size=outliers, replace=False) if outliers else np.zeros(0, int)
    x = rng.standard_normal((rows, n), dtype=np.float32) * np.float32(scale)
    if outliers:
        x[:, ch] *= np.float32(outlier_gain)
    if dtype == F32:
        return x, s
    if dtype == BF16:
        return to_bf16_bits(x), s
    return x.astype(np.float16).view(np.uint16), s


def spiked_gaussian_row(seed: int, n: int, index: int, value: float) -> np.ndarray:
    """One fp32 row [1, n] of standard-normal draws from numpy's default
    generator seeded with `seed` (drawn in double precision, then rounded to
    fp32), with entry `index` replaced by `value`: the single-outlier row of
    the error-reduction example in "旋转量化：大模型低比特量化中的离群值克星"
    section 2.2 (seed 42, n 4096, a spike of 30)."""
    rng = np.random.default_rng(seed)
    row = rng.standard_normal((1, n)).astype(np.float32)
    row[0, index] = np.float32(value)
    return row
