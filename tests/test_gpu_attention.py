"""GPU parity of hq_decode_attention, the consumer of the INT4 K/V codes,
against the oracle's decode attention (dequantise, rotate q with the cache's
rotation, softmax, weighted sum of V, rotate back).

The cache is written by the oracle from seeded K/V rows, so neither the
inputs nor the expected values come from the HIP path.  Tolerance (derived in
the design notes): |gpu - oracle| <= 1e-5 * (1 + max|c|) * max|o| per head,
where c are the attention scores: the GPU's scores carry a relative error of
about 1e-6 (hi/lo f16 split of q, fp32 sums), which moves every softmax weight
by at most that much times |c|.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import hadamard_rotation_amd as hq
from hadamard_rotation_amd import workloads as W
from oracle import oracle as O
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    G.require_gpu()


def _cache(seed, tokens, kv_heads, b, sd, outlier=30.0):
    rng = np.random.default_rng(seed)
    s = np.where(rng.integers(0, 2, 128) == 1, 1, -1).astype(np.int8)
    k = rng.standard_normal((tokens * kv_heads, 128), dtype=np.float32)
    k[:, 5] *= np.float32(outlier)
    v = rng.standard_normal((tokens * kv_heads, 128), dtype=np.float32)
    kb, vb = W.to_bf16_bits(k), W.to_bf16_bits(v)
    kr = O.rotate_quant(kb, W.BF16, b, s, 4, sd, want_preround=False)
    vr = O.rotate_quant(vb, W.BF16, b, s, 4, sd, want_preround=False)
    return s, kr, vr, kb


def _check(q_raw, q_dtype, kv_heads, b, s, kr, vr, sd, tag, kb=None):
    q_heads = q_raw.shape[0]
    tokens = kr["codes"].shape[0] // kv_heads
    print(f"[attn] {tag} q_heads={q_heads} kv_heads={kv_heads} tokens={tokens}", flush=True)
    ref = O.decode_attention(q_raw, q_dtype, kv_heads, b, s, kr["codes"], kr["scales"],
                             vr["codes"], vr["scales"], sd, 4)
    dev = "cuda"
    sc_t = torch.float32 if sd == W.F32 else torch.float16
    kc = torch.from_numpy(kr["codes"]).to(dev).view(tokens, kv_heads, 64)
    vc = torch.from_numpy(vr["codes"]).to(dev).view(tokens, kv_heads, 64)
    ks = torch.from_numpy(np.ascontiguousarray(kr["scales"])).to(dev).view(tokens, kv_heads)
    vs = torch.from_numpy(np.ascontiguousarray(vr["scales"])).to(dev).view(tokens, kv_heads)
    if sd == W.F16:
        ks, vs = ks.view(sc_t), vs.view(sc_t)
    out = hq.hq_decode_attention(G.to_dev(q_raw, q_dtype), G.s_dev(s), b, kc, ks, vc, vs, 4)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    # scores in the input space (orthogonality): q . k_t / sqrt(n), k_t the
    # dequantised key row rotated back, for the tolerance
    kin = O.dequant_rotate_inv(kr["codes"], kr["scales"], sd, b, s, 4, 128)
    qin = O.decode(q_raw, q_dtype)
    group = q_heads // kv_heads
    worst = 0.0
    for h in range(q_heads):
        rows = np.arange(tokens) * kv_heads + h // group
        cmax = np.abs(kin[rows] @ qin[h]).max() / np.sqrt(128)
        omax = np.abs(ref[h]).max()
        err = np.abs(got[h] - ref[h]).max()
        lim = 1e-5 * (1.0 + cmax) * omax
        worst = max(worst, err / max(lim, 1e-300))
        assert err <= lim, f"{tag} head {h}: err {err:.3e} > {lim:.3e} (max|c| {cmax:.1f})"
    print(f"[attn] {tag}: worst err/limit {worst:.3f}", flush=True)


@pytest.mark.parametrize("q_heads,kv_heads", [(32, 8), (8, 8), (16, 8), (64, 8), (4, 1)])
@pytest.mark.parametrize("tokens", [1, 15, 16, 17, 517, 4099])
def test_attention_shapes(q_heads, kv_heads, tokens):
    s, kr, vr, _ = _cache(tokens + q_heads, tokens, kv_heads, 128, W.F16)
    rng = np.random.default_rng(tokens)
    q = W.to_bf16_bits(rng.standard_normal((q_heads, 128), dtype=np.float32))
    _check(q, W.BF16, kv_heads, 128, s, kr, vr, W.F16, f"G={q_heads // kv_heads}")


@pytest.mark.parametrize("b", [128, 32, 16])
@pytest.mark.parametrize("q_dtype,sd", [(W.F32, W.F32), (W.F16, W.F16), (W.BF16, W.F32)])
def test_attention_blocks_and_dtypes(b, q_dtype, sd):
    tokens, kv_heads, q_heads = 300, 4, 16
    s, kr, vr, _ = _cache(b + q_dtype, tokens, kv_heads, b, sd)
    rng = np.random.default_rng(b)
    qf = rng.standard_normal((q_heads, 128), dtype=np.float32) * np.float32(3.0)
    q = qf if q_dtype == W.F32 else (W.to_bf16_bits(qf) if q_dtype == W.BF16
                                     else qf.astype(np.float16).view(np.uint16))
    _check(q, q_dtype, kv_heads, b, s, kr, vr, sd, f"b={b} q={q_dtype} sd={sd}")


def test_attention_peaked_scores():
    # a query aligned with one cached key: large scores, nearly one-hot weights
    tokens, kv_heads, q_heads = 257, 2, 8
    s, kr, vr, kb = _cache(9, tokens, kv_heads, 128, W.F32, outlier=1.0)
    kin = O.dequant_rotate_inv(kr["codes"], kr["scales"], W.F32, 128, s, 4, 128)
    q = np.stack([kin[(37 + 11 * h) * kv_heads + h // 4] * 0.8 for h in range(q_heads)])
    _check(q.astype(np.float32), W.F32, kv_heads, 128, s, kr, vr, W.F32, "peaked")


def test_attention_full_kv_cache():
    # the 131072-token x 8-head K/V cache with 32 query heads
    data = W.generate("kv_cache", seed=42)
    s = data["s"]
    kr = O.rotate_quant(data["k"], W.BF16, 128, s, 4, W.F16, want_preround=False)
    vr = O.rotate_quant(data["v"], W.BF16, 128, s, 4, W.F16, want_preround=False)
    rng = np.random.default_rng(43)
    q = W.to_bf16_bits(rng.standard_normal((32, 128), dtype=np.float32))
    _check(q, W.BF16, 8, 128, s, kr, vr, W.F16, "kv_cache 131072 x 8")


def test_one_workspace_serves_calls_of_any_shape():
    # One workspace, sized for the largest call, serves calls of different
    # shapes one after the other (more kv heads, then fewer, with the
    # partials of earlier calls left behind, never zeroed): each call must
    # give what a fresh workspace gives, bit for bit.
    dev = "cuda"
    shapes = [(8, 2, 3000), (32, 8, 20000), (8, 1, 500), (64, 8, 7000), (32, 8, 20000)]
    need = max(hq.hq_decode_attention_workspace(qh, kvh, t) for qh, kvh, t in shapes)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=dev)
    for i, (q_heads, kv_heads, tokens) in enumerate(shapes):
        print(f"[attn] shared workspace call {i}: q_heads={q_heads} kv_heads={kv_heads} "
              f"tokens={tokens}", flush=True)
        s, kr, vr, _ = _cache(100 + i, tokens, kv_heads, 128, W.F16)
        q = G.to_dev(W.to_bf16_bits(np.random.default_rng(i).standard_normal(
            (q_heads, 128), dtype=np.float32)), W.BF16)
        kc = torch.from_numpy(kr["codes"]).to(dev).view(tokens, kv_heads, 64)
        vc = torch.from_numpy(vr["codes"]).to(dev).view(tokens, kv_heads, 64)
        ks = torch.from_numpy(np.ascontiguousarray(kr["scales"])).to(dev)
        vs = torch.from_numpy(np.ascontiguousarray(vr["scales"])).to(dev)
        ks = ks.view(torch.float16).view(tokens, kv_heads)
        vs = vs.view(torch.float16).view(tokens, kv_heads)
        ref = hq.hq_decode_attention(q, G.s_dev(s), 128, kc, ks, vc, vs, 4)
        got = hq.hq_decode_attention(q, G.s_dev(s), 128, kc, ks, vc, vs, 4, workspace=ws)
        torch.cuda.synchronize()
        assert torch.isfinite(ref).all()
        assert torch.equal(got, ref), (i, (got - ref).abs().max().item())
