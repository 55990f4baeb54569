"""hq_decode_attention_noalloc (the entry point for callers that cannot
allocate: the partials live in the library's own per-GPU array) against
hq_decode_attention with a caller workspace, through the C ABI.

Both run the same kernels on the same inputs, so the outputs must be equal
bit for bit (a stricter bar than the oracle tolerance of the attention
tests).  Two calls in a row, the second with a smaller cache, so the second
reads a static array that still holds the first call's partials.  The cache
is written by the oracle from seeded K/V rows ("手把手教你用QuaRot实现LLM的4位量化：
从原理到代码实践" section 2.2: K and V rotated online into a 4-bit cache).
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


def _inputs(seed, tokens, kv_heads, q_heads):
    rng = np.random.default_rng(seed)
    s = np.where(rng.integers(0, 2, 128) == 1, 1, -1).astype(np.int8)
    k = rng.standard_normal((tokens * kv_heads, 128), dtype=np.float32)
    k[:, 9] *= np.float32(30.0)
    v = rng.standard_normal((tokens * kv_heads, 128), dtype=np.float32)
    kr = O.rotate_quant(W.to_bf16_bits(k), W.BF16, 128, s, 4, W.F16, want_preround=False)
    vr = O.rotate_quant(W.to_bf16_bits(v), W.BF16, 128, s, 4, W.F16, want_preround=False)
    q = W.to_bf16_bits(rng.standard_normal((q_heads, 128), dtype=np.float32))
    dev = "cuda"
    kc = torch.from_numpy(kr["codes"]).to(dev).view(tokens, kv_heads, 64)
    vc = torch.from_numpy(vr["codes"]).to(dev).view(tokens, kv_heads, 64)
    ks = torch.from_numpy(np.ascontiguousarray(kr["scales"]).view(np.uint16)).to(dev)
    vs = torch.from_numpy(np.ascontiguousarray(vr["scales"]).view(np.uint16)).to(dev)
    ks = ks.view(torch.float16).view(tokens, kv_heads)
    vs = vs.view(torch.float16).view(tokens, kv_heads)
    return G.to_dev(q, W.BF16), G.s_dev(s), kc, ks, vc, vs


@pytest.mark.parametrize("q_heads,kv_heads", [(32, 8), (8, 2)])
def test_noalloc_matches_workspace_entry_point(q_heads, kv_heads):
    for tokens in (20000, 777):  # the second call is smaller
        print(f"[noalloc] q_heads={q_heads} kv_heads={kv_heads} tokens={tokens}", flush=True)
        q, s, kc, ks, vc, vs = _inputs(tokens + q_heads, tokens, kv_heads, q_heads)
        ref = hq.hq_decode_attention(q, s, 128, kc, ks, vc, vs, 4)
        out = torch.full((q_heads, 128), float("nan"), dtype=torch.float32, device="cuda")
        got = hq.hq_decode_attention_noalloc(q, s, 128, kc, ks, vc, vs, 4, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.isfinite(ref).all()
        assert torch.equal(got, ref), (tokens, (got - ref).abs().max().item())


def test_noalloc_rejects_requests_beyond_its_array():
    # 1024 kv heads x 8 query heads each need more than the static array
    need = hq.hq_decode_attention_workspace(8192, 1024, 64)
    assert need > hq.binding.NOALLOC_WORKSPACE_BYTES
    q, s, kc, ks, vc, vs = _inputs(5, 64, 1024, 8192)
    with pytest.raises(NotImplementedError):
        hq.hq_decode_attention_noalloc(q, s, 128, kc, ks, vc, vs, 4)
