"""Host-side tests of the C ABI: the library loads, exports what include/hq.h
declares, and rejects every invalid-argument class before touching the GPU.
None of these calls reaches the HIP runtime (rows == 0 or invalid input)."""
import ctypes
import os
import re

import pytest

import hadamard_rotation_amd as hq
from hadamard_rotation_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hq.h")

A = ctypes.c_void_p(0x10000)      # 16-byte aligned, never dereferenced
MIS = ctypes.c_void_p(0x10001)    # misaligned
A2 = ctypes.c_void_p(0x10002)     # 2-byte aligned, not 4


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hq_[a-z_0-9]+)\s*\(", text)))


def test_library_loads_and_exports_header_symbols():
    lib = hq.load()
    syms = declared_symbols()
    assert set(syms) == {"hq_rotate_quant", "hq_dequant_rotate_inv", "hq_rotate_quant_grouped",
                         "hq_dequant_rotate_inv_grouped", "hq_rotate_quant_append", "hq_rotate",
                         "hq_decode_attention", "hq_decode_attention_workspace",
                         "hq_decode_attention_noalloc", "hq_status_str",
                         "hq_last_hip_error", "hq_max_n", "hq_version"}
    for name in syms:
        assert hasattr(lib, name), name
    assert set(B.EXPORTS) == set(syms)


def test_status_strings():
    for code, frag in ((0, "HQ_OK"), (1, "HQ_EINVAL"), (2, "HQ_EUNSUPPORTED"), (3, "HQ_EHIP"),
                       (99, "unknown")):
        assert frag in hq.status_str(code)
    assert hq.hq_version() == 10300


def rq(x=A, xd=1, rows=4, n=128, b=128, s=A, bits=4, codes=A, scales=A, sd=0):
    return hq.load().hq_rotate_quant(x, xd, rows, n, b, s, bits, codes, scales, sd, None)


def inv(codes=A, scales=A, sd=0, rows=4, n=128, b=128, s=A, bits=4, y=A, yd=0):
    return hq.load().hq_dequant_rotate_inv(codes, scales, sd, rows, n, b, s, bits, y, yd, None)


def rqg(x=A, xd=1, rows=4, n=256, b=128, s=A, bits=4, group=64, codes=A, scales=A, sd=0):
    return hq.load().hq_rotate_quant_grouped(x, xd, rows, n, b, s, bits, group, codes, scales,
                                             sd, None)


def invg(codes=A, scales=A, sd=0, rows=4, n=256, b=128, s=A, bits=4, group=64, y=A, yd=0):
    return hq.load().hq_dequant_rotate_inv_grouped(codes, scales, sd, rows, n, b, s, bits, group,
                                                   y, yd, None)


def rqa(x=A, xd=1, rows=4, n=128, b=128, s=A, bits=4, dst=A, codes=A, scales=A, sd=0,
        cache_rows=1024):
    return hq.load().hq_rotate_quant_append(x, xd, rows, n, b, s, bits, dst, codes, scales, sd,
                                            cache_rows, None)


def att(q=A, qd=1, qh=32, kvh=8, n=128, b=128, s=A, tokens=100, bits=4, kc=A, ks=A, vc=A, vs=A,
        sd=2, out=A, ws=A, wsb=1 << 40):
    return hq.load().hq_decode_attention(q, qd, qh, kvh, n, b, s, tokens, bits, kc, ks, vc, vs, sd,
                                         out, ws, wsb, None)


def attn0(q=A, qd=1, qh=32, kvh=8, n=128, b=128, s=A, tokens=100, bits=4, kc=A, ks=A, vc=A,
          vs=A, sd=2, out=A):
    return hq.load().hq_decode_attention_noalloc(q, qd, qh, kvh, n, b, s, tokens, bits, kc, ks,
                                                 vc, vs, sd, out, None)


def rot(x=A, xd=1, rows=4, n=128, b=128, s=A, y=A):
    return hq.load().hq_rotate(x, xd, rows, n, b, s, y, None)


@pytest.mark.parametrize("kw", [
    dict(x=None), dict(s=None), dict(codes=None), dict(scales=None),
    dict(rows=-1), dict(n=0), dict(n=-128), dict(n=120), dict(n=8), dict(b=0), dict(b=3),
    dict(b=96), dict(n=384, b=256), dict(bits=3), dict(bits=16), dict(xd=7), dict(sd=1),
    dict(sd=9), dict(x=MIS), dict(s=MIS), dict(codes=MIS), dict(scales=A2),
])
def test_rotate_quant_einval(kw):
    assert rq(**kw) == hq.HQ_EINVAL


@pytest.mark.parametrize("kw", [
    dict(codes=None), dict(scales=None), dict(y=None), dict(s=None), dict(rows=-5),
    dict(n=100), dict(b=5), dict(bits=2), dict(sd=1), dict(yd=2), dict(yd=5),
    dict(codes=MIS), dict(y=MIS), dict(scales=A2),
])
def test_dequant_einval(kw):
    assert inv(**kw) == hq.HQ_EINVAL


@pytest.mark.parametrize("kw", [
    dict(x=None), dict(y=None), dict(s=None), dict(rows=-1), dict(n=24), dict(b=6),
    dict(xd=3), dict(x=MIS), dict(y=MIS),
])
def test_rotate_einval(kw):
    assert rot(**kw) == hq.HQ_EINVAL


@pytest.mark.parametrize("fn", [rqg, invg])
@pytest.mark.parametrize("group", [0, -64, 1, 3, 48, 96, 512, 1024])
def test_grouped_bad_group_einval(fn, group):
    # n = 256: a group must be n itself or a power of two >= 2 dividing n
    assert fn(group=group) == hq.HQ_EINVAL
    assert fn(group=group, rows=0) == hq.HQ_EINVAL


@pytest.mark.parametrize("kw", [
    dict(x=None), dict(s=None), dict(codes=None), dict(scales=None), dict(rows=-1),
    dict(n=120, group=8), dict(b=3), dict(bits=5), dict(xd=7), dict(sd=1), dict(x=MIS),
    dict(codes=MIS), dict(scales=A2),
])
def test_rotate_quant_grouped_einval(kw):
    assert rqg(**kw) == hq.HQ_EINVAL


@pytest.mark.parametrize("kw", [
    dict(codes=None), dict(scales=None), dict(y=None), dict(s=None), dict(rows=-1),
    dict(n=100, group=4), dict(b=5), dict(bits=2), dict(sd=1), dict(yd=2), dict(codes=MIS),
    dict(y=MIS), dict(scales=A2),
])
def test_dequant_grouped_einval(kw):
    assert invg(**kw) == hq.HQ_EINVAL


def test_grouped_valid_groups_noop_at_zero_rows():
    # rows == 0: valid groups pass every check and return without launching
    for n, group in ((256, 256), (256, 2), (256, 128), (11008, 11008), (11008, 128),
                     (11008, 256), (48, 48), (48, 16)):
        assert rqg(rows=0, n=n, b=16, group=group, x=None, codes=None, scales=None,
                   s=None) == hq.HQ_OK, (n, group)
        assert invg(rows=0, n=n, b=16, group=group, codes=None, scales=None, y=None,
                    s=None) == hq.HQ_OK, (n, group)


@pytest.mark.parametrize("kw", [
    dict(x=None), dict(s=None), dict(dst=None), dict(codes=None), dict(scales=None),
    dict(rows=-1), dict(n=120), dict(b=3), dict(bits=5), dict(xd=7), dict(sd=1),
    dict(cache_rows=-1), dict(dst=A2), dict(x=MIS), dict(codes=MIS), dict(scales=A2),
])
def test_rotate_quant_append_einval(kw):
    assert rqa(**kw) == hq.HQ_EINVAL


def test_rotate_quant_append_zero_rows_noop():
    assert rqa(rows=0, x=None, dst=None, codes=None, scales=None, s=None) == hq.HQ_OK
    assert rqa(rows=0, cache_rows=0) == hq.HQ_OK


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(s=None), dict(kc=None), dict(ks=None), dict(vc=None), dict(vs=None),
    dict(out=None), dict(ws=None), dict(qh=0), dict(kvh=0), dict(qh=30), dict(tokens=0),
    dict(n=100), dict(b=96), dict(bits=3), dict(qd=5), dict(sd=1), dict(kc=MIS), dict(out=MIS),
    dict(ws=MIS), dict(ks=MIS), dict(wsb=16),
])
def test_decode_attention_einval(kw):
    assert att(**kw) == hq.HQ_EINVAL


@pytest.mark.parametrize("kw", [dict(n=64, b=64), dict(bits=8), dict(qh=24, kvh=8),
                                dict(qh=32, kvh=2)])
def test_decode_attention_unsupported(kw):
    assert att(**kw) == hq.HQ_EUNSUPPORTED


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(s=None), dict(kc=None), dict(ks=None), dict(vc=None), dict(vs=None),
    dict(out=None), dict(qh=0), dict(kvh=0), dict(qh=30), dict(tokens=0), dict(n=100),
    dict(b=96), dict(bits=3), dict(qd=5), dict(sd=1), dict(kc=MIS), dict(out=MIS), dict(ks=MIS),
])
def test_decode_attention_noalloc_einval(kw):
    # the same validation as hq_decode_attention, before anything else
    assert attn0(**kw) == hq.HQ_EINVAL


@pytest.mark.parametrize("kw", [dict(n=64, b=64), dict(bits=8), dict(qh=24, kvh=8),
                                dict(qh=32, kvh=2)])
def test_decode_attention_noalloc_unsupported(kw):
    assert attn0(**kw) == hq.HQ_EUNSUPPORTED


def test_decode_attention_noalloc_limit():
    # requests whose partials exceed the library's own workspace are
    # rejected before any device call (HQ_NOALLOC_WORKSPACE_BYTES)
    from hadamard_rotation_amd import binding as Bd
    text = open(HEADER).read()
    m = re.search(r"#define HQ_NOALLOC_WORKSPACE_BYTES \((\d+) \* 1024 \* 1024\)", text)
    assert m and int(m.group(1)) * 2 ** 20 == Bd.NOALLOC_WORKSPACE_BYTES
    assert hq.hq_decode_attention_workspace(32, 8, 131072) <= Bd.NOALLOC_WORKSPACE_BYTES
    big = 1024
    assert hq.hq_decode_attention_workspace(big * 8, big, 131072) > Bd.NOALLOC_WORKSPACE_BYTES
    assert attn0(qh=big * 8, kvh=big, tokens=131072) == hq.HQ_EUNSUPPORTED


def test_decode_attention_workspace_size():
    w = hq.hq_decode_attention_workspace(32, 8, 131072)
    assert w > 0 and w % 16 == 0
    assert hq.hq_decode_attention_workspace(32, 8, 0) == 0
    # one partial at least per query head, 130 floats each
    assert hq.hq_decode_attention_workspace(1, 1, 1) >= 130 * 4


def test_block_above_4096_unsupported():
    assert rq(rows=1, n=8192, b=8192) == hq.HQ_EUNSUPPORTED
    assert rot(rows=1, n=8192, b=8192) == hq.HQ_EUNSUPPORTED
    assert inv(rows=1, n=8192, b=8192) == hq.HQ_EUNSUPPORTED
    # an invalid argument still wins over "unsupported"
    assert rq(rows=1, n=8192, b=8192, bits=5) == hq.HQ_EINVAL


def test_zero_rows_is_noop_without_pointers():
    assert rq(x=None, codes=None, scales=None, s=None, rows=0) == hq.HQ_OK
    assert inv(codes=None, scales=None, y=None, s=None, rows=0) == hq.HQ_OK
    assert rot(x=None, y=None, s=None, rows=0) == hq.HQ_OK
    # shape checks still apply at rows == 0
    assert rq(rows=0, n=100) == hq.HQ_EINVAL


def test_binding_rejects_host_tensors_and_bad_layouts():
    import torch
    x = torch.zeros((4, 128), dtype=torch.bfloat16)
    s = torch.ones(128, dtype=torch.int8)
    with pytest.raises(ValueError, match="GPU"):
        hq.hq_rotate_quant(x, s, 128)
    with pytest.raises(ValueError, match="GPU"):
        hq.hq_rotate(x, s, 128)
    with pytest.raises(ValueError, match="GPU"):
        hq.hq_dequant_rotate_inv(torch.zeros((4, 64), dtype=torch.uint8),
                                 torch.zeros(4), s, 128)
    with pytest.raises(ValueError, match="GPU"):
        hq.hq_rotate_quant_grouped(x, s, 128, 64)
    with pytest.raises(ValueError, match="GPU"):
        hq.hq_dequant_rotate_inv_grouped(torch.zeros((4, 64), dtype=torch.uint8),
                                         torch.zeros((4, 2)), s, 128, 64)
    with pytest.raises(ValueError, match="GPU"):
        hq.hq_rotate_quant_append(x, s, 128, torch.zeros(4, dtype=torch.int64),
                                  torch.zeros((16, 64), dtype=torch.uint8), torch.zeros(16))
    with pytest.raises(TypeError):
        hq.hq_rotate_quant(x.numpy() if False else [1, 2], s, 128)


def test_product_package_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "hadamard_rotation_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not re.search(r"^\s*(from|import)\s+oracle", text, re.M), f
                assert "hq_oracle" not in text and "liboracle" not in text, f


def test_full_width_rotation_that_is_not_a_power_of_two():
    # b == n with n = k * 2^m, k a Paley order: accepted (a no-op at rows 0)
    for n in (96, 688, 11008):
        assert rq(rows=0, n=n, b=n) == hq.HQ_OK
        assert inv(rows=0, n=n, b=n) == hq.HQ_OK
        assert rot(rows=0, n=n, b=n) == hq.HQ_OK
    # 496 = 31 * 16: no order 31 * 2^a - 1 is a prime power = 3 (mod 4)
    assert rq(rows=0, n=496, b=496) == hq.HQ_EINVAL
    # a block size that is neither a power of two nor the whole width
    assert rq(rows=0, n=11008, b=344) == hq.HQ_EINVAL
    assert rq(rows=0, n=11008, b=5504) == hq.HQ_EINVAL


def test_header_documents_every_accepted_block_size():
    # The header's shape rule, restated here: b a power of two dividing n
    # (above 4096 unsupported), or b == n for a width with a Paley split
    # (oracle.hadamard_split finds one); every other b is invalid.  The
    # library's decisions over a sweep of widths and block sizes must follow
    # it, and the header must state both accepted classes.
    from oracle import oracle as O
    text = open(HEADER).read()
    assert "b a power of two with n % b == 0" in text
    assert "b == n for a width n = k * 2^m that is not a power of two" in text
    assert "inverse" in text and "transpose" in text
    for n in list(range(16, 2049, 16)) + [11008, 10624, 8192, 16384]:
        pow2_n = (n & (n - 1)) == 0
        split = O.hadamard_split(n)
        for b in sorted({1, 2, 16, 128, 4096, 8192, n, n // 2, 3, 96, 344}):
            if b < 1:
                continue
            got = rq(rows=0, n=n, b=b, x=None, codes=None, scales=None, s=None)
            if (b & (b - 1)) == 0:
                want = hq.HQ_EINVAL if n % b else (hq.HQ_EUNSUPPORTED if b > 4096 else hq.HQ_OK)
            elif b == n and not pow2_n and split is not None:
                want = hq.HQ_OK
            else:
                want = hq.HQ_EINVAL
            if got == hq.HQ_EUNSUPPORTED and want == hq.HQ_EUNSUPPORTED:
                continue
            assert got == want, (n, b, got, want)


def test_decode_attention_binding_rejects_code_width():
    # codes of the wrong width would be read past their end by the kernel:
    # the binding raises on the host before anything is launched
    import torch
    q = torch.zeros((32, 128), dtype=torch.bfloat16)
    s = torch.ones(128, dtype=torch.int8)
    sc = torch.zeros((100, 8), dtype=torch.float16)
    good = torch.zeros((100, 8, 64), dtype=torch.uint8)
    for bad in (torch.zeros((100, 8, 32), dtype=torch.uint8),
                torch.zeros((100, 8, 128), dtype=torch.uint8),
                torch.zeros((100, 4, 64), dtype=torch.uint8),
                torch.zeros((100, 512), dtype=torch.uint8)):
        with pytest.raises(ValueError, match="codes must"):
            hq.hq_decode_attention(q, s, 128, bad, sc, good, sc)
        with pytest.raises(ValueError, match="codes must"):
            hq.hq_decode_attention(q, s, 128, good, sc, bad, sc)
    # the right width gets as far as the device check
    with pytest.raises(ValueError, match="GPU"):
        hq.hq_decode_attention(q, s, 128, good, sc, good, sc)
