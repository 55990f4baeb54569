"""Helpers for the GPU tests: move seeded host inputs to the device, call the
library through its binding, bring results back as numpy."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import hadamard_rotation_amd as hq
from hadamard_rotation_amd.workloads import BF16, F16, F32

TORCH_DT = {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16}


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    hq.load()  # fail loudly if the HIP library is missing


def to_dev(raw: np.ndarray, dtype: int, device="cuda") -> torch.Tensor:
    if dtype == F32:
        return torch.from_numpy(np.ascontiguousarray(raw, dtype=np.float32)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).to(device)
    return t.view(TORCH_DT[dtype])


def s_dev(s: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(s, dtype=np.int8)).to(device)


def gpu_rotate_quant(raw, x_dtype, s, b, bits, scale_dtype, stream=None):
    x = to_dev(raw, x_dtype)
    sd = torch.float32 if scale_dtype == F32 else torch.float16
    codes, scales = hq.hq_rotate_quant(x, s_dev(s), b, bits, sd, stream=stream)
    torch.cuda.synchronize()
    c = codes.cpu().numpy().view(np.uint8)
    sc = scales.cpu().numpy()
    return c, sc


def gpu_rotate(raw, x_dtype, s, b):
    y = hq.hq_rotate(to_dev(raw, x_dtype), s_dev(s), b)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def gpu_dequant_inv(codes: np.ndarray, scales: np.ndarray, s, b, bits, out_bf16=False):
    c = torch.from_numpy(np.ascontiguousarray(codes).view(np.uint8 if bits == 4 else np.int8)).cuda()
    sc = torch.from_numpy(np.ascontiguousarray(scales)).cuda()
    y = hq.hq_dequant_rotate_inv(c, sc, s_dev(s), b, bits,
                                 torch.bfloat16 if out_bf16 else torch.float32)
    torch.cuda.synchronize()
    if out_bf16:
        return y.view(torch.int16).cpu().numpy().view(np.uint16)
    return y.cpu().numpy()


def gpu_rotate_quant_grouped(raw, x_dtype, s, b, group, bits, scale_dtype):
    x = to_dev(raw, x_dtype)
    sd = torch.float32 if scale_dtype == F32 else torch.float16
    codes, scales = hq.hq_rotate_quant_grouped(x, s_dev(s), b, group, bits, sd)
    torch.cuda.synchronize()
    return codes.cpu().numpy().view(np.uint8), scales.cpu().numpy()


def gpu_dequant_inv_grouped(codes: np.ndarray, scales: np.ndarray, s, b, group, bits,
                            out_bf16=False):
    c = torch.from_numpy(np.ascontiguousarray(codes).view(np.uint8 if bits == 4 else np.int8)).cuda()
    sc = torch.from_numpy(np.ascontiguousarray(scales)).cuda()
    y = hq.hq_dequant_rotate_inv_grouped(c, sc, s_dev(s), b, group, bits,
                                         torch.bfloat16 if out_bf16 else torch.float32)
    torch.cuda.synchronize()
    if out_bf16:
        return y.view(torch.int16).cpu().numpy().view(np.uint16)
    return y.cpu().numpy()
