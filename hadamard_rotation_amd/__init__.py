"""MI355X-native randomized Hadamard rotation fused with symmetric low-bit
quantisation.

The computation lives in libhq.so (hand-written HIP kernels for gfx950,
C ABI in include/hq.h); this package is its thin ctypes binding plus the
seeded synthetic workloads used by the tests and the benchmark.
"""
from .binding import (HQ_BF16, HQ_EHIP, HQ_EINVAL, HQ_EUNSUPPORTED, HQ_F16, HQ_F32,  # noqa: F401
                      HQ_OK, HQError, hq_decode_attention, hq_decode_attention_noalloc,
                      hq_decode_attention_workspace,
                      hq_dequant_rotate_inv, hq_dequant_rotate_inv_grouped,
                      hq_max_n, hq_rotate, hq_rotate_quant, hq_rotate_quant_append,
                      hq_rotate_quant_grouped, hq_version, load, status_str)

__all__ = ["hq_rotate_quant", "hq_dequant_rotate_inv", "hq_rotate_quant_grouped",
           "hq_rotate_quant_append", "hq_decode_attention", "hq_decode_attention_workspace",
           "hq_decode_attention_noalloc",
           "hq_dequant_rotate_inv_grouped", "hq_rotate", "hq_max_n", "hq_version",
           "status_str", "load", "HQError"]
