"""MI355X-native KIVI-style low-bit KV cache: HIP kernels behind a C ABI.

``bit_quantization_amd.kivi`` is the thin Python binding of ``libkivi.so``.
"""
from . import kivi  # noqa: F401
from .kivi import (Cache, Dims, KiviError, kivi_append_flush, kivi_cache_sizes,  # noqa: F401
                   kivi_decode_attn, kivi_decode_splits, kivi_decode_workspace_bytes,
                   kivi_quantize_k, kivi_quantize_v, new_workspace)
