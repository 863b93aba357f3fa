"""CPU oracle (test infrastructure only; never imported by the product path).

See ``oracle/kivi_ref.py`` for the definitions, the page citations and the readings
taken where the pages are silent.
"""
from .kivi_ref import *  # noqa: F401,F403
from .kivi_ref import (LayerCache, attention_fp64, dequantize, dequantize_keys,  # noqa: F401
                       dequantize_values, gqa_attention_fp64, kivi_cache_bytes,
                       kv_cache_bytes, pack_keys, pack_words, pack_values,
                       quantize_groups, quantize_keys, quantize_values, quantized_len,
                       residual_len, residual_len_grouped, unpack_keys, unpack_words,
                       unpack_values)
from .fp8_ref import (FP8Cache, RUN_ORDER, dequantize_fp8, fp8_decode, fp8_encode,  # noqa: F401
                      fp8_value, finite_table, pack_value_runs, quantize_fp8,
                      unpack_value_runs)
from .mxfp4_ref import (MXFP4Cache, block_exponent, dequantize_mx, e2m1_decode,  # noqa: F401
                        e2m1_encode, e2m1_value, pack_nibbles, pack_value_runs as pack_mx_value_runs,
                        pack_value_scales, quantize_mx, unpack_nibbles)
