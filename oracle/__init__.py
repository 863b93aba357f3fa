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
