"""MI355X-native batch-1 Llama decode: one persistent cooperative HIP kernel per token.

The product is the C-ABI library ``libamk.so`` (include/amk.h); ``amk`` is its ctypes binding.
"""
from .amk import (AMK_BF16, AMK_W4A16, AMK_W4A16_G128, AMK_W8A16, AMK_W8A16_BF16_HEAD, AmkError, Decoder, amk_decode_step, amk_decode_step_noalloc,  # noqa: F401
                  amk_decode_step_greedy, amk_export_quantized, amk_free, amk_get_info, amk_kv_cache_bytes,
                  amk_load_weights, amk_quantize_int4, amk_quantize_int4_g128, amk_quantize_int8, amk_set_dump, amk_set_spin_limit,
                  amk_set_trace, amk_status_string, amk_sync, amk_validate_config, make_config)
from .checkpoint import CheckpointError, LlamaShape, load_checkpoint  # noqa: F401,E402
