"""MI355X-native forward pass of the nanochat-style GPT decoder block.

The compute path is libgpt.so (hand-written HIP for gfx950, C ABI in
include/gpt.h); ``binding`` is its ctypes wrapper.
"""
from .binding import (GptConfig, GptError, GptWeights, DeviceKV, DeviceModel, gpt_decode_step,
                      gpt_prefill, gpt_profile_enable, gpt_profile_read, gpt_select_tokens,
                      gpt_workspace_bytes, kv_cache_alloc, kv_cache_bytes, kv_cache_free,
                      kv_cache_lengths, lib, make_config, rope_tables, ROWS_ALL, ROWS_LAST)
