"""MI355X-native fused causal grouped-query flash-attention prefill.

The compute lives in libattn_prefill.so (hand-written HIP for gfx950 behind
the C ABI in include/attn_prefill.h); this package is its Python binding
(`binding`) and the seeded synthetic-input generator (`synth`).
"""
from .binding import (AttnDeclined, AttnError, attn_config_count, attn_config_name,  # noqa: F401
                      attn_force_config, attn_last_error, attn_prefill, attn_prefill_varlen,
                      attn_tune_reset, attn_tune_stats)
