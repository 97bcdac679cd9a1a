"""CPU float64 oracle for the DeepSeekMoE layer (test infrastructure only; see moe_oracle)."""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (affinities, selection_keys, topk_select, group_limited_select, gates, route, dispatch,
                         dispatch_by_rank, pack_fp8_payload, unpack_fp8_payload,  # noqa: F401
                         e4m3fn_decode, e4m3fn_encode, quantize_tiles, dequantize_tiles, fp8_roundtrip,
                         fp8_roundtrip_row_blocks, swiglu_ffn_backward_fp8,
                         silu, swiglu_ffn, swiglu_ffn_backward, layer_forward, layer_backward, seq_balance_loss, bias_update, load_stats, bf16_to_f64, as_f64,
                         E4M3_MAX)
