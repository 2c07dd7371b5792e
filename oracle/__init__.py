"""Float64 CPU oracle (test infrastructure only; see attention_oracle's header)."""
from .attention_oracle import (attention, attention_head, block_means, block_scores,  # noqa: F401
                               block_token_ids, keep_count, n_blocks_of, near_tie_rows,
                               qk_norm_rope, rms_norm, rope3d, rope_frequencies,
                               sparse_attention, sparse_attention_rows, subblock_select,
                               token_positions, topk_blocks, threshold_blocks,
                               subblock_select_threshold, near_threshold_entries,
                               sparse_attention_csr, adaln_modulate, swiglu, residual_change,
                               CacheGate, E4M3_MAX, e4m3_values, e4m3_round, pow2_scale,
                               quantize_blocks, quantize_channels, attention_fp8,
                               sparse_attention_fp8, attention_fp8_rows,
                               attention_fp8_detail)
