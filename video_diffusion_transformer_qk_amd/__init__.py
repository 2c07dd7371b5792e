"""h3attn: MI355X-native (gfx950) attention hot path of a MiniMax-H3-class video DiT.

Four calls, each a hand-written HIP kernel behind a C ABI (include/h3attn.h):
  qk_norm_rope      fused per-head QK RMSNorm + 3D (t/h/w) RoPE
                    (qk_norm_rope_pool also pools q', k' for the selection in the same pass, and
                    subblock_select_pooled finishes the selection from that)
  dense_fwd         dense bf16 self-attention over the full latent sequence
  subblock_select   SubBlock 64-token block scores and per-query-block top-k
  block_sparse_fwd  attention over the kept key blocks only
Threshold mode: subblock_select_threshold (blocks within tau of the row's best, CSR) and
block_sparse_csr_fwd (variable kept set per query block).
Other fused block ops of the runtime: adaln_modulate (LayerNorm * (1 + scale) + shift) and swiglu.
Cache-DiT step reuse: residual_change (L1 change between adjacent steps) and CacheGate (policy).
FP8 (e4m3) attention: fp8_quantize, fp8_dense_fwd, fp8_block_sparse_fwd.
"""
from ._lib import (LIB_PATH, SIGNATURES, H3AttnError, block_sparse_csr_fwd, block_sparse_fwd,  # noqa: F401
                   dense_fwd, keep_count, load_library, qk_norm_rope, select_workspace_bytes,
                   subblock_select, subblock_select_threshold, threshold_workspace_bytes, version,
                   adaln_modulate, swiglu, residual_change, CacheGate, Fp8QKV, fp8_workspace_bytes,
                   fp8_quantize, fp8_dense_fwd, fp8_block_sparse_fwd, frame_group_stride, check_block_idx, check_csr,
                   qk_norm_rope_pool, subblock_select_pooled, PooledBlocks)

__all__ = ["qk_norm_rope", "qk_norm_rope_pool", "subblock_select_pooled", "PooledBlocks", "dense_fwd", "subblock_select", "block_sparse_fwd", "keep_count",
           "select_workspace_bytes", "subblock_select_threshold", "block_sparse_csr_fwd",
           "threshold_workspace_bytes", "adaln_modulate", "swiglu",
           "residual_change", "CacheGate", "Fp8QKV", "fp8_workspace_bytes", "fp8_quantize",
           "fp8_dense_fwd", "fp8_block_sparse_fwd", "frame_group_stride", "check_block_idx", "check_csr", "version",
           "H3AttnError", "load_library"]
