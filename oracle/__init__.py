"""CPU oracle (test infrastructure only; the library never imports it)."""
from .pf_oracle import *  # noqa: F401,F403
from .pf_oracle import (HEAD_DIM, T_DIMS, H_DIMS, W_DIMS, ROPE_BASE, bf16_to_f64, f64_to_bf16,
                        tokens_per_block, compressed_tokens, context_size, kv_cache_bytes,
                        axis_freqs, rope_encode, rope_shift, rope_shift_blocks, block_scores,
                        select_topk, topk_gap, topk_acceptable, initial_pos_tags,
                        placement_deltas, gather_mid, attn_bruteforce, attn_partitioned,
                        partitions, layer_step, HR_STAGE_KERNELS, silu, hr_conv_stage,
                        hr_branch)
