"""Float64 CPU oracle of the FOCUS eviction hot path.

TEST INFRASTRUCTURE ONLY: importable by the test suite, the smoke entry
point and the benchmark's CPU-baseline leg, never by the product path.
"""
from .focus_oracle import (attention_rows, block_attn_importance,  # noqa: F401
                           block_step, compact, default_scale, dynamic_budget,
                           head_mean_maxpool, importance_delta,
                           retained_attn, select_constrained, topk_keep)
