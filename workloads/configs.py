"""The seeded synthetic workloads of the FOCUS eviction hot path.

Shapes follow the block-diffusion setting reviewed on the pith.science page
for "FOCUS: DLLMs Know How to Tame Their Compute Bound" (arXiv 2601.23278):
blocks of B tokens (B = 32 and larger blocks, Fig. 9 / Figs. 6-7), about 10%
of a block decodable per step (Fig. 2), 65-80% of per-step token processing
removed ("The pith"), MaxPool1D kernel 3 (Free-Parameter Ledger, Eq. 15).
The attention shape (32 query heads, 8 KV heads, head_dim 128) is an 8B-class
GQA layout. The public chat datasets the pages measure throughput on are not
used; lognormal prefix lengths stand in for their history lengths.

This module holds no arithmetic of the method; it only describes inputs.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple


@dataclasses.dataclass(frozen=True)
class FocusConfig:
    name: str
    index: int                 # stable id used in seeds
    batch: int                 # N sequences
    block: int                 # B block tokens per sequence
    hq: int                    # query heads
    hkv: int                   # KV heads
    head_dim: int              # d
    dtype: str                 # "bf16" or "f32"
    pool_k: int                # MaxPool1D kernel (odd)
    # prefix lengths: fixed, or lognormal(median, sigma) clipped to [lo, hi]
    prefix_fixed: Optional[int] = None
    prefix_lognormal: Optional[Tuple[float, float, int, int]] = None
    # retention budget: fixed fraction, or uniform [lo, hi] per sequence
    budget_fixed: Optional[float] = None
    budget_uniform: Optional[Tuple[float, float]] = None
    # planted decodable fraction: fixed, or uniform [lo, hi] per sequence
    planted_fixed: Optional[float] = None
    planted_uniform: Optional[Tuple[float, float]] = None
    planted_bias: float = 0.5  # multiple of the unit mean-query direction
    extra_layers: int = 0      # retained-attention layers after layer 1

    @property
    def group(self) -> int:
        return self.hq // self.hkv


CONFIGS = {
    "c1": FocusConfig(
        name="c1_tiny_f32", index=1, batch=1, block=32, hq=4, hkv=1,
        head_dim=64, dtype="f32", pool_k=3, prefix_fixed=64,
        budget_fixed=8 / 32, planted_fixed=0.10),
    "c2": FocusConfig(
        name="c2_bf16_n32_p512", index=2, batch=32, block=32, hq=32, hkv=8,
        head_dim=128, dtype="bf16", pool_k=3, prefix_fixed=512,
        budget_fixed=0.35, planted_fixed=0.10),
    "c3": FocusConfig(
        name="c3_bf16_n256_b32_lognormal1024", index=3, batch=256, block=32,
        hq=32, hkv=8, head_dim=128, dtype="bf16", pool_k=3,
        prefix_lognormal=(1024.0, 0.8, 128, 4096),
        budget_uniform=(0.20, 0.35), planted_uniform=(0.05, 0.20)),
    "c4": FocusConfig(
        name="c4_bf16_n64_b128_p2048", index=4, batch=64, block=128, hq=32,
        hkv=8, head_dim=128, dtype="bf16", pool_k=5, prefix_fixed=2048,
        budget_fixed=0.25, planted_fixed=0.10),
    "c5": FocusConfig(
        name="c5_bf16_n128_b32_lognormal2048_fullstep", index=5, batch=128,
        block=32, hq=32, hkv=8, head_dim=128, dtype="bf16", pool_k=3,
        prefix_lognormal=(2048.0, 0.8, 256, 8192), budget_fixed=0.30,
        planted_fixed=0.10, extra_layers=34),
    # Block size 64, the setting of the pages' largest speed-up (Fig. 7,
    # per the Pith page's Referee Report; B = 64 also in Fig. 9); otherwise
    # shaped like c3.
    "c6": FocusConfig(
        name="c6_bf16_n128_b64_lognormal1024", index=6, batch=128, block=64,
        hq=32, hkv=8, head_dim=128, dtype="bf16", pool_k=3,
        prefix_lognormal=(1024.0, 0.8, 128, 4096),
        budget_uniform=(0.20, 0.35), planted_uniform=(0.05, 0.20)),
}


def get(name: str) -> FocusConfig:
    return CONFIGS[name]


def scaled(cfg: FocusConfig, **changes) -> FocusConfig:
    """A copy of ``cfg`` with some fields replaced (smaller parity cases)."""
    return dataclasses.replace(cfg, **changes)
