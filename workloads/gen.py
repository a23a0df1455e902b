"""Seeded synthetic inputs for the FOCUS eviction hot path.

Both the HIP path and the float64 oracle consume exactly the tensors made
here: the GPU directly, the oracle after an exact bf16 -> float32 -> float64
widening. Nothing in this module computes any step of the method.

Recipe (per configuration, per seed):
  * prefix length P_b: fixed, or round(exp(ln(median) + sigma * z)) with
    z ~ N(0, 1), clipped to [lo, hi];
  * budget K_b = clamp(floor(f_b * B), 1, B) with f_b fixed or ~ U[lo, hi];
  * planted decodable tokens: n_b = max(1, round(p_b * B)) distinct block
    positions drawn uniformly, p_b fixed or ~ U[lo, hi];
  * per layer, Q / block K,V / prefix K,V are i.i.d. N(0, 1) float32 rounded
    to bf16 by round-to-nearest-even (float32 configs keep the float32
    values);
  * decoding-yield history (for the dynamic budget): halves in [0, 6];
  * still-masked flags (for the masked-candidate selection): decoded
    fraction f_b ~ U[0, 0.75], position j decoded with probability
    clip(f_b * (1.5 - j / B), 0, 1);
  * layer 1 only: the block keys of planted tokens get + bias * u_hat, where
    u is the mean of that sequence's layer-1 block queries over the B
    positions and the G query heads of the key's KV group, u_hat = u / |u|,
    added before the bf16 rounding of the keys.
Host metadata comes from numpy PCG64 seeded with SeedSequence([0xF0C5,
config, seed, ...]); tensors from torch generators seeded from the same
sequence, on the device they are made on (so CPU-made and GPU-made tensors of
one seed differ; every comparison feeds the same tensor to both sides).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

from .configs import FocusConfig

_ROOT = 0xF0C5
TENSOR_IDS = {"q": 0, "k_blk": 1, "v_blk": 2, "k_cache": 3, "v_cache": 4}


def seed_for(cfg: FocusConfig, seed: int, *parts: int) -> int:
    ss = np.random.SeedSequence([_ROOT, cfg.index, seed, *parts])
    return int(ss.generate_state(1, dtype=np.uint32)[0])


def torch_dtype(cfg: FocusConfig) -> torch.dtype:
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


@dataclasses.dataclass
class Metadata:
    prefix_lens: np.ndarray   # [N] int64
    k_keep: np.ndarray        # [N] int32
    planted: np.ndarray       # [N, B] bool

    @property
    def cu_prefix(self) -> np.ndarray:
        cu = np.zeros(len(self.prefix_lens) + 1, dtype=np.int64)
        np.cumsum(self.prefix_lens, out=cu[1:])
        return cu.astype(np.int32)


def draw_metadata(cfg: FocusConfig, seed: int = 0) -> Metadata:
    rng = np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([_ROOT, cfg.index, seed, 0x4D455441])))
    n, blk = cfg.batch, cfg.block
    if cfg.prefix_fixed is not None:
        plen = np.full(n, cfg.prefix_fixed, dtype=np.int64)
    else:
        median, sigma, lo, hi = cfg.prefix_lognormal
        z = rng.standard_normal(n)
        plen = np.clip(np.rint(np.exp(np.log(median) + sigma * z)), lo, hi)
        plen = plen.astype(np.int64)
    if cfg.budget_fixed is not None:
        frac = np.full(n, cfg.budget_fixed)
    else:
        frac = rng.uniform(cfg.budget_uniform[0], cfg.budget_uniform[1], n)
    k_keep = np.clip(np.floor(frac * blk + 1e-9), 1, blk).astype(np.int32)
    if cfg.planted_fixed is not None:
        pfrac = np.full(n, cfg.planted_fixed)
    else:
        pfrac = rng.uniform(cfg.planted_uniform[0], cfg.planted_uniform[1], n)
    planted = np.zeros((n, blk), dtype=bool)
    for b in range(n):
        cnt = max(1, int(np.rint(pfrac[b] * blk)))
        planted[b, rng.choice(blk, size=min(cnt, blk), replace=False)] = True
    return Metadata(plen, k_keep, planted)


def draw_masked(cfg: FocusConfig, seed: int = 0,
                decoded_max: float = 0.75) -> np.ndarray:
    """Still-masked flags [N, B] uint8 for a later denoising step of the
    block: sequence b has decoded fraction f_b ~ U[0, decoded_max], and
    position j is already decoded with probability
    clip(f_b * (1.5 - j / B), 0, 1) (earlier positions decode first, as in
    semi-autoregressive block decoding). 1 = still masked."""
    rng = np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([_ROOT, cfg.index, seed, 0x4D41534B])))
    n, blk = cfg.batch, cfg.block
    f = rng.uniform(0.0, decoded_max, n)
    pos = np.arange(blk) / blk
    p_dec = np.clip(f[:, None] * (1.5 - pos[None, :]), 0.0, 1.0)
    decoded = rng.random((n, blk)) < p_dec
    return (~decoded).astype(np.uint8)


def draw_yield(cfg: FocusConfig, seed: int = 0) -> np.ndarray:
    """Decoding-yield history per sequence for the dynamic budget: tokens
    decoded at the previous step, drawn as halves in [0, 6] (exact in
    float32) with mean near the pages' ~3 decoded tokens per step."""
    rng = np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([_ROOT, cfg.index, seed, 0x59494C44])))
    return (rng.integers(0, 13, cfg.batch) / 2.0).astype(np.float32)


def _randn(shape, cfg, seed, layer, name, device) -> torch.Tensor:
    gen = torch.Generator(device=device)
    gen.manual_seed(seed_for(cfg, seed, 0x4C59, layer, TENSOR_IDS[name]))
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def make_layer(cfg: FocusConfig, meta: Metadata, seed: int, layer: int,
               device="cpu", planted: bool = False) -> Dict[str, torch.Tensor]:
    """One layer's tensors in the library layout.

    q [N*B, Hq, d]; k_blk, v_blk [N*B, Hkv, d]; k_cache, v_cache
    [sum P_b, Hkv, d]; all in the config's dtype on ``device``.
    """
    n, blk, hq, hkv, d = cfg.batch, cfg.block, cfg.hq, cfg.hkv, cfg.head_dim
    total_prefix = int(meta.prefix_lens.sum())
    dt = torch_dtype(cfg)
    out: Dict[str, torch.Tensor] = {}
    out["q"] = _randn((n * blk, hq, d), cfg, seed, layer, "q", device).to(dt)
    kb = _randn((n * blk, hkv, d), cfg, seed, layer, "k_blk", device)
    if planted:
        # mean layer-1 query direction per (sequence, KV group)
        qf = out["q"].float().view(n, blk, hkv, cfg.group, d)
        u = qf.mean(dim=(1, 3))                               # [N, Hkv, d]
        u_hat = u / u.norm(dim=-1, keepdim=True).clamp_min(1e-30)
        mask = torch.as_tensor(meta.planted, device=device).to(torch.float32)
        kb = kb.view(n, blk, hkv, d)
        kb = kb + cfg.planted_bias * mask[:, :, None, None] * u_hat[:, None]
        kb = kb.reshape(n * blk, hkv, d)
    out["k_blk"] = kb.to(dt)
    del kb
    out["v_blk"] = _randn((n * blk, hkv, d), cfg, seed, layer, "v_blk",
                          device).to(dt)
    out["k_cache"] = _randn((total_prefix, hkv, d), cfg, seed, layer,
                            "k_cache", device).to(dt)
    out["v_cache"] = _randn((total_prefix, hkv, d), cfg, seed, layer,
                            "v_cache", device).to(dt)
    return out


@dataclasses.dataclass
class Inputs:
    cfg: FocusConfig
    seed: int
    meta: Metadata
    layers: List[Dict[str, torch.Tensor]]   # layer 0, layer 1, extra...

    @property
    def cu_prefix(self) -> np.ndarray:
        return self.meta.cu_prefix


def make_inputs(cfg: FocusConfig, seed: int = 0, device="cpu",
                n_layers: Optional[int] = None,
                prefix_lens: Optional[Sequence[int]] = None,
                k_keep: Optional[Sequence[int]] = None) -> Inputs:
    """Layers 0 and 1 (planted bias on layer 1) plus ``n_layers - 2``
    further layers (default: the config's extra layers)."""
    meta = draw_metadata(cfg, seed)
    if prefix_lens is not None:
        meta.prefix_lens = np.asarray(prefix_lens, dtype=np.int64)
    if k_keep is not None:
        meta.k_keep = np.asarray(k_keep, dtype=np.int32)
    if n_layers is None:
        n_layers = 2 + cfg.extra_layers
    layers = [make_layer(cfg, meta, seed, l, device, planted=(l == 1))
              for l in range(n_layers)]
    return Inputs(cfg, seed, meta, layers)


def to_f32_numpy(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a bf16/f32 tensor to a float32 numpy array."""
    return t.detach().to("cpu", torch.float32).numpy()
