"""One importance + evict block-step through the libfocus entry points.

Order of calls per step (one stream, no host synchronisation):
  focus_schedule (longest-prefix-first visiting order, shared by the
  attention calls of the step; with shared_order=False there is no such
  call and each attention call computes the order itself, order=NULL);
  focus_block_attn_importance on layer 0, then on layer 1 (with
  l1_output=False layer 1 gets out=NULL: importance and lse only, no V
  read, no P V product);
  focus_select (head mean, MaxPool1D, delta, top-K and the retained
  indices with per-sequence offsets, in one launch), or the same as two
  calls, focus_delta_topk then focus_compact (fused=False); with a mask of
  still-masked positions or structural rules, focus_select_masked instead
  (the retained count is then data-dependent: the retained buffers are
  sized for all batch*B tokens and max_ret = B);
  focus_retained_attn once per further layer.
This module only allocates the output buffers (torch device memory) and
calls the binding; it computes nothing itself.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

from . import (dtype_code, focus_block_attn_importance,
               focus_block_attn_importance_workspace, focus_compact,
               focus_delta_topk, focus_retained_attn,
               focus_retained_attn_workspace, focus_schedule, focus_select,
               focus_select_dynamic, focus_select_masked)


@dataclasses.dataclass(frozen=True)
class Dims:
    batch: int
    block: int
    hq: int
    hkv: int
    head_dim: int
    dtype: torch.dtype
    pool_k: int = 3
    scale: float = 0.0  # <= 0: 1/sqrt(head_dim)


def retained_counts(k_keep_host: Sequence[int], block: int):
    """n_ret and max_ret known on the host from the budgets alone: top-K
    keeps exactly min(max(K_b, 0), B) tokens of sequence b."""
    kb = np.clip(np.asarray(k_keep_host, dtype=np.int64), 0, block)
    return int(kb.sum()), int(kb.max()) if len(kb) else 0


class FocusStep:
    """Buffers and calls for one block-step over a fixed batch."""

    def __init__(self, dims: Dims, cu_prefix_host: Sequence[int],
                 k_keep_host: Sequence[int], n_further: int = 0,
                 device="cuda", with_lse: bool = False, fused: bool = True,
                 l1_output: bool = True, masked=None, rules: int = 0,
                 yield_hist=None, alpha: float = 1.5, shared_order: bool = True):
        self.dims = dims
        self.fused = fused
        # shared_order=False: no focus_schedule call; every attention call
        # gets order=NULL and writes the visiting order into its workspace
        self.shared_order = shared_order
        self.l1_output = l1_output
        self.constrained = (masked is not None or rules != 0
                            or yield_hist is not None)
        self.rules = rules
        self.alpha = alpha
        dv = torch.device(device)
        n, blk, hq, d = dims.batch, dims.block, dims.hq, dims.head_dim
        cu = np.asarray(cu_prefix_host, dtype=np.int64)
        self.max_prefix = int(np.diff(cu).max()) if n else 0
        self.cu_prefix = torch.as_tensor(cu.astype(np.int32), device=dv)
        self.k_keep = torch.as_tensor(
            np.asarray(k_keep_host, dtype=np.int32), device=dv)
        self.n_ret, self.max_ret = retained_counts(k_keep_host, blk)
        self.masked = None
        self.cand = None
        if self.constrained:
            # upper bounds: every retained count is at most B
            self.n_ret, self.max_ret = n * blk, blk
            if masked is not None:
                self.masked = torch.as_tensor(
                    np.asarray(masked, dtype=np.uint8), device=dv).contiguous()
            self.cand = torch.empty((n, blk), device=dv, dtype=torch.uint8)
        self.yield_hist = None
        self.k_used = None
        if yield_hist is not None:
            self.yield_hist = torch.as_tensor(
                np.asarray(yield_hist, dtype=np.float32), device=dv).contiguous()
            self.k_used = torch.empty((n,), device=dv, dtype=torch.int32)
        f32 = dict(device=dv, dtype=torch.float32)
        self.out = [torch.empty((n * blk, hq, d), device=dv, dtype=dims.dtype)
                    if w == 0 or l1_output else None for w in range(2)]
        self.imp = [torch.empty((n, hq, blk), **f32) for _ in range(2)]
        self.lse = ([torch.empty((n, hq, blk), **f32) for _ in range(2)]
                    if with_lse else [None, None])
        self.dI = torch.empty((n, blk), **f32)
        self.keep = torch.empty((n, blk), device=dv, dtype=torch.uint8)
        self.idx = torch.empty((max(n * blk, 1),), device=dv,
                               dtype=torch.int32)
        self.cu_ret = torch.empty((n + 1,), device=dv, dtype=torch.int32)
        self.order = torch.empty((n,), device=dv, dtype=torch.int32)
        self.ret_out = [torch.empty((max(self.n_ret, 1), hq, d), device=dv,
                                    dtype=dims.dtype)
                        for _ in range(n_further)]
        ws_a = focus_block_attn_importance_workspace(
            n, blk, hq, dims.hkv, d, self.max_prefix)
        ws_r = focus_retained_attn_workspace(
            n, hq, dims.hkv, d, self.max_prefix, self.n_ret, self.max_ret)
        self.ws_bytes = max(ws_a, ws_r)
        self.ws = (torch.empty((self.ws_bytes,), device=dv, dtype=torch.uint8)
                   if self.ws_bytes else None)

    # -- single calls -----------------------------------------------------
    def schedule(self, stream=None) -> None:
        if self.shared_order:
            focus_schedule(self.dims.batch, self.cu_prefix, self.order, stream)

    def _order(self):
        return self.order if self.shared_order else None

    def block_attn(self, layer: Dict[str, torch.Tensor], which: int,
                   stream=None) -> None:
        dm = self.dims
        focus_block_attn_importance(
            dtype_code(dm.dtype), dm.batch, dm.block, dm.hq, dm.hkv,
            dm.head_dim, dm.scale, layer["q"], layer["k_blk"],
            layer["v_blk"] if self.out[which] is not None else None,
            layer["k_cache"],
            layer["v_cache"] if self.out[which] is not None else None,
            self.cu_prefix, self._order(),
            self.max_prefix, self.out[which], self.imp[which],
            self.lse[which], self.ws, self.ws_bytes, stream)

    def select(self, stream=None) -> None:
        dm = self.dims
        if self.yield_hist is not None:
            focus_select_dynamic(dm.batch, dm.block, dm.hq, dm.pool_k,
                                 self.imp[0], self.imp[1], self.masked,
                                 self.yield_hist, self.alpha, self.rules,
                                 self.keep, self.k_used, self.cand, self.dI,
                                 self.idx, self.cu_ret, stream)
            return
        if self.constrained:
            focus_select_masked(dm.batch, dm.block, dm.hq, dm.pool_k,
                                self.imp[0], self.imp[1], self.masked,
                                self.k_keep, self.rules, self.keep, self.cand,
                                self.dI, self.idx, self.cu_ret, stream)
            return
        if self.fused:
            focus_select(dm.batch, dm.block, dm.hq, dm.pool_k, self.imp[0],
                         self.imp[1], self.k_keep, self.keep, self.dI,
                         self.idx, self.cu_ret, stream)
            return
        focus_delta_topk(dm.batch, dm.block, dm.hq, dm.pool_k, self.imp[0],
                         self.imp[1], self.k_keep, self.keep, self.dI, stream)
        focus_compact(dm.batch, dm.block, self.keep, self.idx, self.cu_ret,
                      stream)

    def retained(self, layer: Dict[str, torch.Tensor], which: int,
                 stream=None) -> None:
        dm = self.dims
        focus_retained_attn(
            dtype_code(dm.dtype), dm.batch, dm.block, dm.hq, dm.hkv,
            dm.head_dim, dm.scale, layer["q"], layer["k_blk"], layer["v_blk"],
            self.idx, self.cu_ret, self.n_ret, self.max_ret,
            layer["k_cache"], layer["v_cache"], self.cu_prefix, self._order(),
            self.max_prefix, self.ret_out[which], self.ws, self.ws_bytes,
            stream)

    # -- the whole step ---------------------------------------------------
    def run(self, layers: List[Dict[str, torch.Tensor]], stream=None) -> None:
        """layers[0], layers[1]: importance layers; layers[2:]: further
        layers run on the retained tokens."""
        self.schedule(stream)
        self.block_attn(layers[0], 0, stream)
        self.block_attn(layers[1], 1, stream)
        self.select(stream)
        for i, lay in enumerate(layers[2:2 + len(self.ret_out)]):
            self.retained(lay, i, stream)
