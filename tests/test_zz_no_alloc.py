"""focus_block_attn_importance_noalloc against focus_block_attn_importance
(order = NULL, caller workspace) through the C ABI (needs an MI355X).

Both run the same kernels, so every output must be bitwise equal. Two calls
in a row share the library's static scratch: the second, on a smaller
batch and on a stream of its own, must not see the first call's order.
"""
import numpy as np
import pytest
import torch

import workloads
from tests import parity
from tests.parity import log

pytestmark = pytest.mark.gpu


def _both(F, inp, lay, stream):
    cfg = inp.cfg
    dm = parity.dims_of(cfg)
    cu = torch.as_tensor(inp.cu_prefix.astype(np.int32), device="cuda")
    max_prefix = int(inp.meta.prefix_lens.max())
    res = []
    for variant in ("workspace", "noalloc"):
        out = torch.full_like(lay[0]["q"], float("nan"))
        imp = torch.full((cfg.batch, cfg.hq, cfg.block), float("nan"), device="cuda")
        lse = torch.full_like(imp, float("nan"))
        if variant == "workspace":
            nbytes = F.focus_block_attn_importance_workspace(
                cfg.batch, cfg.block, cfg.hq, cfg.hkv, cfg.head_dim, max_prefix)
            ws = torch.full((max(nbytes, 16),), 0x5A, dtype=torch.uint8, device="cuda")
            F.focus_block_attn_importance(
                F.FOCUS_BF16, dm.batch, dm.block, dm.hq, dm.hkv, dm.head_dim, 0.0,
                lay[0]["q"], lay[0]["k_blk"], lay[0]["v_blk"], lay[0]["k_cache"],
                lay[0]["v_cache"], cu, None, max_prefix, out, imp, lse, ws, nbytes,
                stream=stream)
        else:
            F.focus_block_attn_importance_noalloc(
                F.FOCUS_BF16, dm.batch, dm.block, dm.hq, dm.hkv, dm.head_dim, 0.0,
                lay[0]["q"], lay[0]["k_blk"], lay[0]["v_blk"], lay[0]["k_cache"],
                lay[0]["v_cache"], cu, max_prefix, out, imp, lse, stream=stream)
        res.append((out, imp, lse))
    torch.cuda.synchronize()
    return res


def test_noalloc_equals_workspace_call_twice():
    import attention_delta_token_focus_amd as F
    side = torch.cuda.Stream()
    for i, (batch, seed, stream) in enumerate([(48, 21, None), (9, 22, side)]):
        cfg = workloads.scaled(workloads.get("c3"), batch=batch)
        log(f"[no-alloc] call {i + 1}: N={batch} B={cfg.block} seed={seed}")
        inp = workloads.make_inputs(cfg, seed, n_layers=2)
        lay = parity.to_device(inp)
        (o1, i1, l1), (o2, i2, l2) = _both(F, inp, lay, stream)
        assert torch.equal(o1, o2), "out differs"
        assert torch.equal(i1, i2), "imp differs"
        assert torch.equal(l1, l2), "lse differs"
        assert not torch.isnan(o2).any() and not torch.isnan(i2).any()
        # and both agree with the oracle on a few sequences (the bars of
        # the parity tests)
        seqs = [0, batch - 1]
        sub, sub_cu = parity.sub_layers(inp.layers[:1], inp.cu_prefix, cfg.block, seqs)
        import oracle
        ref = oracle.block_attn_importance(
            sub[0]["q"], sub[0]["k_blk"], sub[0]["v_blk"], sub[0]["k_cache"],
            sub[0]["v_cache"], sub_cu, cfg.block, cfg.hq, cfg.hkv)
        parity.assert_close("out", parity.rows_of(workloads.to_f32_numpy(o2), seqs,
                                                  cfg.block),
                            ref[0], 2e-2, 8e-3, rel_scale=True)
        parity.assert_close("imp", i2.cpu().numpy()[seqs], ref[1], 2e-2, 1e-4)
