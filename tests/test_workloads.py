"""The seeded input generator (CPU only): determinism, shapes, recipe."""
import numpy as np
import pytest
import torch

import workloads
from workloads import gen


def test_metadata_ranges_follow_the_configs():
    m = workloads.draw_metadata(workloads.get("c3"), 0)
    assert m.prefix_lens.min() >= 128 and m.prefix_lens.max() <= 4096
    assert 900 < np.median(m.prefix_lens) < 1150
    assert m.k_keep.min() >= 6 and m.k_keep.max() <= 11
    cnt = m.planted.sum(axis=1)
    assert cnt.min() >= 2 and cnt.max() <= 6
    for name, k in (("c1", 8), ("c2", 11), ("c4", 32), ("c5", 9)):
        m = workloads.draw_metadata(workloads.get(name), 0)
        assert (m.k_keep == k).all(), name
    m5 = workloads.draw_metadata(workloads.get("c5"), 0)
    assert m5.prefix_lens.min() >= 256 and m5.prefix_lens.max() <= 8192
    assert (workloads.draw_metadata(workloads.get("c4"), 0)
            .planted.sum(axis=1) == 13).all()


def test_same_seed_same_bits_other_seed_other_bits():
    cfg = workloads.scaled(workloads.get("c2"), batch=2, prefix_fixed=16)
    a = workloads.make_inputs(cfg, 7)
    b = workloads.make_inputs(cfg, 7)
    c = workloads.make_inputs(cfg, 8)
    for la, lb, lc in zip(a.layers, b.layers, c.layers):
        for k in la:
            assert la[k].dtype == torch.bfloat16
            assert torch.equal(la[k].view(torch.int16), lb[k].view(torch.int16))
            assert not torch.equal(la[k], lc[k])
    assert not torch.equal(a.layers[0]["q"], a.layers[1]["q"])


def test_shapes():
    cfg = workloads.scaled(workloads.get("c3"), batch=3)
    inp = workloads.make_inputs(cfg, 0)
    tot = int(inp.meta.prefix_lens.sum())
    lay = inp.layers[1]
    assert lay["q"].shape == (3 * 32, 32, 128)
    assert lay["k_blk"].shape == (3 * 32, 8, 128)
    assert lay["k_cache"].shape == (tot, 8, 128)
    assert inp.cu_prefix[-1] == tot and inp.cu_prefix.dtype == np.int32
    c1 = workloads.make_inputs(workloads.get("c1"), 0)
    assert c1.layers[0]["q"].dtype == torch.float32


def test_bf16_rounding_is_nearest_even():
    """Hand-picked float32 values and their bf16 roundings."""
    vals = torch.tensor([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9,
                         -(1.0 + 2 ** -7 + 2 ** -9)], dtype=torch.float32)
    want = [1.0, 1.0 + 2 ** -6, 1.0, -(1.0 + 2 ** -7)]
    assert vals.to(torch.bfloat16).float().tolist() == want


def test_planted_bias_moves_planted_keys_along_mean_query_direction():
    cfg = workloads.scaled(workloads.get("c2"), batch=2, prefix_fixed=4,
                           dtype="f32")
    meta = workloads.draw_metadata(cfg, 3)
    biased = gen.make_layer(cfg, meta, 3, 1, planted=True)
    plain = gen.make_layer(cfg, meta, 3, 1, planted=False)
    assert torch.equal(biased["q"], plain["q"])
    diff = (biased["k_blk"] - plain["k_blk"]).view(2, 32, 8, 128)
    q = plain["q"].view(2, 32, 8, 4, 128).mean(dim=(1, 3))
    u_hat = q / q.norm(dim=-1, keepdim=True)
    for b in range(2):
        for j in range(32):
            if meta.planted[b, j]:
                torch.testing.assert_close(diff[b, j], 0.5 * u_hat[b],
                                           atol=1e-6, rtol=1e-5)
            else:
                assert (diff[b, j] == 0).all()


def test_masked_flags_are_seeded_and_left_biased():
    cfg = workloads.get("c3")
    a = workloads.draw_masked(cfg, 0)
    b = workloads.draw_masked(cfg, 0)
    c = workloads.draw_masked(cfg, 1)
    assert a.shape == (cfg.batch, cfg.block) and a.dtype == np.uint8
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert set(np.unique(a).tolist()) <= {0, 1}
    # earlier positions are decoded (0) more often than later ones
    assert a[:, :8].mean() < a[:, -8:].mean()
