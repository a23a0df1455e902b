"""Pins of the float64 oracle to things other than itself (CPU only).

Each test names what fixes the expected value: a hand-worked example under
tests/golden/, a closed form, an invariant of the definitions, a library
routine (torch float64) on small inputs, or brute force on tiny inputs.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests import golden_io

RNG = np.random.default_rng(1234)


def _rand_case(n, blk, hq, hkv, d, plens, rng, q_scale=1.0):
    cu = np.concatenate([[0], np.cumsum(plens)]).astype(np.int64)
    return dict(
        q=rng.standard_normal((n * blk, hq, d)) * q_scale,
        k_blk=rng.standard_normal((n * blk, hkv, d)),
        v_blk=rng.standard_normal((n * blk, hkv, d)),
        k_cache=rng.standard_normal((cu[-1], hkv, d)),
        v_cache=rng.standard_normal((cu[-1], hkv, d)),
        cu_prefix=cu)


def _s1(c, blk, hq, hkv, **kw):
    return oracle.block_attn_importance(
        c["q"], c["k_blk"], c["v_blk"], c["k_cache"], c["v_cache"],
        c["cu_prefix"], blk, hq, hkv, **kw)


# ---------------------------------------------------------------- golden


@pytest.mark.parametrize("name", ["importance_gqa_tiny.json", "scale_d4.json"])
def test_golden_block_attention_importance(name):
    g = golden_io.load(name)
    a = {k: golden_io.arr(g[k]) for k in
         ("q", "k_blk", "v_blk", "k_cache", "v_cache")}
    out, imp, lse, full = oracle.block_attn_importance(
        a["q"], a["k_blk"], a["v_blk"], a["k_cache"], a["v_cache"],
        g["cu_prefix"], g["block"], g["hq"], g["hkv"], full_columns=True)
    np.testing.assert_allclose(out, golden_io.arr(g["expect_out"]), atol=1e-14)
    np.testing.assert_allclose(imp, golden_io.arr(g["expect_imp"]), atol=1e-14)
    np.testing.assert_allclose(lse, golden_io.arr(g["expect_lse"]), atol=1e-14)
    if "expect_full_columns_head0" in g:
        np.testing.assert_allclose(
            full[0][0], golden_io.arr(g["expect_full_columns_head0"]),
            atol=1e-14)


def _golden_block_step_layers(g):
    """The layer dicts of tests/golden/block_step_tiny.json (d = 1)."""
    n = len(g["cu_prefix"]) - 1
    rows = n * g["block"]
    qh = golden_io.arr(g["q_heads"])
    q = np.broadcast_to(qh[None, :, None], (rows, g["hq"], 1)).copy()

    def lay(name):
        L = g["layers"][name]
        d = {k: golden_io.arr(L[k]).reshape(-1, g["hkv"], 1)
             for k in ("k_blk", "v_blk", "k_cache", "v_cache")}
        d["q"] = q
        return d
    return [lay(name) for name in ("l0", "l1", "fA", "fB")]


def test_golden_block_step():
    """The whole step, worked by hand (layer order of the delta, budgets,
    compaction, and which layer each further retained attention reads)."""
    g = golden_io.load("block_step_tiny.json")
    blk, hq = g["block"], g["hq"]
    l0, l1, fa, fb = _golden_block_step_layers(g)
    res = oracle.block_step(l0, l1, g["cu_prefix"], g["k_keep"], blk, hq,
                            g["hkv"], g["pool_k"], further_layers=[fa, fb])
    e = g["expect"]
    for name in ("out_l0", "out_l1"):
        per_seq = golden_io.arr(e[name])                  # [N, Hq]
        want = np.repeat(per_seq, blk, axis=0)[:, :, None]
        np.testing.assert_allclose(res[name], want, atol=1e-13)
    for name in ("lse_l0", "lse_l1"):
        want = np.repeat(golden_io.arr(e[name])[:, :, None], blk, axis=2)
        np.testing.assert_allclose(res[name], want, atol=1e-13)
    for name in ("imp_l0", "imp_l1", "dI"):
        np.testing.assert_allclose(res[name], golden_io.arr(e[name]), atol=1e-13)
    np.testing.assert_array_equal(res["keep"], np.array(e["keep"]))
    np.testing.assert_array_equal(res["idx"], e["idx"])
    np.testing.assert_array_equal(res["cu_ret"], e["cu_ret"])
    assert len(res["retained_out"]) == 2
    for got, want in zip(res["retained_out"], e["retained_out"]):
        np.testing.assert_allclose(got, golden_io.arr(want)[:, :, None], atol=1e-12)


def test_golden_delta_topk_compact():
    g = golden_io.load("delta_topk_compact.json")
    imp0, imp1 = golden_io.arr(g["imp0"]), golden_io.arr(g["imp1"])
    k = g["pool_k"]
    p0 = oracle.head_mean_maxpool(imp0, k)
    p1 = oracle.head_mean_maxpool(imp1, k)
    np.testing.assert_array_equal(p0, golden_io.arr(g["expect_pooled0"]))
    np.testing.assert_array_equal(p1, golden_io.arr(g["expect_pooled1"]))
    dI = oracle.importance_delta(imp0, imp1, k)
    np.testing.assert_array_equal(dI, golden_io.arr(g["expect_dI"]))
    keep = oracle.topk_keep(dI, g["k_keep"])
    np.testing.assert_array_equal(keep, np.array(g["expect_keep"]))
    idx, cu = oracle.compact(keep)
    np.testing.assert_array_equal(idx, g["expect_idx"])
    np.testing.assert_array_equal(cu, g["expect_cu_ret"])
    c = g["compact_only"]
    idx, cu = oracle.compact(np.array(c["keep"], dtype=np.uint8))
    np.testing.assert_array_equal(idx, c["expect_idx"])
    np.testing.assert_array_equal(cu, c["expect_cu_ret"])


def test_golden_retained():
    base = golden_io.load("importance_gqa_tiny.json")
    a = {k: golden_io.arr(base[k]) for k in
         ("q", "k_blk", "v_blk", "k_cache", "v_cache")}
    for case in golden_io.load("retained_tiny.json")["cases"]:
        out = oracle.retained_attn(
            a["q"], a["k_blk"], a["v_blk"], case["idx"], case["cu_ret"],
            a["k_cache"], a["v_cache"], base["cu_prefix"], base["block"],
            base["hq"], base["hkv"])
        np.testing.assert_allclose(out, golden_io.arr(case["expect_out"]),
                                   atol=1e-14)


# ------------------------------------------------------- invariants, closed


@pytest.mark.parametrize("blk,hq,hkv,d,plens", [
    (32, 4, 1, 64, [64]), (7, 4, 2, 16, [0, 5, 13]), (1, 2, 1, 8, [3, 0]),
    (16, 8, 2, 32, [31, 1, 0, 40])])
def test_column_sums_equal_block_size(blk, hq, hkv, d, plens):
    """Rows of a softmax sum to 1, so summing the block queries' weights
    over every key (prefix and block) gives B for every head."""
    c = _rand_case(len(plens), blk, hq, hkv, d, plens, RNG, q_scale=2.0)
    _, imp, _, full = _s1(c, blk, hq, hkv, full_columns=True)
    for b, cols in enumerate(full):
        np.testing.assert_allclose(cols.sum(axis=1), blk, rtol=1e-12)
        np.testing.assert_allclose(cols[:, plens[b]:], imp[b], atol=0)
        if plens[b] == 0:
            np.testing.assert_allclose(imp[b].sum(axis=1), blk, rtol=1e-12)
    assert (imp > 0).all()


def test_zero_queries_closed_form():
    """Q = 0 makes every score 0: uniform weights 1/(P+B), so
    I_j = B/(P+B), O = mean of the value rows, lse = ln(P+B)."""
    blk, hq, hkv, d, plens = 8, 4, 2, 16, [0, 3, 10]
    c = _rand_case(3, blk, hq, hkv, d, plens, RNG)
    c["q"][:] = 0
    out, imp, lse = _s1(c, blk, hq, hkv)
    grp = hq // hkv
    for b, plen in enumerate(plens):
        np.testing.assert_allclose(imp[b], blk / (plen + blk), rtol=1e-13)
        np.testing.assert_allclose(lse[b], math.log(plen + blk), rtol=1e-13)
        p0 = int(c["cu_prefix"][b])
        for h in range(hq):
            vals = np.concatenate([c["v_cache"][p0:p0 + plen, h // grp],
                                   c["v_blk"][b * blk:(b + 1) * blk, h // grp]])
            np.testing.assert_allclose(
                out[b * blk:(b + 1) * blk, h],
                np.broadcast_to(vals.mean(axis=0), (blk, d)), atol=1e-13)


def test_dominant_key_takes_all_weight():
    """A block key far along a direction every query shares takes almost
    all of each row's weight: its importance tends to B, others to 0."""
    blk, hq, hkv, d = 6, 2, 1, 8
    c = _rand_case(1, blk, hq, hkv, d, [5], RNG, q_scale=0.01)
    u = np.ones(d) / math.sqrt(d)
    c["q"] += u
    c["k_blk"][3, 0] = 400.0 * u
    _, imp, _ = _s1(c, blk, hq, hkv)
    np.testing.assert_allclose(imp[0, :, 3], blk, rtol=1e-9)
    assert imp[0, :, [0, 1, 2, 4, 5]].max() < 1e-9


@pytest.mark.parametrize("blk,hq,hkv,d,plens", [
    (32, 4, 1, 64, [64]), (5, 8, 2, 32, [0, 7, 19]), (3, 4, 4, 16, [2, 2])])
def test_attention_matches_torch_sdpa(blk, hq, hkv, d, plens):
    """O against torch float64 scaled_dot_product_attention (GQA by
    repeating each KV head over its query-head group); lse against torch
    logsumexp of the scaled scores."""
    c = _rand_case(len(plens), blk, hq, hkv, d, plens, RNG, q_scale=1.5)
    out, _, lse = _s1(c, blk, hq, hkv)
    grp = hq // hkv
    for b, plen in enumerate(plens):
        p0 = int(c["cu_prefix"][b])
        rows = slice(b * blk, (b + 1) * blk)
        keys = np.concatenate([c["k_cache"][p0:p0 + plen], c["k_blk"][rows]])
        vals = np.concatenate([c["v_cache"][p0:p0 + plen], c["v_blk"][rows]])
        qt = torch.from_numpy(c["q"][rows]).permute(1, 0, 2)       # [Hq,B,d]
        kt = torch.from_numpy(keys).permute(1, 0, 2).repeat_interleave(grp, 0)
        vt = torch.from_numpy(vals).permute(1, 0, 2).repeat_interleave(grp, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)
        np.testing.assert_allclose(out[rows], ref.permute(1, 0, 2).numpy(),
                                   atol=1e-12)
        s = torch.matmul(qt, kt.transpose(1, 2)) / math.sqrt(d)
        np.testing.assert_allclose(lse[b], torch.logsumexp(s, -1).numpy(),
                                   atol=1e-12)


def test_importance_brute_force_loops():
    """Pure-Python loops with math.exp on a tiny case."""
    blk, hq, hkv, d, plens = 3, 2, 1, 2, [2]
    c = _rand_case(1, blk, hq, hkv, d, plens, RNG)
    _, imp, _ = _s1(c, blk, hq, hkv)
    keys = [list(c["k_cache"][t, 0]) for t in range(2)] + \
        [list(c["k_blk"][j, 0]) for j in range(blk)]
    for h in range(hq):
        for j in range(blk):
            tot = 0.0
            for i in range(blk):
                qi = c["q"][i, h]
                sc = [sum(qi[e] * kk[e] for e in range(d)) / math.sqrt(d)
                      for kk in keys]
                z = sum(math.exp(x) for x in sc)
                tot += math.exp(sc[2 + j]) / z
            assert abs(tot - imp[0, h, j]) < 1e-12


def test_permutations():
    """Reordering prefix tokens changes nothing; reordering block tokens
    (queries, keys and values together) permutes O rows, I and lse."""
    blk, hq, hkv, d, plens = 6, 4, 2, 16, [9]
    c = _rand_case(1, blk, hq, hkv, d, plens, RNG)
    out, imp, lse = _s1(c, blk, hq, hkv)
    pp = RNG.permutation(9)
    c2 = dict(c, k_cache=c["k_cache"][pp], v_cache=c["v_cache"][pp])
    o2, i2, l2 = _s1(c2, blk, hq, hkv)
    np.testing.assert_allclose(o2, out, atol=1e-13)
    np.testing.assert_allclose(i2, imp, atol=1e-13)
    np.testing.assert_allclose(l2, lse, atol=1e-13)
    bp = RNG.permutation(blk)
    c3 = dict(c, q=c["q"][bp], k_blk=c["k_blk"][bp], v_blk=c["v_blk"][bp])
    o3, i3, l3 = _s1(c3, blk, hq, hkv)
    np.testing.assert_allclose(o3, out[bp], atol=1e-13)
    np.testing.assert_allclose(i3[0], imp[0][:, bp], atol=1e-13)
    np.testing.assert_allclose(l3[0], lse[0][:, bp], atol=1e-13)


# ------------------------------------------------------------- S2 .. S5


@pytest.mark.parametrize("k", [1, 3, 5, 7])
def test_maxpool_matches_torch(k):
    """Head mean then torch float64 max_pool1d (stride 1, padding (k-1)/2,
    which pads with -inf); signed inputs so zero padding would differ."""
    imp = RNG.standard_normal((5, 4, 11))
    got = oracle.head_mean_maxpool(imp, k)
    mean = torch.from_numpy(imp).mean(dim=1, keepdim=True)
    ref = torch.nn.functional.max_pool1d(mean, k, 1, (k - 1) // 2)[:, 0]
    np.testing.assert_array_equal(got, ref.numpy())
    if k == 1:
        np.testing.assert_array_equal(got, imp.mean(axis=1))


@pytest.mark.parametrize("blk,k", [(1, 3), (2, 3), (2, 5), (4, 9), (5, 7), (3, 255)])
def test_maxpool_window_wider_than_block(blk, k):
    """A window wider than the block is cut at the block edges (-inf
    padding): torch float64 max_pool1d with padding (k-1)/2 gives the same,
    and from k >= 2B-1 on every position holds the block's maximum."""
    imp = RNG.standard_normal((6, 3, blk))
    got = oracle.head_mean_maxpool(imp, k)
    mean = torch.from_numpy(imp).mean(dim=1, keepdim=True)
    ref = torch.nn.functional.max_pool1d(mean, k, 1, (k - 1) // 2)[:, 0]
    np.testing.assert_array_equal(got, ref.numpy())
    if k >= 2 * blk - 1:
        np.testing.assert_array_equal(
            got, np.repeat(imp.mean(axis=1).max(axis=1, keepdims=True), blk, axis=1))


def test_delta_of_identical_layers_is_zero_and_keeps_first_positions():
    imp = RNG.random((3, 4, 10))
    dI = oracle.importance_delta(imp, imp.copy(), 3)
    assert (dI == 0).all()
    keep = oracle.topk_keep(dI, [0, 4, 10])
    np.testing.assert_array_equal(keep.sum(axis=1), [0, 4, 10])
    np.testing.assert_array_equal(keep[1], [1] * 4 + [0] * 6)


def test_topk_matches_torch_and_invariants():
    dI = RNG.standard_normal((16, 32))           # distinct with prob. 1
    kk = RNG.integers(-2, 40, size=16)
    keep = oracle.topk_keep(dI, kk)
    for b in range(16):
        kb = min(max(int(kk[b]), 0), 32)
        assert keep[b].sum() == kb
        if 0 < kb:
            ref = torch.topk(torch.from_numpy(dI[b]), kb).indices.numpy()
            assert set(ref.tolist()) == set(np.nonzero(keep[b])[0].tolist())
        if 0 < kb < 32:
            assert dI[b][keep[b] == 1].min() > dI[b][keep[b] == 0].max()


def test_compact_matches_nonzero_and_cumsum():
    keep = (RNG.random((9, 13)) < 0.3).astype(np.uint8)
    keep[4] = 0
    idx, cu = oracle.compact(keep)
    np.testing.assert_array_equal(idx, np.flatnonzero(keep.reshape(-1)))
    np.testing.assert_array_equal(cu[1:], np.cumsum(keep.sum(axis=1)))
    assert cu[0] == 0


def test_retained_with_full_budget_equals_block_attention():
    blk, hq, hkv, d, plens = 8, 4, 2, 16, [5, 0, 12]
    c = _rand_case(3, blk, hq, hkv, d, plens, RNG)
    out, _, _ = _s1(c, blk, hq, hkv)
    keep = np.ones((3, blk), dtype=np.uint8)
    idx, cu = oracle.compact(keep)
    ret = oracle.retained_attn(c["q"], c["k_blk"], c["v_blk"], idx, cu,
                               c["k_cache"], c["v_cache"], c["cu_prefix"],
                               blk, hq, hkv)
    np.testing.assert_allclose(ret, out, atol=1e-13)


def test_retained_matches_torch_sdpa_on_gathered_rows():
    blk, hq, hkv, d, plens = 10, 4, 1, 8, [4, 7]
    c = _rand_case(2, blk, hq, hkv, d, plens, RNG)
    keep = np.zeros((2, blk), dtype=np.uint8)
    keep[0, [1, 5, 9]] = 1
    keep[1, [0]] = 1
    idx, cu = oracle.compact(keep)
    ret = oracle.retained_attn(c["q"], c["k_blk"], c["v_blk"], idx, cu,
                               c["k_cache"], c["v_cache"], c["cu_prefix"],
                               blk, hq, hkv)
    for b in range(2):
        rows = idx[cu[b]:cu[b + 1]]
        p0, p1 = int(c["cu_prefix"][b]), int(c["cu_prefix"][b + 1])
        keys = np.concatenate([c["k_cache"][p0:p1], c["k_blk"][rows]])
        vals = np.concatenate([c["v_cache"][p0:p1], c["v_blk"][rows]])
        qt = torch.from_numpy(c["q"][rows]).permute(1, 0, 2)
        kt = torch.from_numpy(keys).permute(1, 0, 2).repeat_interleave(hq, 0)
        vt = torch.from_numpy(vals).permute(1, 0, 2).repeat_interleave(hq, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)
        np.testing.assert_allclose(ret[cu[b]:cu[b + 1]],
                                   ref.permute(1, 0, 2).numpy(), atol=1e-12)


def test_block_step_budget_and_order():
    blk, hq, hkv, d, plens = 12, 4, 2, 16, [3, 9, 0]
    l0 = _rand_case(3, blk, hq, hkv, d, plens, RNG)
    l1 = _rand_case(3, blk, hq, hkv, d, plens, RNG)
    l2 = _rand_case(3, blk, hq, hkv, d, plens, RNG)
    res = oracle.block_step(l0, l1, l0["cu_prefix"], [4, 0, 12], blk, hq,
                            hkv, 3, further_layers=[l2])
    np.testing.assert_array_equal(np.diff(res["cu_ret"]), [4, 0, 12])
    assert (np.diff(res["idx"][:4]) > 0).all()
    assert res["retained_out"][0].shape == (16, hq, d)
