"""Property tests of the float64 oracle on shapes hypothesis draws (CPU).

Each property is fixed by something other than the oracle: torch float64
routines (scaled_dot_product_attention with the GQA heads repeated,
logsumexp, max_pool1d, topk), the softmax invariant (a row's weights sum to
1, so a head's importance over every key sums to B), and a re-selection of
the kept rows by plain NumPy indexing.
"""
import math

import numpy as np
import torch
from hypothesis import given, settings, strategies as st

import oracle

SETTINGS = settings(max_examples=25, deadline=None, derandomize=True)


@st.composite
def attn_case(draw):
    blk = draw(st.integers(1, 9))
    hkv = draw(st.integers(1, 3))
    grp = draw(st.sampled_from([1, 2, 4]))
    d = draw(st.sampled_from([2, 4, 8, 16]))
    plens = draw(st.lists(st.integers(0, 40), min_size=1, max_size=3))
    seed = draw(st.integers(0, 2**31 - 1))
    scale = draw(st.sampled_from([0.3, 1.0, 3.0]))
    rng = np.random.default_rng(seed)
    n, hq = len(plens), hkv * grp
    cu = np.concatenate([[0], np.cumsum(plens)]).astype(np.int64)
    c = dict(q=rng.standard_normal((n * blk, hq, d)) * scale,
             k_blk=rng.standard_normal((n * blk, hkv, d)),
             v_blk=rng.standard_normal((n * blk, hkv, d)),
             k_cache=rng.standard_normal((cu[-1], hkv, d)),
             v_cache=rng.standard_normal((cu[-1], hkv, d)), cu_prefix=cu)
    return c, blk, hq, hkv, d, plens


@SETTINGS
@given(attn_case())
def test_block_attention_against_torch_and_column_sums(case):
    c, blk, hq, hkv, d, plens = case
    out, imp, lse, full = oracle.block_attn_importance(
        c["q"], c["k_blk"], c["v_blk"], c["k_cache"], c["v_cache"], c["cu_prefix"],
        blk, hq, hkv, full_columns=True)
    grp = hq // hkv
    for b, plen in enumerate(plens):
        p0 = int(c["cu_prefix"][b])
        rows = slice(b * blk, (b + 1) * blk)
        keys = np.concatenate([c["k_cache"][p0:p0 + plen], c["k_blk"][rows]])
        vals = np.concatenate([c["v_cache"][p0:p0 + plen], c["v_blk"][rows]])
        qt = torch.from_numpy(c["q"][rows]).permute(1, 0, 2)
        kt = torch.from_numpy(keys).permute(1, 0, 2).repeat_interleave(grp, 0)
        vt = torch.from_numpy(vals).permute(1, 0, 2).repeat_interleave(grp, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)
        np.testing.assert_allclose(out[rows], ref.permute(1, 0, 2).numpy(), atol=1e-11)
        s = torch.matmul(qt, kt.transpose(1, 2)) / math.sqrt(d)
        np.testing.assert_allclose(lse[b], torch.logsumexp(s, -1).numpy(), atol=1e-11)
        # softmax weights of each row sum to 1: over all keys a head's
        # column sums add up to B; the block columns are the importance
        np.testing.assert_allclose(full[b].sum(axis=1), blk, rtol=1e-11)
        np.testing.assert_array_equal(full[b][:, plen:], imp[b])
        w = torch.softmax(s, -1).sum(dim=1).numpy()          # [Hq, P + B]
        np.testing.assert_allclose(imp[b], w[:, plen:], atol=1e-11)


@SETTINGS
@given(st.integers(1, 4), st.integers(1, 6), st.integers(1, 40),
       st.sampled_from([1, 3, 5, 7, 9]), st.integers(0, 2**31 - 1))
def test_maxpool_delta_topk_compact(n, hq, blk, k, seed):
    rng = np.random.default_rng(seed)
    imp0, imp1 = rng.standard_normal((2, n, hq, blk))
    mp = torch.nn.functional.max_pool1d
    pooled = [mp(torch.from_numpy(x).mean(dim=1, keepdim=True), k, 1, (k - 1) // 2)[:, 0]
              for x in (imp0, imp1)]
    # the head mean may round differently (summation order) by an ulp
    np.testing.assert_allclose(oracle.head_mean_maxpool(imp1, k), pooled[1].numpy(),
                               rtol=0, atol=1e-14)
    dI = oracle.importance_delta(imp0, imp1, k)
    np.testing.assert_allclose(dI, (pooled[1] - pooled[0]).numpy(), rtol=0, atol=1e-14)
    kk = rng.integers(-1, blk + 2, size=n)
    keep = oracle.topk_keep(dI, kk)
    for b in range(n):
        kb = min(max(int(kk[b]), 0), blk)
        # stable order of (-delta, position): the first kb positions
        want = np.zeros(blk, dtype=keep.dtype)
        want[np.argsort(-dI[b], kind="stable")[:kb]] = 1
        np.testing.assert_array_equal(keep[b], want)
        if 0 < kb:
            ref = torch.topk(torch.from_numpy(dI[b]), kb).values.numpy()
            np.testing.assert_array_equal(np.sort(dI[b][keep[b] == 1]), np.sort(ref))
    idx, cu = oracle.compact(keep)
    np.testing.assert_array_equal(idx, np.flatnonzero(keep.reshape(-1)))
    np.testing.assert_array_equal(np.diff(cu), keep.sum(axis=1))


@SETTINGS
@given(attn_case(), st.integers(0, 2**31 - 1))
def test_retained_equals_attention_over_the_kept_rows(case, seed):
    """Retained attention over a random kept set equals SDPA of the kept
    queries over the prefix keys plus the kept block keys only."""
    c, blk, hq, hkv, d, plens = case
    rng = np.random.default_rng(seed)
    keep = (rng.random((len(plens), blk)) < 0.5).astype(np.uint8)
    idx, cu_ret = oracle.compact(keep)
    ret = oracle.retained_attn(c["q"], c["k_blk"], c["v_blk"], idx, cu_ret,
                               c["k_cache"], c["v_cache"], c["cu_prefix"], blk, hq, hkv)
    grp = hq // hkv
    for b, plen in enumerate(plens):
        rows = idx[cu_ret[b]:cu_ret[b + 1]]
        if rows.size == 0:
            continue
        p0 = int(c["cu_prefix"][b])
        keys = np.concatenate([c["k_cache"][p0:p0 + plen], c["k_blk"][rows]])
        vals = np.concatenate([c["v_cache"][p0:p0 + plen], c["v_blk"][rows]])
        qt = torch.from_numpy(c["q"][rows]).permute(1, 0, 2)
        kt = torch.from_numpy(keys).permute(1, 0, 2).repeat_interleave(grp, 0)
        vt = torch.from_numpy(vals).permute(1, 0, 2).repeat_interleave(grp, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)
        np.testing.assert_allclose(ret[cu_ret[b]:cu_ret[b + 1]],
                                   ref.permute(1, 0, 2).numpy(), atol=1e-11)
