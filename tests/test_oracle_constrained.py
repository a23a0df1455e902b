"""Pins of the oracle's constrained selection (masked-token eligibility and
the two structural constraints), against hand-worked examples and against a
set-based characterisation that is written independently of the oracle's
construction."""
import numpy as np
import pytest

import oracle
from tests import golden_io


def _cases():
    return golden_io.load("constrained_select.json")["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_golden_constrained(case):
    dI = golden_io.arr(case["dI"])[None, :]
    masked = np.array(case["masked"], dtype=np.uint8)[None, :]
    k = [case["k_keep"]]
    keep, cand = oracle.select_constrained(dI, masked, k)
    np.testing.assert_array_equal(cand[0], case["expect_cand"])
    np.testing.assert_array_equal(keep[0], case["expect_keep"])
    keep_p, cand_p = oracle.select_constrained(dI, masked, k, True, False)
    np.testing.assert_array_equal(keep_p[0], case["expect_keep_predecessor_only"])
    keep_m, _ = oracle.select_constrained(dI, masked, k, False, True)
    np.testing.assert_array_equal(keep_m[0], case["expect_keep_masked_prefix_only"])
    keep_0, cand_0 = oracle.select_constrained(dI, masked, k, False, False)
    np.testing.assert_array_equal(keep_0[0], case["expect_cand"])
    np.testing.assert_array_equal(cand_p, cand)


def test_golden_constrained_batched_compaction():
    g = golden_io.load("constrained_select.json")["batched"]
    keep, _ = oracle.select_constrained(golden_io.arr(g["dI"]),
                                        np.array(g["masked"]), g["k_keep"])
    np.testing.assert_array_equal(keep, g["expect_keep"])
    idx, cu = oracle.compact(keep)
    np.testing.assert_array_equal(idx, g["expect_idx"])
    np.testing.assert_array_equal(cu, g["expect_cu_ret"])


def _characterise(dI, masked, kb, pred, mprefix, keep, cand):
    """The result, stated as properties of sets: cand is a top-min(K, #M)
    subset of the masked positions M under the order (larger delta, then
    lower position); keep is the closure of cand under the chosen rules and
    nothing more."""
    blk = len(dI)
    M = {j for j in range(blk) if masked[j]}
    C = {j for j in range(blk) if cand[j]}
    R = {j for j in range(blk) if keep[j]}
    k = min(max(kb, 0), len(M))
    assert C <= M and len(C) == k
    for c in C:
        for e in M - C:
            assert (dI[c], -c) > (dI[e], -e), (c, e)
    need = set(C)
    if pred:
        need |= {c - 1 for c in C if c > 0}
    if mprefix and C:
        need |= {j for j in M if j < max(C)}
    assert R == need


@pytest.mark.parametrize("seed", range(40))
def test_constrained_matches_characterisation(seed):
    rng = np.random.default_rng(seed)
    blk = int(rng.integers(1, 40))
    n = 3
    # few distinct values so ties are common
    dI = rng.integers(-3, 4, size=(n, blk)) / 4.0
    masked = (rng.random((n, blk)) < rng.uniform(0.1, 1.0)).astype(np.uint8)
    k = rng.integers(-1, blk + 3, size=n)
    for pred in (False, True):
        for mp in (False, True):
            keep, cand = oracle.select_constrained(dI, masked, k, pred, mp)
            for b in range(n):
                _characterise(dI[b], masked[b], int(k[b]), pred, mp, keep[b], cand[b])


def test_all_masked_without_constraints_is_plain_topk():
    rng = np.random.default_rng(7)
    dI = rng.standard_normal((5, 32))
    k = [0, 1, 11, 32, 40]
    keep, cand = oracle.select_constrained(dI, np.ones((5, 32)), k, False, False)
    ref = oracle.topk_keep(dI, k)
    np.testing.assert_array_equal(keep, ref)
    np.testing.assert_array_equal(cand, ref)


def test_all_masked_with_prefix_rule_keeps_a_contiguous_head():
    """Every position masked: the masked-prefix rule makes the retained set
    exactly [0, rightmost candidate]."""
    rng = np.random.default_rng(3)
    dI = rng.standard_normal((6, 32))
    k = [1, 2, 5, 9, 20, 32]
    keep, cand = oracle.select_constrained(dI, np.ones((6, 32)), k)
    for b in range(6):
        r = int(np.flatnonzero(cand[b]).max())
        np.testing.assert_array_equal(keep[b], (np.arange(32) <= r).astype(np.uint8))


def test_nothing_masked_retains_nothing():
    keep, cand = oracle.select_constrained(np.ones((2, 8)), np.zeros((2, 8)), [3, 8])
    assert keep.sum() == 0 and cand.sum() == 0


# ------------------------------------------------------------ dynamic budget
def _budget_cases():
    return golden_io.load("dynamic_budget.json")


@pytest.mark.parametrize("case", _budget_cases()["cases"], ids=lambda c: c["name"])
def test_golden_dynamic_budget(case):
    alpha = float(golden_io.arr(_budget_cases()["alpha"]))
    k = oracle.dynamic_budget(golden_io.arr(case["dI"])[None, :],
                              np.array(case["masked"])[None, :],
                              [float(golden_io.arr(case["yield"]))], alpha)
    assert int(k[0]) == case["expect_k"]


def test_dynamic_budget_against_numpy_statistics():
    """The same reading through numpy's mean / std (ddof 0) on random
    inputs, and its bounds."""
    rng = np.random.default_rng(11)
    n, blk = 50, 32
    dI = rng.standard_normal((n, blk))
    masked = (rng.random((n, blk)) < 0.6).astype(np.uint8)
    y = rng.integers(0, 12, n) / 2.0
    k = oracle.dynamic_budget(dI, masked, y, 1.5)
    for b in range(n):
        v = dI[b][masked[b] == 1]
        if v.size == 0:
            assert k[b] == 0
            continue
        above = int((v > v.mean() + v.std()).sum())
        want = min(v.size, max(1, int(np.ceil(1.5 * max(y[b], above)))))
        assert k[b] == want
        assert 1 <= k[b] <= v.size


def test_dynamic_budget_grows_with_alpha_and_history():
    rng = np.random.default_rng(12)
    dI = rng.standard_normal((20, 32))
    masked = np.ones((20, 32), dtype=np.uint8)
    y = np.full(20, 3.0)
    k1 = oracle.dynamic_budget(dI, masked, y, 1.2)
    k2 = oracle.dynamic_budget(dI, masked, y, 1.8)
    k3 = oracle.dynamic_budget(dI, masked, y + 4, 1.8)
    assert (k1 <= k2).all() and (k2 <= k3).all() and (k3 > k1).any()
