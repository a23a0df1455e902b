"""Mistakes planted in a copy of the oracle must be caught by its pins.

Each mutant is a small textual edit of oracle/focus_oracle.py (a dropped
term, a wrong axis, sign, index or offset). The edited source is executed
into a fresh module on the CPU, swapped in for the oracle's functions, and
at least one pin of tests/test_oracle_pins.py must then fail. The real
oracle is never modified.
"""
import inspect
import types

import pytest

import oracle
from oracle import focus_oracle
from tests import test_oracle_constrained as PC
from tests import test_oracle_pins as P

PINS = [
    lambda: P.test_golden_block_attention_importance("importance_gqa_tiny.json"),
    lambda: P.test_golden_block_attention_importance("scale_d4.json"),
    P.test_golden_delta_topk_compact,
    P.test_golden_retained,
    P.test_golden_block_step,
    lambda: P.test_column_sums_equal_block_size(7, 4, 2, 16, [0, 5, 13]),
    P.test_zero_queries_closed_form,
    P.test_dominant_key_takes_all_weight,
    lambda: P.test_attention_matches_torch_sdpa(5, 8, 2, 32, [0, 7, 19]),
    P.test_importance_brute_force_loops,
    P.test_permutations,
    lambda: P.test_maxpool_matches_torch(3),
    P.test_delta_of_identical_layers_is_zero_and_keeps_first_positions,
    P.test_topk_matches_torch_and_invariants,
    P.test_compact_matches_nonzero_and_cumsum,
    P.test_retained_with_full_budget_equals_block_attention,
    P.test_retained_matches_torch_sdpa_on_gathered_rows,
    *[(lambda c=c: PC.test_golden_constrained(c)) for c in PC._cases()],
    PC.test_golden_constrained_batched_compaction,
    *[(lambda s=s: PC.test_constrained_matches_characterisation(s)) for s in range(6)],
    PC.test_all_masked_without_constraints_is_plain_topk,
    PC.test_all_masked_with_prefix_rule_keeps_a_contiguous_head,
    PC.test_nothing_masked_retains_nothing,
    *[(lambda c=c: PC.test_golden_dynamic_budget(c)) for c in PC._budget_cases()["cases"]],
]

# (name, [(old, new, occurrence)])
MUTANTS = [
    ("scale dropped", [("return 1.0 / math.sqrt(d)", "return 1.0", 0)]),
    ("scale 1/d", [("return 1.0 / math.sqrt(d)", "return 1.0 / d", 0)]),
    ("softmax over queries", [
        ("m = s.max(axis=1, keepdims=True)", "m = s.max(axis=0, keepdims=True)", 0),
        ("l = e.sum(axis=1, keepdims=True)", "l = e.sum(axis=0, keepdims=True)", 0)]),
    ("lse without max", [("lse = m[:, 0] + np.log(l[:, 0])",
                          "lse = np.log(l[:, 0])", 0)]),
    ("values replaced by keys", [("return p, p @ v, lse", "return p, p @ k, lse", 0)]),
    ("GQA map h % Hkv in S1", [("g = h // grp", "g = h % hkv", 0)]),
    ("GQA map h % Hkv in S5", [("g = h // grp", "g = h % hkv", 1)]),
    ("prefix columns taken as block", [("imp[b, h] = colsum[plen:]",
                                        "imp[b, h] = colsum[:block]", 0)]),
    ("prefix offset ignored in S1", [("p0, p1 = int(cu[b]), int(cu[b + 1])",
                                      "p0, p1 = 0, int(cu[b + 1]) - int(cu[b])", 0)]),
    ("heads summed", [("mean = np.asarray(imp, dtype=F64).mean(axis=1)",
                       "mean = np.asarray(imp, dtype=F64).sum(axis=1)", 0)]),
    ("pool radius k-1", [("r = (pool_k - 1) // 2", "r = pool_k - 1", 0)]),
    ("pool window short on the right", [
        ("lo, hi = max(0, j - r), min(blk, j + r + 1)",
         "lo, hi = max(0, j - r), min(blk, j + r)", 0)]),
    ("delta sign", [(
        "return head_mean_maxpool(imp1, pool_k) - head_mean_maxpool(imp0, pool_k)",
        "return head_mean_maxpool(imp0, pool_k) - head_mean_maxpool(imp1, pool_k)", 0)]),
    ("ties to higher index", [("key=lambda j: (-d_imp[b, j], j)",
                               "key=lambda j: (-d_imp[b, j], -j)", 0)]),
    ("smallest kept", [("key=lambda j: (-d_imp[b, j], j)",
                        "key=lambda j: (d_imp[b, j], j)", 0)]),
    ("budget off by one", [("kb = min(max(int(k_keep[b]), 0), blk)",
                            "kb = min(max(int(k_keep[b]) - 1, 0), blk)", 0)]),
    ("idx without sequence offset", [("idx.append(b * blk + j)", "idx.append(j)", 0)]),
    ("cu_ret inclusive", [("cu = [0]", "cu = []", 0)]),
    ("retained sees every block key", [
        ("np.asarray(k_src[rows, g], F64)",
         "np.asarray(k_src[b * block:(b + 1) * block, g], F64)", 0),
        ("np.asarray(v_src[rows, g], F64)",
         "np.asarray(v_src[b * block:(b + 1) * block, g], F64)", 0)]),
    ("retained prefix from token 0", [("p0, p1 = int(cu_p[b]), int(cu_p[b + 1])",
                                       "p0, p1 = 0, int(cu_p[b + 1])", 0)]),
    ("constrained: mask ignored", [(
        "eligible = [j for j in range(blk) if masked[b, j]]",
        "eligible = list(range(blk))", 0)]),
    ("constrained: successor kept", [("keep[b, j - 1] = 1",
                                      "keep[b, min(j + 1, blk - 1)] = 1", 0)]),
    ("constrained: decoded positions in the prefix rule", [
        ("                if masked[b, j]:", "                if True:", 0)]),
    ("constrained: leftmost candidate", [("rightmost = max(chosen)",
                                          "rightmost = min(chosen)", 0)]),
    ("constrained: prefix rule to the block end", [("for j in range(rightmost):",
                                                    "for j in range(blk):", 0)]),
    ("constrained: ties to higher index", [("key=lambda j: (-d_imp[b, j], j)",
                                            "key=lambda j: (-d_imp[b, j], -j)", 1)]),
    ("constrained: smallest deltas", [("key=lambda j: (-d_imp[b, j], j)",
                                       "key=lambda j: (d_imp[b, j], j)", 1)]),
    ("budget: sample std", [("sum((v - mu) ** 2 for v in vals) / len(vals)",
                             "sum((v - mu) ** 2 for v in vals) / max(len(vals) - 1, 1)", 0)]),
    ("budget: threshold inclusive", [("if v > mu + sigma", "if v >= mu + sigma", 0)]),
    ("budget: floor", [("want = math.ceil(", "want = math.floor(", 0)]),
    ("budget: yield plus count", [("max(float(yield_hist[b]), float(above))",
                                   "(float(yield_hist[b]) + float(above))", 0)]),
    ("budget: decoded positions counted", [(
        "vals = [float(d_imp[b, j]) for j in range(blk) if m[b, j]]",
        "vals = [float(d_imp[b, j]) for j in range(blk)]", 0)]),
    ("budget: no floor of one", [("k[b] = min(len(vals), max(1, want))",
                                  "k[b] = min(len(vals), want)", 0)]),
    ("step: layers 0 and 1 swapped", [(
        'for name, lay in (("l0", layer0), ("l1", layer1)):',
        'for name, lay in (("l0", layer1), ("l1", layer0)):', 0)]),
    ("step: delta arguments swapped", [(
        'importance_delta(res["imp_l0"], res["imp_l1"], pool_k)',
        'importance_delta(res["imp_l1"], res["imp_l0"], pool_k)', 0)]),
    ("step: pool size ignored", [(
        'importance_delta(res["imp_l0"], res["imp_l1"], pool_k)',
        'importance_delta(res["imp_l0"], res["imp_l1"], 1)', 0)]),
    ("step: k_keep replaced by B", [(
        'res["keep"] = topk_keep(res["dI"], k_keep)',
        'res["keep"] = topk_keep(res["dI"], [block] * len(k_keep))', 0)]),
    ("step: further layer i reads layer i+1", [(
        "for lay in further_layers]",
        "for lay in list(further_layers[1:]) + list(further_layers[:1])]", 0)]),
    ("step: further layers read layer 1's block tensors", [(
        'retained_attn(lay["q"], lay["k_blk"], lay["v_blk"], res["idx"],',
        'retained_attn(lay["q"], layer1["k_blk"], layer1["v_blk"], res["idx"],', 0)]),
    ("step: further layers read layer 0's prefix cache", [(
        'res["cu_ret"], lay["k_cache"], lay["v_cache"],',
        'res["cu_ret"], layer0["k_cache"], layer0["v_cache"],', 0)]),
]

EXPORTED = ["attention_rows", "block_attn_importance", "block_step", "compact",
            "default_scale", "head_mean_maxpool", "importance_delta",
            "retained_attn", "select_constrained", "topk_keep", "dynamic_budget"]


def _replace_nth(src, old, new, n):
    pos = -1
    for _ in range(n + 1):
        pos = src.find(old, pos + 1)
        assert pos >= 0, f"mutation anchor not found: {old!r} #{n}"
    return src[:pos] + new + src[pos + len(old):]


def _mutant_module(edits):
    src = inspect.getsource(focus_oracle)
    for old, new, n in edits:
        src = _replace_nth(src, old, new, n)
    mod = types.ModuleType("focus_oracle_mutant")
    exec(compile(src, "<mutant>", "exec"), mod.__dict__)
    return mod


def test_unmutated_oracle_passes_every_pin():
    for pin in PINS:
        pin()


@pytest.mark.parametrize("name,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, edits, monkeypatch):
    mod = _mutant_module(edits)
    for fn in EXPORTED:
        monkeypatch.setattr(oracle, fn, getattr(mod, fn))
    caught = []
    for i, pin in enumerate(PINS):
        try:
            pin()
        except Exception as exc:  # a failed assertion or a shape error
            caught.append((i, type(exc).__name__))
    assert caught, f"no pin caught mutant {name!r}"
