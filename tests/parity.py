"""Helpers for comparing the HIP path with the float64 oracle.

Both sides read the same seeded tensors: the HIP path on the device, the
oracle after an exact widening to float32 (and float64 inside the oracle).
"""
from __future__ import annotations

import dataclasses
import sys
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

import oracle
import workloads
from workloads import to_f32_numpy

# Acceptance bars: the benchmark spec's tolerances, and tighter internal bars that
# the fp32-accumulating kernels are expected to meet.
TOL = {"bf16": dict(out=2e-2, imp=2e-2), "f32": dict(out=1e-5, imp=1e-5)}
# The bf16 output bar scales with max|O|: probabilities enter the PV MFMA
# as bf16 and O is stored as bf16, each a relative rounding of 2^-9, so the
# error of one element is bounded by about 2^-8 * sum_j p_j |v_j| + 2^-9 |O|
# (|v| <= ~4.5 for these inputs); 8e-3 * max(1, max|O|) is two bf16 ulps at
# magnitude 1, 2.5x inside the acceptance bar.
TIGHT = {"bf16": dict(out=8e-3, imp=1e-4, lse=1e-4, dI=1e-5),
         "f32": dict(out=1e-5, imp=1e-5, lse=1e-5, dI=1e-6)}
GAP = 1e-4  # K-th / (K+1)-th delta gap under which a selection is excused


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(inp: workloads.Inputs, device="cuda") -> List[Dict[str, torch.Tensor]]:
    return [{k: v.to(device) for k, v in lay.items()} for lay in inp.layers]


def dims_of(cfg: workloads.FocusConfig):
    from attention_delta_token_focus_amd.step import Dims
    return Dims(cfg.batch, cfg.block, cfg.hq, cfg.hkv, cfg.head_dim,
                workloads.torch_dtype(cfg), cfg.pool_k)


def run_gpu(inp: workloads.Inputs, layers_dev=None, n_further: Optional[int] = None,
            with_lse: bool = True, step=None, l1_output: bool = True):
    """Runs one block-step on the GPU; returns (step object, host results)."""
    from attention_delta_token_focus_amd.step import FocusStep
    cfg = inp.cfg
    if layers_dev is None:
        layers_dev = to_device(inp)
    if n_further is None:
        n_further = len(layers_dev) - 2
    if step is None:
        step = FocusStep(dims_of(cfg), inp.cu_prefix, inp.meta.k_keep,
                         n_further=n_further, with_lse=with_lse,
                         l1_output=l1_output)
    step.run(layers_dev)
    torch.cuda.synchronize()
    res = dict(
        out=[to_f32_numpy(o) if o is not None else None for o in step.out],
        imp=[i.cpu().numpy() for i in step.imp],
        lse=[l.cpu().numpy() if l is not None else None for l in step.lse],
        dI=step.dI.cpu().numpy(), keep=step.keep.cpu().numpy(),
        cand=step.cand.cpu().numpy() if step.cand is not None else None,
        k_used=step.k_used.cpu().numpy() if getattr(step, "k_used", None) is not None
        else None,
        idx=step.idx.cpu().numpy()[:step.n_ret],
        cu_ret=step.cu_ret.cpu().numpy(),
        ret=[to_f32_numpy(r)[:step.n_ret] for r in step.ret_out])
    return step, res


def sub_layers(layers, cu_prefix, block: int, seqs: Sequence[int]):
    """float32 numpy copies of the tensors of sequences `seqs`, repacked."""
    cu = np.asarray(cu_prefix, dtype=np.int64)
    out = []
    for lay in layers:
        d = {}
        for name in ("q", "k_blk", "v_blk"):
            d[name] = np.concatenate(
                [to_f32_numpy(lay[name][b * block:(b + 1) * block]) for b in seqs])
        for name in ("k_cache", "v_cache"):
            d[name] = np.concatenate(
                [to_f32_numpy(lay[name][int(cu[b]):int(cu[b + 1])]) for b in seqs])
        out.append(d)
    lens = np.array([cu[b + 1] - cu[b] for b in seqs])
    sub_cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return out, sub_cu


def rows_of(arr, seqs, block):
    return np.concatenate([arr[b * block:(b + 1) * block] for b in seqs])


@dataclasses.dataclass
class SelectionReport:
    exact: int = 0
    excused: int = 0
    failed: List[str] = dataclasses.field(default_factory=list)
    # max abs error per compared quantity (name -> error), for the record
    errors: Dict[str, float] = dataclasses.field(default_factory=dict)
    retained_seqs: int = 0    # sequences whose retained attention was compared


def check_selection(keep_gpu_b, dI_ref_b, k_b, label, rep: SelectionReport):
    """Bit-exact retained set, unless the oracle's K-th/(K+1)-th gap is
    below GAP; then every clearly-above token must be kept, none of the
    clearly-below ones, and exactly K in total."""
    blk = len(dI_ref_b)
    kb = min(max(int(k_b), 0), blk)
    order = sorted(range(blk), key=lambda j: (-dI_ref_b[j], j))
    ref = set(order[:kb])
    got = set(np.flatnonzero(keep_gpu_b).tolist())
    if got == ref:
        rep.exact += 1
        return
    ok = len(got) == kb and 0 < kb < blk
    if ok:
        top, nxt = dI_ref_b[order[kb - 1]], dI_ref_b[order[kb]]
        ok = top - nxt < GAP
        must = {j for j in range(blk) if dI_ref_b[j] >= top + GAP}
        never = {j for j in range(blk) if dI_ref_b[j] <= nxt - GAP}
        ok = ok and must <= got and not (never & got)
    if ok:
        rep.excused += 1
    else:
        rep.failed.append(f"{label}: gpu {sorted(got)} oracle {sorted(ref)}")


def assert_close(name, got, ref, tol, tight=None, rel_scale=False):
    if rel_scale and tight is not None and np.size(ref):
        tight = tight * max(1.0, float(np.max(np.abs(ref))))
    err = float(np.max(np.abs(np.asarray(got, np.float64) - ref))) if np.size(ref) else 0.0
    log(f"  {name}: max abs err {err:.3e} (bar {tol:.1e}"
        + (f", internal {tight:.1e})" if tight is not None else ")"))
    assert err <= tol, f"{name}: max abs err {err} > {tol}"
    if tight is not None:
        assert err <= tight, f"{name}: max abs err {err} > internal bar {tight}"
    return err


def compare_step(inp: workloads.Inputs, res, seqs: Sequence[int], layers_host=None,
                 further_check: bool = True, bar_scale: float = 1.0,
                 further_seqs: Optional[Sequence[int]] = None) -> SelectionReport:
    """Oracle block-step on sequences `seqs` against the GPU results.

    bar_scale multiplies the bars of lse, importance and delta: with scores
    far from O(1) their rounding error grows with the magnitude (one fp32
    ulp of an exponent argument s is |s| * 2^-23); O is a normalised mix
    and keeps its bars.

    further_seqs: the sequences (a subset of seqs) on which the retained
    attention of the further layers is compared; default all of seqs."""
    cfg = inp.cfg
    blk, kind = cfg.block, cfg.dtype
    tol = {k: v * (bar_scale if k != "out" else 1.0) for k, v in TOL[kind].items()}
    tight = {k: v * (bar_scale if k != "out" else 1.0) for k, v in TIGHT[kind].items()}
    seqs = list(seqs)
    layers = layers_host if layers_host is not None else inp.layers
    sub, sub_cu = sub_layers(layers[:2], inp.cu_prefix, blk, seqs)
    k_keep = inp.meta.k_keep[seqs]
    rep = SelectionReport()
    o = [oracle.block_attn_importance(sub[l]["q"], sub[l]["k_blk"], sub[l]["v_blk"],
                                      sub[l]["k_cache"], sub[l]["v_cache"], sub_cu,
                                      blk, cfg.hq, cfg.hkv) for l in (0, 1)]
    del sub
    for l in (0, 1):
        if res["out"][l] is not None:   # None: importance-only call
            rep.errors[f"out L{l}"] = assert_close(
                f"out L{l}", rows_of(res["out"][l], seqs, blk), o[l][0],
                tol["out"], tight["out"], rel_scale=True)
        rep.errors[f"imp L{l}"] = assert_close(
            f"imp L{l}", res["imp"][l][seqs], o[l][1], tol["imp"], tight["imp"])
        if res["lse"][l] is not None:
            rep.errors[f"lse L{l}"] = assert_close(
                f"lse L{l}", res["lse"][l][seqs], o[l][2], tight["lse"])
    dI_ref = oracle.importance_delta(o[0][1], o[1][1], cfg.pool_k)
    del o
    rep.errors["dI"] = assert_close("dI", res["dI"][seqs], dI_ref, tight["dI"])

    # The GPU's selection is a valid top-K of the GPU's own delta: every
    # kept position beats every evicted one, equal deltas by lower index.
    for b in seqs:
        d_b, k_b = res["dI"][b], res["keep"][b]
        kept, evicted = np.flatnonzero(k_b), np.flatnonzero(k_b == 0)
        for j in kept:
            bad = evicted[(d_b[evicted] > d_b[j]) |
                          ((d_b[evicted] == d_b[j]) & (evicted < j))]
            assert bad.size == 0, f"seq {b}: kept {j} loses to {bad.tolist()}"

    # Retained sets against the oracle's own selection.
    keep_ref = oracle.topk_keep(dI_ref, k_keep)
    idx_ref, cu_ref = oracle.compact(keep_ref)
    exact = []
    for i, b in enumerate(seqs):
        before = rep.exact
        check_selection(res["keep"][b], dI_ref[i], k_keep[i], f"seq {b}", rep)
        if rep.exact > before:
            exact.append(i)
    log(f"  selection: {rep.exact} exact, {rep.excused} excused (gap < {GAP}), "
        f"{len(rep.failed)} failed")
    assert not rep.failed, rep.failed[:5]

    # Compaction: offsets follow the budgets for the whole batch; the index
    # list of every exactly matched sequence equals the oracle's.
    kb_all = np.clip(inp.meta.k_keep, 0, blk)
    assert res["cu_ret"][0] == 0 and np.array_equal(np.diff(res["cu_ret"]), kb_all)
    g_cu = res["cu_ret"]
    for i in exact:
        b = seqs[i]
        mine = res["idx"][g_cu[b]:g_cu[b + 1]] - b * blk
        ref_j = idx_ref[cu_ref[i]:cu_ref[i + 1]] - i * blk
        assert np.array_equal(mine, ref_j), f"seq {b}: idx {mine} vs {ref_j}"

    # Retained attention, oracle on its own retained set; compared on the
    # sequences (of further_seqs) whose set matched exactly.
    if further_check and res["ret"]:
        pos = {b: i for i, b in enumerate(seqs)}
        fsel = [pos[b] for b in (seqs if further_seqs is None else further_seqs)]
        exact_set = set(exact)
        fex = [i for i in fsel if i in exact_set]
        fseqs = [seqs[i] for i in fex]
        rep.retained_seqs = len(fex)
        if fex:
            f_idx, f_cu = oracle.compact(keep_ref[fex])
            worst = 0.0
            for li, ret in enumerate(res["ret"]):
                lay, f_pcu = sub_layers([layers[2 + li]], inp.cu_prefix, blk, fseqs)
                lay = lay[0]
                ref = oracle.retained_attn(lay["q"], lay["k_blk"], lay["v_blk"], f_idx,
                                           f_cu, lay["k_cache"], lay["v_cache"], f_pcu,
                                           blk, cfg.hq, cfg.hkv)
                got = np.concatenate([ret[g_cu[b]:g_cu[b + 1]] for b in fseqs])
                err = assert_close(f"retained L{2 + li}", got, ref, tol["out"],
                                   tight["out"], rel_scale=True)
                worst = max(worst, err)
            rep.errors["retained"] = worst
    return rep


def compare_constrained(inp: workloads.Inputs, res, masked, rules: int,
                        k_keep=None, k_gpu=None, skip=()):
    """The masked-candidate selection with structural rules against the
    oracle's own selection on the oracle's own importance (all sequences),
    plus the retained attention of the further layers on exactly matched
    sequences. The GPU's result must also be a valid selection of its own
    delta (set-based characterisation)."""
    from tests.test_oracle_constrained import _characterise
    cfg = inp.cfg
    blk, kind, n = cfg.block, cfg.dtype, cfg.batch
    pred, mpre = bool(rules & 1), bool(rules & 2)
    seqs = list(range(n))
    sub, sub_cu = sub_layers(inp.layers, inp.cu_prefix, blk, seqs)
    o = [oracle.block_attn_importance(sub[l]["q"], sub[l]["k_blk"], sub[l]["v_blk"],
                                      sub[l]["k_cache"], sub[l]["v_cache"], sub_cu,
                                      blk, cfg.hq, cfg.hkv) for l in (0, 1)]
    for l in (0, 1):
        assert_close(f"imp L{l}", res["imp"][l], o[l][1], TOL[kind]["imp"],
                     TIGHT[kind]["imp"])
    dI_ref = oracle.importance_delta(o[0][1], o[1][1], cfg.pool_k)
    assert_close("dI", res["dI"], dI_ref, TIGHT[kind]["dI"])
    if k_keep is None:
        k_keep = inp.meta.k_keep
    if k_gpu is None:
        k_gpu = k_keep
    keep_ref, cand_ref = oracle.select_constrained(dI_ref, masked, k_keep, pred, mpre)
    exact, excused = [], 0
    for b in seqs:
        _characterise(res["dI"][b].astype(np.float64), masked[b], int(k_gpu[b]),
                      pred, mpre, res["keep"][b], res["cand"][b])
        if b in skip:
            excused += 1
            continue
        if (np.array_equal(res["keep"][b], keep_ref[b])
                and np.array_equal(res["cand"][b], cand_ref[b])):
            exact.append(b)
            continue
        elig = [j for j in range(blk) if masked[b, j]]
        order = sorted(elig, key=lambda j: (-dI_ref[b, j], j))
        kb = min(max(int(k_keep[b]), 0), len(elig))
        assert 0 < kb < len(elig), f"seq {b}: mismatch without a tie candidate"
        gap = dI_ref[b, order[kb - 1]] - dI_ref[b, order[kb]]
        assert gap < GAP, f"seq {b}: gpu {np.flatnonzero(res['cand'][b])} " \
                          f"oracle {np.flatnonzero(cand_ref[b])} gap {gap}"
        excused += 1
    log(f"  constrained selection: {len(exact)} exact, {excused} excused")
    # compaction of the GPU's own retained set
    cnt = res["keep"].sum(axis=1)
    cu = res["cu_ret"]
    assert cu[0] == 0 and np.array_equal(np.diff(cu), cnt)
    total = int(cu[-1])
    assert np.array_equal(res["idx"][:total], np.flatnonzero(res["keep"].ravel()))
    # retained attention of the further layers on exactly matched sequences
    idx_ref, cu_ref = oracle.compact(keep_ref)
    for li, ret in enumerate(res["ret"]):
        lay = sub[2 + li]
        ref = oracle.retained_attn(lay["q"], lay["k_blk"], lay["v_blk"], idx_ref,
                                   cu_ref, lay["k_cache"], lay["v_cache"], sub_cu,
                                   blk, cfg.hq, cfg.hkv)
        got = [ret[cu[b]:cu[b + 1]] for b in exact if cu[b + 1] > cu[b]]
        want = [ref[cu_ref[b]:cu_ref[b + 1]] for b in exact if cu[b + 1] > cu[b]]
        if got:
            assert_close(f"retained L{2 + li}", np.concatenate(got),
                         np.concatenate(want), TOL[kind]["out"], TIGHT[kind]["out"],
                         rel_scale=True)
    return exact


def compare_dynamic(inp: workloads.Inputs, res, masked, yield_hist, alpha: float,
                    rules: int):
    """Dynamic budget: the GPU's K_b equals the oracle's reading except
    where an oracle delta lies within GAP of the +Std threshold (the count
    is then decided by rounding); the selection is then compared as in
    compare_constrained with the oracle's K."""
    cfg = inp.cfg
    seqs = list(range(cfg.batch))
    sub, sub_cu = sub_layers(inp.layers, inp.cu_prefix, cfg.block, seqs)
    imps = [oracle.block_attn_importance(sub[l]["q"], sub[l]["k_blk"], sub[l]["v_blk"],
                                         sub[l]["k_cache"], sub[l]["v_cache"], sub_cu,
                                         cfg.block, cfg.hq, cfg.hkv)[1] for l in (0, 1)]
    dI_ref = oracle.importance_delta(imps[0], imps[1], cfg.pool_k)
    k_ref = oracle.dynamic_budget(dI_ref, masked, yield_hist, alpha)
    k_gpu = res["k_used"]
    skip = set()
    for b in seqs:
        if k_gpu[b] == k_ref[b]:
            continue
        v = dI_ref[b][np.asarray(masked[b]).astype(bool)]
        margin = float(np.min(np.abs(v - (v.mean() + v.std()))))
        assert margin < GAP, f"seq {b}: K gpu {k_gpu[b]} oracle {k_ref[b]} margin {margin}"
        skip.add(b)
    log(f"  dynamic budget: {cfg.batch - len(skip)} of {cfg.batch} K_b equal "
        f"(K range {int(k_ref.min())}..{int(k_ref.max())})")
    return compare_constrained(inp, res, masked, rules, k_keep=k_ref, k_gpu=k_gpu,
                               skip=skip)
