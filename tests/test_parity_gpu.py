"""HIP path vs the float64 oracle, element by element (needs an MI355X).

Small cases run the oracle on every sequence; the full-size workloads are
checked on sampled sequences that the oracle computes one by one. Every
call goes through the C ABI of libfocus (via the thin Python binding).
"""
import json
import os

import numpy as np
import pytest
import torch

import workloads
from tests import parity
from tests.parity import log

pytestmark = pytest.mark.gpu


def _case(name, cfg, seed=0, n_layers=None, prefix_lens=None, k_keep=None,
          seqs=None):
    log(f"[parity] {name}: N={cfg.batch} B={cfg.block} Hq={cfg.hq} "
        f"Hkv={cfg.hkv} d={cfg.head_dim} {cfg.dtype} seed={seed}")
    inp = workloads.make_inputs(cfg, seed, n_layers=n_layers,
                                prefix_lens=prefix_lens, k_keep=k_keep)
    step, res = parity.run_gpu(inp)
    rep = parity.compare_step(inp, res, range(cfg.batch) if seqs is None else seqs)
    return inp, step, res, rep


def test_c1_tiny_f32():
    _case("c1", workloads.get("c1"), n_layers=3)


def test_c2_bf16_full():
    _case("c2", workloads.get("c2"), n_layers=3)


def test_c3_reduced_batch():
    cfg = workloads.scaled(workloads.get("c3"), batch=24)
    _case("c3 reduced", cfg, n_layers=3)


def test_c4_reduced_batch():
    cfg = workloads.scaled(workloads.get("c4"), batch=3)
    _case("c4 reduced", cfg, n_layers=3)


def test_c5_reduced_batch_several_layers():
    cfg = workloads.scaled(workloads.get("c5"), batch=6, extra_layers=3)
    _case("c5 reduced", cfg)


def test_c6_b64_reduced_batch():
    cfg = workloads.scaled(workloads.get("c6"), batch=16)
    _case("c6 reduced", cfg, n_layers=3)


EDGE = [
    # name, overrides, prefix lengths, budgets
    ("B1 P0/1/63 d64", dict(block=1, hq=4, hkv=1, head_dim=64), [0, 1, 63], [0, 1, 1]),
    ("B7 G8 ragged", dict(block=7, hq=8, hkv=1), [0, 65, 129], [0, 3, 7]),
    ("B64 G4 tile edges", dict(block=64, hq=8, hkv=2), [63, 64, 1], [1, 32, 64]),
    ("B128 P4096 full budget", dict(block=128, hq=8, hkv=2, pool_k=5), [4096], [128]),
    ("B128 ragged", dict(block=128, hq=4, hkv=1), [0, 127, 129], [0, 1, 31]),
    ("f32 d64 G1", dict(dtype="f32", head_dim=64, hq=4, hkv=4), [5, 77], [3, 32]),
    ("f32 d128 G2", dict(dtype="f32", head_dim=128, hq=4, hkv=2), [64, 0], [8, 8]),
    ("bf16 d64 G8 B32", dict(head_dim=64, hq=16, hkv=2), [100, 300], [11, 6]),
    ("B16 G8 two chunks", dict(block=16, hq=16, hkv=1), [33, 17], [4, 16]),
    ("B33 G4", dict(block=33, hq=8, hkv=2), [31, 200], [10, 33]),
    ("G1 bf16 d128", dict(hq=8, hkv=8), [100, 2000, 0], [5, 32, 3]),
    ("G2 bf16 d128", dict(hq=8, hkv=4), [33, 700], [12, 1]),
    ("G16 B8 one workgroup", dict(block=8, hq=32, hkv=2, pool_k=3), [64, 257, 5], [2, 8, 4]),
    ("B96 three block tiles", dict(block=96, hq=8, hkv=2, pool_k=5), [300, 0, 97], [24, 96, 1]),
    ("B65 one-key block tile", dict(block=65, hq=8, hkv=2), [64, 129], [65, 13]),
    ("G32 eight head chunks", dict(hq=64, hkv=2), [200, 31], [8, 32]),
    # prefixes past 4096 tokens beside short ones
    ("long B32", dict(block=32, hq=8, hkv=2), [5000, 4200, 33, 1], [5, 32, 1, 0]),
    ("long B128", dict(block=128, hq=8, hkv=2, pool_k=5), [4500, 0], [32, 128]),
    ("long B48 G8", dict(block=48, hq=16, hkv=2), [4100, 4097, 95], [9, 48, 3]),
    # pool windows wider than the block (cut at the block edges; from
    # 2B - 1 on every position takes the block's maximum)
    ("B2 pool 5", dict(block=2, hq=8, hkv=2, pool_k=5), [100, 3, 0], [1, 1, 2]),
    ("B4 pool 9 block max", dict(block=4, hq=8, hkv=2, pool_k=9), [40, 0, 7], [1, 2, 4]),
    ("B5 pool 7", dict(block=5, hq=8, hkv=2, pool_k=7), [33, 64], [2, 3]),
]


@pytest.mark.parametrize("name,over,plens,kk", EDGE, ids=[e[0] for e in EDGE])
def test_edge_cases(name, over, plens, kk):
    base = workloads.get("c2")
    cfg = workloads.scaled(base, batch=len(plens), prefix_fixed=1, **over)
    _case(name, cfg, n_layers=3, prefix_lens=plens, k_keep=kk)


def _random_shapes(n=24, seed=7321):
    """Seeded draws over the supported shapes (B 1..128, d 64 or 128, both
    dtypes, G 1..16, odd pools up to 9), with prefix lengths near tile
    edges and budgets from 0 to B, for combinations no list above names."""
    rng = np.random.default_rng(seed)
    near_edge = [0, 1, 31, 32, 33, 63, 64, 65, 95, 96, 97, 127, 128, 129]
    cases = []
    for i in range(n):
        dtype = "bf16" if rng.random() < 0.75 else "f32"
        d = 128 if rng.random() < 0.7 else 64
        hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([g for g in (1, 2, 4, 8, 16) if g * hkv <= 32]))
        blk = int(rng.choice([int(rng.integers(1, 129)), int(rng.choice([1, 32, 64, 96, 128]))]))
        pool = int(rng.choice([1, 3, 5, 7, 9]))
        nseq = int(rng.integers(1, 5))
        plens = [int(rng.choice(near_edge)) + 32 * int(rng.integers(0, 48))
                 if rng.random() < 0.7 else int(rng.integers(0, 1600)) for _ in range(nseq)]
        kk = [int(rng.integers(0, blk + 1)) for _ in range(nseq)]
        over = dict(block=blk, hq=g * hkv, hkv=hkv, head_dim=d, dtype=dtype, pool_k=pool)
        name = f"r{i} {dtype} d{d} B{blk} G{g} Hkv{hkv} k{pool} P{plens}"
        cases.append((name, over, plens, kk))
    return cases


RANDOM = _random_shapes()


@pytest.mark.parametrize("name,over,plens,kk", RANDOM, ids=[r[0].split()[0] for r in RANDOM])
def test_random_shapes(name, over, plens, kk):
    base = workloads.get("c2")
    cfg = workloads.scaled(base, batch=len(plens), prefix_fixed=1, **over)
    _case(name, cfg, n_layers=3, prefix_lens=plens, k_keep=kk)


def test_retained_with_full_budget_equals_block_attention():
    """Cross-call pin: keeping every token, retained attention on layer L
    must reproduce block attention's output for layer L."""
    cfg = workloads.scaled(workloads.get("c3"), batch=5)
    log("[parity] cross pin retained == block attention")
    inp = workloads.make_inputs(cfg, 3, n_layers=2, k_keep=[32] * 5)
    lay = parity.to_device(inp)
    lay = [lay[0], lay[1], lay[1]]       # further layer = layer 1 itself
    step, res = parity.run_gpu(inp, layers_dev=lay)
    assert step.n_ret == 5 * 32
    assert np.array_equal(res["idx"], np.arange(160))
    got, ref = res["ret"][0], res["out"][1]
    err = float(np.abs(got - ref).max())
    log(f"  retained vs block max abs diff {err:.3e}")
    assert err <= 1e-6


def test_retained_with_full_budget_equals_block_attention_long():
    """The same cross-call pin with prefixes past 4096 tokens."""
    cfg = workloads.scaled(workloads.get("c3"), batch=3, hq=8, hkv=2)
    log("[parity] cross pin retained == block attention, long prefixes")
    inp = workloads.make_inputs(cfg, 4, n_layers=2, prefix_lens=[5000, 33, 4097],
                                k_keep=[32] * 3)
    lay = parity.to_device(inp)
    lay = [lay[0], lay[1], lay[1]]
    step, res = parity.run_gpu(inp, layers_dev=lay)
    got, ref = res["ret"][0], res["out"][1]
    err = float(np.abs(got - ref).max())
    log(f"  retained vs block max abs diff {err:.3e}")
    assert err <= 1e-6


HOT = [
    # name, overrides, prefix lengths, hot keys (layer, tensor, seq, pos, scale)
    ("bf16 d128 G4", dict(hq=8, hkv=2), [300, 97, 1000, 40], [
        (0, "k_cache", 0, 100, 1.3),    # full prefix tile 3, sum above 2^8
        (0, "k_cache", 1, 96, 13.0),    # last, one-key prefix tile, overflow
        (0, "k_blk", 2, 5, 13.0),       # block key (kept raw scores)
        (0, "k_cache", 3, 3, 13.0),     # first tile: sets the running max
        (1, "k_cache", 2, 700, 1.3),
        (1, "k_blk", 3, 20, 1.3),
        (2, "k_cache", 0, 250, 13.0),   # retained attention, prefix tile
        (2, "k_blk", 1, 10, 1.3),       # retained attention, gathered keys
        (2, "k_blk", 3, 31, 13.0),
    ]),
    ("bf16 B128 G4", dict(block=128, hq=8, hkv=2, pool_k=5), [130, 0], [
        (0, "k_cache", 0, 129, 13.0),
        (0, "k_blk", 0, 100, 1.3),
        (0, "k_blk", 1, 70, 13.0),
        (2, "k_blk", 1, 127, 1.3),
        (2, "k_cache", 0, 40, 1.3),
    ]),
    ("f32 d64 G4", dict(dtype="f32", head_dim=64, hq=4, hkv=1), [200, 65], [
        (0, "k_cache", 0, 150, 1.3),
        (0, "k_cache", 1, 64, 13.0),
        (0, "k_blk", 1, 2, 13.0),
        (2, "k_cache", 1, 33, 13.0),
    ]),
]


@pytest.mark.parametrize("name,over,plens,hot", HOT, ids=[h[0] for h in HOT])
def test_rescale_path_hot_keys(name, over, plens, hot):
    """Keys planted as a scaled copy of one query of their group make that
    query's score jump far above the running max after the first tile
    (scale 1.3: about 15 above, the tile's exponential sum passes 2^8;
    scale 13: about 150 above, the exponentials overflow), so the kernels'
    rescale path runs on prefix, block and retained tiles, packed and
    paged, with and without O. Every token is kept, so retained attention
    is compared on every sequence."""
    import attention_delta_token_focus_amd as F
    cfg = workloads.scaled(workloads.get("c2"), batch=len(plens), prefix_fixed=1,
                           **over)
    log(f"[parity] hot keys {name}: N={cfg.batch} B={cfg.block} {cfg.dtype} "
        f"d={cfg.head_dim}")
    inp = workloads.make_inputs(cfg, 21, n_layers=3, prefix_lens=plens,
                                k_keep=[cfg.block] * cfg.batch)
    cu = np.asarray(inp.cu_prefix, dtype=np.int64)
    blk, G = cfg.block, cfg.hq // cfg.hkv
    smax = 0.0
    for li, where, b, pos, scale in hot:
        L = inp.layers[li]
        g = cfg.hkv - 1                       # the last KV group
        qv = L["q"][b * blk + pos % blk, g * G].float()
        row = int(cu[b]) + pos if where == "k_cache" else b * blk + pos
        assert (where == "k_blk" and pos < blk) or pos < cu[b + 1] - cu[b]
        L[where][row, g] = (scale * qv).to(L[where].dtype)
        smax = max(smax, float(qv @ L[where][row, g].float()) / cfg.head_dim ** 0.5)
    lay = parity.to_device(inp)
    step, res = parity.run_gpu(inp, layers_dev=lay)
    # fp32 bars (1e-5) are about one ulp of an exponent argument near 94;
    # they grow with the planted magnitude. The bf16 bars are ten times
    # wider and hold as they are.
    scale = max(1.0, smax / 8.0) if cfg.dtype == "f32" else 1.0
    parity.compare_step(inp, res, range(cfg.batch), bar_scale=scale)
    # Layer 0 again: importance only, and paged prefix (bf16 kernels), both
    # bitwise equal to the packed call with O.
    dm = step.dims
    L = lay[0]
    imp = torch.empty_like(step.imp[0])
    lse = torch.empty_like(step.lse[0])
    F.focus_block_attn_importance(
        F.dtype_code(dm.dtype), dm.batch, dm.block, dm.hq, dm.hkv, dm.head_dim, 0.0,
        L["q"], L["k_blk"], None, L["k_cache"], None, step.cu_prefix, step.order,
        step.max_prefix, None, imp, lse, step.ws, step.ws_bytes)
    torch.cuda.synchronize()
    assert torch.equal(imp, step.imp[0]) and torch.equal(lse, step.lse[0])
    if cfg.dtype == "bf16":
        kp, table, pps = _paged_pool(L["k_cache"], cu, 64, 7)
        vp, _, _ = _paged_pool(L["v_cache"], cu, 64, 7)
        out = torch.empty_like(step.out[0])
        F.focus_block_attn_importance_paged(
            F.dtype_code(dm.dtype), dm.batch, dm.block, dm.hq, dm.hkv, dm.head_dim,
            0.0, L["q"], L["k_blk"], L["v_blk"], kp, vp, table, 64, pps,
            step.cu_prefix, step.order, step.max_prefix, out, imp, lse, step.ws,
            step.ws_bytes)
        torch.cuda.synchronize()
        assert torch.equal(out, step.out[0])
        assert torch.equal(imp, step.imp[0]) and torch.equal(lse, step.lse[0])


@pytest.mark.parametrize("batch", [1, 7, 256, 257, 1000, 8193, 16384, 16385])
def test_schedule_order(batch):
    """focus_schedule: longest prefix first, equal lengths by lower index
    (a stable sort on the negated lengths), on both sides of the 256-sequence
    rank kernel / bitonic sort switch and of the 16384 limit past which the
    natural order is kept. Lengths repeat often, to exercise the ties."""
    import attention_delta_token_focus_amd as F
    rng = np.random.default_rng(batch)
    lens = rng.integers(0, 40, size=batch) * 32 + rng.integers(0, 2, size=batch)
    cu = torch.as_tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device="cuda")
    order = torch.full((batch,), -1, dtype=torch.int32, device="cuda")
    F.focus_schedule(batch, cu, order)
    torch.cuda.synchronize()
    got = order.cpu().numpy()
    if batch > 16384:
        want = np.arange(batch)
    else:
        want = np.argsort(-lens, kind="stable")
    assert np.array_equal(got, want)


@pytest.mark.parametrize("batch", [5, 256, 300])
def test_schedule_non_monotone_prefix(batch):
    """A non-monotone cu_prefix (negative lengths) still gives a permutation,
    ordered by the signed lengths, longest first, and nothing is written
    past order[batch - 1], on both the rank-count and the sort path."""
    import attention_delta_token_focus_amd as F
    rng = np.random.default_rng(77 + batch)
    lens = rng.integers(-60, 60, size=batch)
    lens[:3] = [-1, -1, 0]
    cu = torch.as_tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32),
                         device="cuda")
    buf = torch.full((batch + 8,), -7, dtype=torch.int32, device="cuda")
    F.focus_schedule(batch, cu, buf[:batch])
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    assert np.array_equal(got[:batch], np.argsort(-lens, kind="stable"))
    assert (got[batch:] == -7).all()


@pytest.mark.parametrize("batch,B", [(1025, 7), (1025, 32), (2049, 16),
                                     (3000, 128), (3000, 7)])
def test_compact_past_one_chunk(batch, B):
    """focus_compact past 1024 sequences (the workgroup walks the batch in
    chunks of 1024 and carries the offset), with keep bytes other than 0/1,
    empty and full rows; byte loads (B = 7) and 16-byte row loads."""
    import attention_delta_token_focus_amd as F
    rng = np.random.default_rng(batch * 131 + B)
    vals = rng.integers(1, 256, size=(batch, B)).astype(np.uint8)
    vals[rng.random((batch, B)) < 0.6] = 0
    vals[5] = 0
    vals[1030 % batch] = 255
    keep = torch.from_numpy(vals).cuda()
    idx = torch.full((batch * B + 8,), -7, dtype=torch.int32, device="cuda")
    cu = torch.full((batch + 1,), -7, dtype=torch.int32, device="cuda")
    F.focus_compact(batch, B, keep, idx, cu)
    torch.cuda.synchronize()
    want_idx = np.flatnonzero(vals.ravel() != 0)
    want_cu = np.concatenate([[0], np.cumsum((vals != 0).sum(axis=1))])
    got = idx.cpu().numpy()
    log(f"[compact] batch {batch} B {B}: {len(want_idx)} kept")
    assert np.array_equal(cu.cpu().numpy(), want_cu)
    assert np.array_equal(got[:len(want_idx)], want_idx)
    assert (got[len(want_idx):] == -7).all()


def test_visiting_order_does_not_change_results():
    """With order=NULL (the call schedules itself), with focus_schedule's
    order, and with the reversed order, every output is bitwise equal."""
    import attention_delta_token_focus_amd as F
    cfg = workloads.scaled(workloads.get("c3"), batch=12)
    log("[parity] visiting order independence")
    inp = workloads.make_inputs(cfg, 4, n_layers=3)
    lay = parity.to_device(inp)
    step, r1 = parity.run_gpu(inp, layers_dev=lay)
    order = step.order.cpu().numpy()
    plen = inp.meta.prefix_lens
    assert sorted(order.tolist()) == list(range(12))
    assert all(plen[order[i]] >= plen[order[i + 1]] for i in range(11))
    outs = []
    for variant in ("none", "reversed"):
        o = [torch.empty_like(step.out[0]), torch.empty_like(step.imp[0])]
        ordr = None if variant == "none" else torch.flip(step.order, [0]).contiguous()
        dm = step.dims
        F.focus_block_attn_importance(
            F.FOCUS_BF16, dm.batch, dm.block, dm.hq, dm.hkv, dm.head_dim, 0.0,
            lay[0]["q"], lay[0]["k_blk"], lay[0]["v_blk"], lay[0]["k_cache"],
            lay[0]["v_cache"], step.cu_prefix, ordr, step.max_prefix, o[0], o[1],
            None, step.ws, step.ws_bytes)
        torch.cuda.synchronize()
        outs.append(o)
    for o in outs:
        assert torch.equal(o[0], step.out[0]) and torch.equal(o[1], step.imp[0])


def test_deterministic_bitwise():
    cfg = workloads.scaled(workloads.get("c3"), batch=8)
    log("[parity] determinism")
    inp = workloads.make_inputs(cfg, 5, n_layers=3)
    lay = parity.to_device(inp)
    step, r1 = parity.run_gpu(inp, layers_dev=lay)
    _, r2 = parity.run_gpu(inp, layers_dev=lay)
    for k in ("dI", "keep", "idx", "cu_ret"):
        assert np.array_equal(r1[k], r2[k]), k
    for k in ("out", "imp", "lse", "ret"):
        for a, b in zip(r1[k], r2[k]):
            assert np.array_equal(a, b), k


@pytest.mark.parametrize("over,plens,kk", [
    (dict(), None, None),
    (dict(block=128, pool_k=5), [100, 0, 3000], [32, 0, 128]),
    (dict(block=7), [5, 9, 1, 0], [0, 7, 3, 1]),
])
def test_fused_select_equals_two_calls(over, plens, kk):
    """focus_select must be bit-identical to focus_delta_topk followed by
    focus_compact (keep, dI, idx, cu_ret)."""
    import attention_delta_token_focus_amd as F
    cfg = workloads.scaled(workloads.get("c3"), batch=len(plens) if plens else 40,
                           **over)
    log(f"[parity] fused select B={cfg.block} N={cfg.batch}")
    inp = workloads.make_inputs(cfg, 9, n_layers=2, prefix_lens=plens, k_keep=kk)
    s1, r1 = parity.run_gpu(inp)
    step = s1
    keep2 = torch.zeros_like(step.keep)
    dI2 = torch.zeros_like(step.dI)
    idx2 = torch.full_like(step.idx, -7)
    cu2 = torch.zeros_like(step.cu_ret)
    dm = step.dims
    F.focus_delta_topk(dm.batch, dm.block, dm.hq, dm.pool_k, step.imp[0], step.imp[1],
                       step.k_keep, keep2, dI2)
    F.focus_compact(dm.batch, dm.block, keep2, idx2, cu2)
    torch.cuda.synchronize()
    assert torch.equal(keep2.cpu(), torch.from_numpy(r1["keep"]))
    assert torch.equal(dI2.cpu(), torch.from_numpy(r1["dI"]))
    assert torch.equal(cu2.cpu(), torch.from_numpy(r1["cu_ret"]))
    assert np.array_equal(idx2.cpu().numpy()[:step.n_ret], r1["idx"])


@pytest.mark.parametrize("batch,B", [(4096, 32), (4097, 32), (9000, 7)])
def test_select_large_batches(batch, B):
    """focus_select on both sides of the switch from the one-launch kernel
    (up to 4096 sequences) to delta/top-K + compaction: the delta against
    the oracle's, the selection against the oracle's (bit-exact, or excused
    by the gap rule), the compaction against the kept flags and budgets."""
    import attention_delta_token_focus_amd as F
    import oracle
    rng = np.random.default_rng(batch + B)
    hq, pool = 8, 3
    imp0 = rng.random((batch, hq, B), dtype=np.float32)
    imp1 = rng.random((batch, hq, B), dtype=np.float32)
    kk = rng.integers(-2, B + 3, size=batch).astype(np.int32)
    dev = lambda x: torch.from_numpy(x).cuda()
    keep = torch.full((batch, B), 7, dtype=torch.uint8, device="cuda")
    dI = torch.empty((batch, B), device="cuda")
    idx = torch.full((batch * B + 4,), -7, dtype=torch.int32, device="cuda")
    cu = torch.empty((batch + 1,), dtype=torch.int32, device="cuda")
    log(f"[select] batch {batch} B {B}")
    F.focus_select(batch, B, hq, pool, dev(imp0), dev(imp1), dev(kk), keep, dI, idx, cu)
    torch.cuda.synchronize()
    dI_ref = oracle.importance_delta(imp0.astype(np.float64), imp1.astype(np.float64), pool)
    parity.assert_close("dI", dI.cpu().numpy(), dI_ref, 1e-6)
    keep_h = keep.cpu().numpy()
    rep = parity.SelectionReport()
    for b in range(batch):
        parity.check_selection(keep_h[b], dI_ref[b], kk[b], f"seq {b}", rep)
    log(f"  selection: {rep.exact} exact, {rep.excused} excused")
    assert not rep.failed, rep.failed[:3]
    kb = np.clip(kk, 0, B)
    assert np.array_equal(cu.cpu().numpy(), np.concatenate([[0], np.cumsum(kb)]))
    got = idx.cpu().numpy()
    n = int(kb.sum())
    assert np.array_equal(got[:n], np.flatnonzero(keep_h.ravel()))
    assert (got[n:] == -7).all()


def _record(entry):
    """Logs one full-size parity record; appended as a JSON line to the file
    named by FOCUS_PARITY_RECORD when that is set."""
    line = json.dumps(entry, sort_keys=True)
    log(f"[record] {line}")
    path = os.environ.get("FOCUS_PARITY_RECORD")
    if path:
        with open(path, "a") as f:
            f.write(line + "\n")


def _full_size(name, cfg_name, n_layers=None, further_pick=None):
    """Every sequence of a full-size workload, in the launch configuration
    the benchmark times, against the oracle: S1 on both layers (O, I, lse),
    the delta, the selection (bit-exact, or excused by the 1e-4 gap rule),
    the compaction, and the retained attention of every further layer on the
    exactly matched sequences (of further_pick's sequences, if given)."""
    cfg = workloads.get(cfg_name)
    log(f"[parity] full size {name}: generating on the device")
    inp = workloads.make_inputs(cfg, 0, device="cuda", n_layers=n_layers)
    plen = inp.meta.prefix_lens
    step, res = parity.run_gpu(inp, layers_dev=inp.layers)
    further = None if further_pick is None else sorted(set(further_pick(plen)))
    if further is not None:
        log(f"  retained layers on sequences {further} "
            f"(P_b {[int(plen[s]) for s in further]})")
    rep = parity.compare_step(inp, res, range(cfg.batch), layers_host=inp.layers,
                              further_seqs=further)
    # properties of the whole batch
    kb = np.clip(inp.meta.k_keep, 0, cfg.block)
    assert np.array_equal(res["keep"].sum(axis=1), kb)
    assert np.array_equal(np.diff(res["cu_ret"]), kb)
    imp_sum = res["imp"][0].sum(axis=2)
    assert (imp_sum > 0).all() and (imp_sum <= cfg.block * (1 + 1e-5)).all()
    assert rep.exact + rep.excused == cfg.batch
    _record(dict(config=cfg.name, sequences=cfg.batch, exact=rep.exact,
                 excused=rep.excused, further_layers=len(res["ret"]),
                 retained_sequences_compared=rep.retained_seqs,
                 max_abs_err={k: float(f"{v:.3e}") for k, v in rep.errors.items()}))
    del inp, step
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_c3_full_size_variants():
    """The variant rows at the full c3 size, in the launch configuration the
    benchmark times them: paged prefix KV (shuffled 64-token pages) bitwise
    equal to the packed call; layer 1 without O bitwise equal (importance,
    lse) to the call with O; the masked-candidate selection with both
    structural rules and the dynamic-budget reading against the oracle
    applied to the GPU's own delta (the delta itself is compared with the
    oracle's on every sequence by test_c3_full_size_every_sequence), with
    their compaction; retained attention on the constrained retained set of
    sampled sequences against the oracle."""
    import attention_delta_token_focus_amd as F
    import oracle
    from tests.test_oracle_constrained import _characterise
    cfg = workloads.get("c3")
    log("[parity] full size c3 variants: generating on the device")
    inp = workloads.make_inputs(cfg, 0, device="cuda", n_layers=3)
    lay = inp.layers
    step, res = parity.run_gpu(inp, layers_dev=lay)
    dm = step.dims
    n, blk = cfg.batch, cfg.block
    cu = np.asarray(inp.cu_prefix, dtype=np.int64)
    code = F.dtype_code(dm.dtype)
    # paged prefix, layer 0 with O
    L = lay[0]
    kp, table, pps = _paged_pool(L["k_cache"], cu, 64, 7)
    vp, _, _ = _paged_pool(L["v_cache"], cu, 64, 7)
    out = torch.empty_like(step.out[0])
    imp = torch.empty_like(step.imp[0])
    lse = torch.empty_like(step.lse[0])
    F.focus_block_attn_importance_paged(
        code, n, blk, dm.hq, dm.hkv, dm.head_dim, 0.0, L["q"], L["k_blk"], L["v_blk"],
        kp, vp, table, 64, pps, step.cu_prefix, step.order, step.max_prefix, out, imp,
        lse, step.ws, step.ws_bytes)
    # layer 1 without O
    L1 = lay[1]
    imp1 = torch.empty_like(step.imp[1])
    lse1 = torch.empty_like(step.lse[1])
    F.focus_block_attn_importance(
        code, n, blk, dm.hq, dm.hkv, dm.head_dim, 0.0, L1["q"], L1["k_blk"], None,
        L1["k_cache"], None, step.cu_prefix, step.order, step.max_prefix, None, imp1,
        lse1, step.ws, step.ws_bytes)
    torch.cuda.synchronize()
    assert torch.equal(out, step.out[0]) and torch.equal(imp, step.imp[0])
    assert torch.equal(lse, step.lse[0])
    assert torch.equal(imp1, step.imp[1]) and torch.equal(lse1, step.lse[1])
    del kp, vp
    # masked candidates + both rules, then the dynamic-budget reading
    masked = workloads.draw_masked(cfg, 0)
    yld = workloads.draw_yield(cfg, 0)
    dI_gpu = res["dI"].astype(np.float64)
    dev = lambda x, t: torch.as_tensor(np.asarray(x), dtype=t, device="cuda")
    m_dev = dev(masked, torch.uint8)
    counts = {}
    for kind in ("masked", "dynamic"):
        keep = torch.empty((n, blk), dtype=torch.uint8, device="cuda")
        cand = torch.empty_like(keep)
        dI = torch.empty((n, blk), device="cuda")
        idx = torch.full((n * blk,), -7, dtype=torch.int32, device="cuda")
        cu_ret = torch.empty((n + 1,), dtype=torch.int32, device="cuda")
        if kind == "masked":
            kk = inp.meta.k_keep
            F.focus_select_masked(n, blk, dm.hq, dm.pool_k, step.imp[0], step.imp[1], m_dev,
                                  step.k_keep, 3, keep, cand, dI, idx, cu_ret)
        else:
            k_used = torch.empty((n,), dtype=torch.int32, device="cuda")
            F.focus_select_dynamic(n, blk, dm.hq, dm.pool_k, step.imp[0], step.imp[1], m_dev,
                                   dev(yld, torch.float32), 1.5, 3, keep, k_used, cand, dI,
                                   idx, cu_ret)
        torch.cuda.synchronize()
        assert torch.equal(dI.cpu(), torch.from_numpy(res["dI"]))
        if kind == "dynamic":
            kk = k_used.cpu().numpy()
            k_ref = oracle.dynamic_budget(dI_gpu, masked, yld, 1.5)
            for b in np.flatnonzero(kk != k_ref):
                v = dI_gpu[b][np.asarray(masked[b]).astype(bool)]
                margin = float(np.min(np.abs(v - (v.mean() + v.std()))))
                assert margin < parity.GAP, (b, kk[b], k_ref[b], margin)
            counts["dynamic_budget_equal"] = int((kk == k_ref).sum())
        keep_h, cand_h = keep.cpu().numpy(), cand.cpu().numpy()
        keep_ref, cand_ref = oracle.select_constrained(dI_gpu, masked, kk, True, True)
        assert np.array_equal(keep_h, keep_ref) and np.array_equal(cand_h, cand_ref)
        for b in range(0, n, 17):
            _characterise(dI_gpu[b], masked[b], int(kk[b]), True, True, keep_h[b], cand_h[b])
        cnt = keep_h.sum(axis=1)
        cu_h = cu_ret.cpu().numpy()
        assert np.array_equal(cu_h, np.concatenate([[0], np.cumsum(cnt)]))
        tot = int(cu_h[-1])
        assert np.array_equal(idx.cpu().numpy()[:tot], np.flatnonzero(keep_h.ravel()))
        counts[kind + "_retained_tokens"] = tot
        log(f"  {kind}: {tot} retained tokens, selection equal to the oracle's on all "
            f"{n} sequences")
    # retained attention on the last (dynamic) constrained set, sampled sequences
    L2 = lay[2]
    ret = torch.empty((n * blk, dm.hq, dm.head_dim), dtype=dm.dtype, device="cuda")
    F.focus_retained_attn(code, n, blk, dm.hq, dm.hkv, dm.head_dim, 0.0, L2["q"],
                          L2["k_blk"], L2["v_blk"], idx, cu_ret, n * blk, blk,
                          L2["k_cache"], L2["v_cache"], step.cu_prefix, step.order,
                          step.max_prefix, ret, step.ws, step.ws_bytes)
    torch.cuda.synchronize()
    plen = inp.meta.prefix_lens
    seqs = sorted({int(np.argmax(plen)), int(np.argmin(plen)), 0, 100, 200, 255})
    sub, sub_cu = parity.sub_layers([L2], inp.cu_prefix, blk, seqs)
    s_idx, s_cu = oracle.compact(keep_ref[seqs])
    ref = oracle.retained_attn(sub[0]["q"], sub[0]["k_blk"], sub[0]["v_blk"], s_idx, s_cu,
                               sub[0]["k_cache"], sub[0]["v_cache"], sub_cu, blk, cfg.hq,
                               cfg.hkv)
    got = workloads.to_f32_numpy(ret)
    got = np.concatenate([got[cu_h[b]:cu_h[b + 1]] for b in seqs])
    err = parity.assert_close("retained (constrained set)", got, ref, parity.TOL["bf16"]["out"],
                              parity.TIGHT["bf16"]["out"], rel_scale=True)
    _record(dict(config=cfg.name, variants="paged 64-token pages == packed; layer 1 without O "
                 "== with O; masked + both rules and dynamic budget == oracle on the GPU delta",
                 sequences=n, retained_constrained_sequences_compared=len(seqs),
                 retained_constrained_max_abs_err=float(f"{err:.3e}"), **counts))
    del inp, step
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_c3_full_size_every_sequence():
    _full_size("c3", "c3", n_layers=3)


@pytest.mark.timeout(900)
def test_c5_full_size_every_sequence():
    """All 128 sequences through S1-S5a; 16 of them (longest, shortest and
    14 evenly spaced) through all 34 further layers."""
    def pick(p, n=16):
        out = [int(np.argmax(p)), int(np.argmin(p))]
        for b in range(0, len(p), 7):
            if len(out) < n and b not in out:
                out.append(b)
        return out
    _full_size("c5", "c5", further_pick=pick)


@pytest.mark.timeout(900)
def test_c4_full_size_every_sequence():
    """B = 128 (four block tiles, four workgroups per KV head), fixed
    2048-token prefixes."""
    _full_size("c4", "c4", n_layers=3)


@pytest.mark.timeout(900)
def test_c6_full_size_every_sequence():
    """B = 64 (two block tiles, two workgroups per KV head), lognormal
    prefixes."""
    _full_size("c6", "c6", n_layers=3)


@pytest.mark.parametrize("over,plens,kk", [
    (dict(), None, None),
    (dict(block=128, pool_k=5), [100, 0, 2100], [32, 0, 128]),
    (dict(block=7), [5, 90, 1, 0], [0, 7, 3, 1]),
    (dict(block=48, hq=16, hkv=2), [40, 333], [9, 48]),
    (dict(dtype="f32", head_dim=64, hq=4, hkv=1), [70, 3], [8, 32]),
    (dict(hq=8, hkv=2), [5000, 300], [8, 32]),
])
def test_layer1_importance_only(over, plens, kk):
    """out=NULL on layer 1 (no V read, no P V): the oracle still matches
    importance and lse, and both are bitwise those of the call with out."""
    import attention_delta_token_focus_amd as F
    cfg = workloads.scaled(workloads.get("c3"), batch=len(plens) if plens else 16,
                           **over)
    log(f"[parity] layer-1 importance only B={cfg.block} N={cfg.batch} "
        f"{cfg.dtype} d={cfg.head_dim}")
    inp = workloads.make_inputs(cfg, 12, n_layers=3, prefix_lens=plens, k_keep=kk)
    lay = parity.to_device(inp)
    step, res = parity.run_gpu(inp, layers_dev=lay, l1_output=False)
    assert step.out[1] is None and res["out"][1] is None
    parity.compare_step(inp, res, range(cfg.batch))
    dm = step.dims
    full_out = torch.empty_like(step.out[0])
    imp = torch.empty_like(step.imp[1])
    lse = torch.empty_like(step.lse[1])
    L1 = lay[1]
    F.focus_block_attn_importance(
        F.dtype_code(dm.dtype), dm.batch, dm.block, dm.hq, dm.hkv, dm.head_dim, 0.0,
        L1["q"], L1["k_blk"], L1["v_blk"], L1["k_cache"], L1["v_cache"],
        step.cu_prefix, step.order, step.max_prefix, full_out, imp, lse,
        step.ws, step.ws_bytes)
    torch.cuda.synchronize()
    assert torch.equal(imp, step.imp[1]) and torch.equal(lse, step.lse[1])


MASKED = [
    # overrides, prefix lengths, budgets, rules
    (dict(), None, None, 3),
    (dict(), None, None, 1),
    (dict(), None, None, 2),
    (dict(), None, None, 0),
    (dict(block=128, pool_k=5), [100, 0, 2100], [32, 0, 128], 3),
    (dict(block=7), [5, 90, 1, 0], [0, 7, 3, 1], 3),
    (dict(block=64, hq=8, hkv=2), [64, 1, 200], [1, 64, 20], 3),
]


@pytest.mark.parametrize("over,plens,kk,rules", MASKED,
                         ids=[f"B{m[0].get('block', 32)}-rules{m[3]}-{i}"
                              for i, m in enumerate(MASKED)])
def test_masked_candidates_and_structural_constraints(over, plens, kk, rules):
    from attention_delta_token_focus_amd.step import FocusStep
    cfg = workloads.scaled(workloads.get("c3"), batch=len(plens) if plens else 24,
                           **over)
    log(f"[parity] masked selection rules={rules} B={cfg.block} N={cfg.batch}")
    inp = workloads.make_inputs(cfg, 21, n_layers=3, prefix_lens=plens, k_keep=kk)
    masked = workloads.draw_masked(cfg, 21)
    step = FocusStep(parity.dims_of(cfg), inp.cu_prefix, inp.meta.k_keep,
                     n_further=1, with_lse=True, masked=masked, rules=rules)
    step, res = parity.run_gpu(inp, step=step)
    parity.compare_constrained(inp, res, masked, rules)


def test_masked_select_without_mask_or_rules_equals_focus_select():
    import attention_delta_token_focus_amd as F
    cfg = workloads.scaled(workloads.get("c3"), batch=40)
    log("[parity] focus_select_masked(NULL, 0) == focus_select")
    inp = workloads.make_inputs(cfg, 22, n_layers=2)
    step, r1 = parity.run_gpu(inp)
    dm = step.dims
    keep = torch.zeros_like(step.keep)
    cand = torch.zeros_like(step.keep)
    dI = torch.zeros_like(step.dI)
    idx = torch.full_like(step.idx, -3)
    cu = torch.zeros_like(step.cu_ret)
    F.focus_select_masked(dm.batch, dm.block, dm.hq, dm.pool_k, step.imp[0],
                          step.imp[1], None, step.k_keep, 0, keep, cand, dI, idx, cu)
    torch.cuda.synchronize()
    assert torch.equal(keep.cpu(), torch.from_numpy(r1["keep"]))
    assert torch.equal(cand, keep)
    assert torch.equal(dI.cpu(), torch.from_numpy(r1["dI"]))
    assert torch.equal(cu.cpu(), torch.from_numpy(r1["cu_ret"]))
    assert np.array_equal(idx.cpu().numpy()[:step.n_ret], r1["idx"])


def _step_outputs(step):
    """Every output of a step, the retained rows cut at the count the step
    wrote (cu_ret[batch], read back after the step)."""
    n = int(step.cu_ret[-1].item())
    ts = [step.imp[0], step.imp[1], step.dI, step.keep, step.cu_ret, step.order,
          step.idx[:n], step.ret_out[0][:n]]
    ts += [o for o in step.out if o is not None]
    ts += [x for x in step.lse if x is not None]
    if step.cand is not None:
        ts.append(step.cand)
    return ts


@pytest.mark.parametrize("masked_rules", [None, 3], ids=["plain", "masked-rules3"])
def test_step_graph_replay_equals_eager(masked_rules):
    """A whole block-step only enqueues work (no allocation, no memset, no
    host synchronisation in any call), so it can be captured in a HIP
    graph: every replay gives the same bits as the eager step, also with
    eager steps run between the replays, including the masked selection
    whose retained count is known only on the device."""
    from attention_delta_token_focus_amd.step import FocusStep
    cfg = workloads.scaled(workloads.get("c2"), batch=24)
    log(f"[parity] graph replay of one block-step (masked rules {masked_rules})")
    inp = workloads.make_inputs(cfg, 31, n_layers=3)
    lay = parity.to_device(inp)
    kw = {}
    if masked_rules is not None:
        kw = dict(masked=workloads.draw_masked(cfg, 31), rules=masked_rules)
    step = FocusStep(parity.dims_of(cfg), inp.cu_prefix, inp.meta.k_keep, n_further=1,
                     with_lse=True, **kw)
    for _ in range(2):
        step.run(lay)
    torch.cuda.synchronize()
    ref = [t.clone() for t in _step_outputs(step)]

    def check():
        got = _step_outputs(step)
        assert len(got) == len(ref)
        for a, b in zip(got, ref):
            assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))

    cur = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        step.run(lay)
    cur.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step.run(lay)
    torch.cuda.synchronize()
    for _ in range(3):
        for t in _step_outputs(step):
            t.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        check()
        step.run(lay)
        torch.cuda.synchronize()
        check()


def _paged_pool(kv, cu, page_size, seed, slack=3):
    """The same prefix rows scattered over shuffled pages of a NaN-filled
    pool (a wrong read shows up as NaN). Returns pool, page_table,
    pages_per_seq."""
    lens = np.diff(cu)
    need = [(int(n) + page_size - 1) // page_size for n in lens]
    pps = max(max(need), 1)
    total = sum(need) + slack
    rng = np.random.default_rng(seed)
    perm = rng.permutation(total)
    pool = torch.full((total * page_size,) + tuple(kv.shape[1:]), float("nan"),
                      dtype=kv.dtype, device=kv.device)
    table = np.full((len(lens), pps), -1, dtype=np.int32)
    k = 0
    for b, n in enumerate(lens):
        for p in range(need[b]):
            pg = int(perm[k])
            k += 1
            table[b, p] = pg
            lo = int(cu[b]) + p * page_size
            hi = min(int(cu[b + 1]), lo + page_size)
            pool[pg * page_size:pg * page_size + hi - lo] = kv[lo:hi]
    return pool.contiguous(), torch.as_tensor(table, device=kv.device), pps


PAGED = [
    ("c3 B32 pages of 64", dict(), None, 64),
    ("c3 B32 pages of 32", dict(), None, 32),
    ("B128 pages of 128", dict(block=128, pool_k=5), [100, 0, 2100], 128),
    ("B7 ragged pages of 96", dict(block=7), [5, 90, 1, 0, 200], 96),
    ("f32 d64 pages of 64", dict(dtype="f32", head_dim=64, hq=4, hkv=1), [70, 3, 130], 64),
    ("long prefixes pages of 64", dict(hq=8, hkv=2), [5000, 4097, 64], 64),
]


@pytest.mark.parametrize("name,over,plens,ps", PAGED, ids=[p[0] for p in PAGED])
def test_paged_prefix_equals_packed(name, over, plens, ps):
    """Paged prefix KV: block attention (with and without O) and retained
    attention are bitwise those of the packed layout, which the other tests
    compare with the oracle; the packed results are re-checked here too."""
    import attention_delta_token_focus_amd as F
    cfg = workloads.scaled(workloads.get("c3"), batch=len(plens) if plens else 12,
                           **over)
    log(f"[parity] paged {name}: N={cfg.batch} B={cfg.block} page_size={ps}")
    inp = workloads.make_inputs(cfg, 31, n_layers=3, prefix_lens=plens)
    lay = parity.to_device(inp)
    step, res = parity.run_gpu(inp, layers_dev=lay)
    parity.compare_step(inp, res, range(cfg.batch))
    dm = step.dims
    cu = np.asarray(inp.cu_prefix, dtype=np.int64)
    for li, which in ((0, "block"), (1, "imp_only"), (2, "retained")):
        L = lay[li]
        kp, table, pps = _paged_pool(L["k_cache"], cu, ps, 100 + li)
        vp, table_v, _ = _paged_pool(L["v_cache"], cu, ps, 100 + li)
        assert torch.equal(table, table_v)
        if which == "retained":
            out = torch.empty_like(step.ret_out[0])
            F.focus_retained_attn_paged(
                F.dtype_code(dm.dtype), dm.batch, dm.block, dm.hq, dm.hkv,
                dm.head_dim, 0.0, L["q"], L["k_blk"], L["v_blk"], step.idx,
                step.cu_ret, step.n_ret, step.max_ret, kp, vp, table, ps, pps,
                step.cu_prefix, step.order, step.max_prefix, out, step.ws,
                step.ws_bytes)
            torch.cuda.synchronize()
            assert torch.equal(out[:step.n_ret], step.ret_out[0][:step.n_ret])
            continue
        with_out = which == "block"
        out = torch.empty_like(step.out[0]) if with_out else None
        imp = torch.empty_like(step.imp[0])
        lse = torch.empty_like(step.lse[0])
        F.focus_block_attn_importance_paged(
            F.dtype_code(dm.dtype), dm.batch, dm.block, dm.hq, dm.hkv, dm.head_dim,
            0.0, L["q"], L["k_blk"], L["v_blk"] if with_out else None,
            kp, vp if with_out else None, table, ps, pps, step.cu_prefix,
            step.order, step.max_prefix, out, imp, lse, step.ws, step.ws_bytes)
        torch.cuda.synchronize()
        assert torch.equal(imp, step.imp[li]) and torch.equal(lse, step.lse[li])
        if with_out:
            assert torch.equal(out, step.out[li])


def test_paged_prefix_longer_than_its_row_is_cut():
    """A cu_prefix length past pages_per_seq * page_size (a broken
    max_prefix promise) is cut at the end of the sequence's page-table row:
    the result is bitwise the packed call on the cut prefix, for the tuned
    bf16 kernel and the generic fp32 one."""
    import attention_delta_token_focus_amd as F
    for over in (dict(hq=8, hkv=2), dict(dtype="f32", head_dim=64, hq=4, hkv=1)):
        cfg = workloads.scaled(workloads.get("c3"), batch=3, prefix_fixed=1, **over)
        ps, pps = 64, 2                              # rows hold 128 tokens
        claimed, cut = [200, 100, 129], [128, 100, 128]
        log(f"[parity] paged prefix cut at its row: {cfg.dtype} d={cfg.head_dim}")
        inp = workloads.make_inputs(cfg, 51, n_layers=2, prefix_lens=claimed)
        L = parity.to_device(inp)[0]
        cu_long = np.concatenate([[0], np.cumsum(claimed)]).astype(np.int32)
        cu_cut = np.concatenate([[0], np.cumsum(cut)]).astype(np.int32)
        keep_rows = np.concatenate([np.arange(cu_long[b], cu_long[b] + cut[b])
                                    for b in range(cfg.batch)])
        rows = torch.as_tensor(keep_rows, device="cuda")
        kc, vc = L["k_cache"][rows].contiguous(), L["v_cache"][rows].contiguous()
        kp, table, got_pps = _paged_pool(kc, cu_cut, ps, 9)
        vp, _, _ = _paged_pool(vc, cu_cut, ps, 9)
        assert got_pps == pps
        dt = F.dtype_code(workloads.torch_dtype(cfg))
        n, blk, hq, hkv, d = cfg.batch, cfg.block, cfg.hq, cfg.hkv, cfg.head_dim
        ws_bytes = F.focus_block_attn_importance_workspace(n, blk, hq, hkv, d, ps * pps)
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
        outs = []
        for paged in (True, False):
            out = torch.empty_like(L["q"])
            imp = torch.empty((n, hq, blk), dtype=torch.float32, device="cuda")
            lse = torch.empty_like(imp)
            if paged:
                F.focus_block_attn_importance_paged(
                    dt, n, blk, hq, hkv, d, 0.0, L["q"], L["k_blk"], L["v_blk"], kp, vp,
                    table, ps, pps, torch.as_tensor(cu_long, device="cuda"), None,
                    ps * pps, out, imp, lse, ws, ws_bytes)
            else:
                F.focus_block_attn_importance(
                    dt, n, blk, hq, hkv, d, 0.0, L["q"], L["k_blk"], L["v_blk"], kc, vc,
                    torch.as_tensor(cu_cut, device="cuda"), None, max(cut), out, imp,
                    lse, ws, ws_bytes)
            torch.cuda.synchronize()
            outs.append((out, imp, lse))
        for x, y in zip(*outs):
            assert torch.equal(x, y)


DYNAMIC = [
    # overrides, prefix lengths, masked?, rules
    (dict(), None, True, 3),
    (dict(), None, False, 0),
    (dict(block=128, pool_k=5), [100, 0, 2100, 64], True, 3),
    (dict(block=7), [5, 90, 1, 0], True, 1),
]


@pytest.mark.parametrize("over,plens,use_mask,rules", DYNAMIC,
                         ids=[f"B{d[0].get('block', 32)}-mask{int(d[2])}-rules{d[3]}"
                              for d in DYNAMIC])
def test_dynamic_budget_reading(over, plens, use_mask, rules):
    """The dynamic budget (a labelled reading; parity against the pages is
    unpinned) against the oracle's implementation of the same reading."""
    from attention_delta_token_focus_amd.step import FocusStep
    cfg = workloads.scaled(workloads.get("c3"), batch=len(plens) if plens else 32,
                           **over)
    log(f"[parity] dynamic budget B={cfg.block} N={cfg.batch} mask={use_mask} rules={rules}")
    inp = workloads.make_inputs(cfg, 41, n_layers=3, prefix_lens=plens)
    masked = (workloads.draw_masked(cfg, 41) if use_mask
              else np.ones((cfg.batch, cfg.block), dtype=np.uint8))
    y = workloads.draw_yield(cfg, 41)
    step = FocusStep(parity.dims_of(cfg), inp.cu_prefix, inp.meta.k_keep,
                     n_further=1, with_lse=True,
                     masked=masked if use_mask else None, rules=rules,
                     yield_hist=y, alpha=1.5)
    step, res = parity.run_gpu(inp, step=step)
    parity.compare_dynamic(inp, res, masked, y, 1.5, rules)
