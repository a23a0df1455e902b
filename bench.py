"""Benchmark of the FOCUS importance + evict block-step on one MI355X.

One step = one pass of the whole hot path over one batch:
  the visiting order of the sequences (longest prefix first),
  block attention + importance on layer 0 and on layer 1,
  head mean / MaxPool1D / importance delta / top-K,
  compaction of the retained tokens,
  retained-query attention for each further layer (one at the default
  workload, 34 at the full-step workload).
Inputs are seeded synthetic tensors made on the device before timing.

Prints one JSON line. `value` is block-steps/s (sequences through the step
per second) over K steps run back to back. `roofline` is for the dominant
kernel (block attention + importance), timed with HIP events around each
of its launches in a second pass of K steps. `cpu_baseline` times the
float64 oracle on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import workloads  # noqa: E402

METRIC = ("block-steps/sec at B=32, batch 256 (importance+evict); "
          "% of HBM peak BW")
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak of an MI355X
ATTN_SRC = os.path.join(ROOT, "attention_delta_token_focus_amd", "csrc",
                        "attn_bf16.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_block_attn_c3.json")


def attn_bytes(cfg, prefix_lens, with_lse=False, with_out=True) -> int:
    """Algorithmic HBM bytes of one block-attention launch: Q in, O out,
    prefix K/V and block K/V in, importance out (and lse if written).
    Importance only (with_out=False): Q, prefix K and block K in,
    importance out."""
    e = 2 if cfg.dtype == "bf16" else 4
    n, blk, hq, hkv, d = cfg.batch, cfg.block, cfg.hq, cfg.hkv, cfg.head_dim
    f = 2 if with_out else 1
    per_seq = f * blk * hq * d * e + f * blk * hkv * d * e + 4 * hq * blk
    if with_lse:
        per_seq += 4 * hq * blk
    return int(n * per_seq + f * int(prefix_lens.sum()) * hkv * d * e)


def attn_flops(cfg, prefix_lens) -> int:
    """Algorithmic flops of one block-attention launch: Q K^T and P V over
    the P_b prefix keys and the B block keys, 2 flops per multiply-add:
    4 * Hq * B * (P_b + B) * d per sequence."""
    blk, hq, d = cfg.block, cfg.hq, cfg.head_dim
    return int(4 * hq * blk * d * (prefix_lens.astype(np.int64) + blk).sum())


def select_bytes(cfg, n_ret) -> int:
    n, blk, hq = cfg.batch, cfg.block, cfg.hq
    topk = n * (2 * 4 * hq * blk + blk + 4 * blk + 4)
    compact = n * blk + 4 * n_ret + 4 * (n + 1)
    return int(topk + compact)


def retained_bytes(cfg, prefix_lens, n_ret) -> int:
    e = 2 if cfg.dtype == "bf16" else 4
    hq, hkv, d = cfg.hq, cfg.hkv, cfg.head_dim
    return int(n_ret * (2 * hq * d * e + 2 * hkv * d * e + 4)
               + 2 * int(prefix_lens.sum()) * hkv * d * e)


def code_sha(path) -> str:
    """Hash of a source file's code: // comments, trailing blanks and empty
    lines removed, so that a comment edit keeps a measurement taken on the
    same code, and any code change invalidates it."""
    lines = []
    with open(path) as f:
        for line in f:
            code = line.split("//", 1)[0].rstrip()
            if code:
                lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


def load_traffic(cfg_name):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, only
    if it was taken on the current kernel code."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_code_sha") != code_sha(ATTN_SRC) or \
            t.get("workload") != cfg_name:
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(inp, n_further, budget_s=20.0):
    """The oracle, as it stands, on a deterministic stride sample of the
    workload's sequences (same tensors), growing the sample until about
    budget_s seconds of CPU work."""
    import oracle
    from workloads import to_f32_numpy
    cfg = inp.cfg
    cu = inp.cu_prefix.astype(np.int64)
    blk = cfg.block
    order = list(range(0, cfg.batch, 16)) + [b for b in range(cfg.batch)
                                            if b % 16]
    done, t_used = 0, 0.0
    chunk = 4
    while done < cfg.batch and t_used < budget_s:
        seqs = order[done:done + chunk]
        layers = []
        for lay in inp.layers[:2 + n_further]:
            d = {}
            for name in ("q", "k_blk", "v_blk"):
                d[name] = np.concatenate([to_f32_numpy(
                    lay[name][b * blk:(b + 1) * blk]) for b in seqs])
            for name in ("k_cache", "v_cache"):
                d[name] = np.concatenate([to_f32_numpy(
                    lay[name][int(cu[b]):int(cu[b + 1])]) for b in seqs])
            layers.append(d)
        lens = np.array([cu[b + 1] - cu[b] for b in seqs])
        sub_cu = np.concatenate([[0], np.cumsum(lens)])
        t0 = time.perf_counter()
        oracle.block_step(layers[0], layers[1], sub_cu, inp.meta.k_keep[seqs],
                          blk, cfg.hq, cfg.hkv, cfg.pool_k,
                          further_layers=layers[2:])
        t_used += time.perf_counter() - t0
        done += len(seqs)
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    return {
        "value": done / t_used, "unit": "block-steps/s", "cores": int(cores),
        "kind": "oracle",
        "sample": (f"{done} of {cfg.batch} sequences (every 16th first, then "
                   f"the rest in order) of the same workload and tensors, "
                   f"float64 numpy, {t_used:.1f} s of CPU time"),
    }


def time_l1_importance_only(cfg, inp, dims, n_further, args, plen):
    """The same step with layer 1 called with out=NULL (importance and lse
    only: no V stream, no P V), on the same tensors. Reported beside the
    step, which produces O for both layers."""
    from attention_delta_token_focus_amd.step import FocusStep
    step = FocusStep(dims, inp.cu_prefix, inp.meta.k_keep, n_further=n_further,
                     l1_output=False)
    layers = inp.layers
    for _ in range(max(1, args.warmup // 2)):
        step.run(layers)
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for s in range(args.steps):
        step.run(layers)
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
          for _ in range(args.steps)]
    for s in range(args.steps):
        step.schedule()
        step.block_attn(layers[0], 0)
        ev[s][0].record(stream)
        step.block_attn(layers[1], 1)
        ev[s][1].record(stream)
        step.select()
        for i, lay in enumerate(layers[2:2 + n_further]):
            step.retained(lay, i)
    torch.cuda.synchronize()
    l1_s = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) / 1e3
    b = attn_bytes(cfg, plen, with_out=False)
    return {
        "block_steps_per_s": round(cfg.batch * args.steps / (total_ms / 1e3), 1),
        "ms_per_step": round(total_ms / args.steps, 4),
        "block_attn_l1_us": round(l1_s * 1e6, 2),
        "l1_algorithmic_bytes_per_launch": b,
        "l1_achieved_GBs": round(b / l1_s / 1e9, 1),
    }


def time_order_per_call(cfg, inp, dims, n_further, args, rounds=4):
    """The step with one shared visiting order (focus_schedule, as timed
    above) against the same step without it: every attention call gets
    order=NULL and writes the longest-prefix-first order into its workspace
    first (one more small launch per attention call). The two forms
    alternate in blocks of steps, so that clock drift over the run does not
    favour either; medians of the blocks."""
    from attention_delta_token_focus_amd.step import FocusStep
    steps = {shared: FocusStep(dims, inp.cu_prefix, inp.meta.k_keep,
                               n_further=n_further, shared_order=shared)
             for shared in (True, False)}
    layers = inp.layers
    for st in steps.values():
        for _ in range(max(1, args.warmup // 2)):
            st.run(layers)
    stream = torch.cuda.current_stream()
    per = max(1, args.steps // rounds)
    ms = {True: [], False: []}
    torch.cuda.synchronize()
    for r in range(2 * rounds):
        shared = (r % 2 == 0) == (r // 2 % 2 == 0)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(per):
            steps[shared].run(layers)
        t1.record(stream)
        torch.cuda.synchronize()
        ms[shared].append(t0.elapsed_time(t1) / per)
    shared_ms = float(np.median(ms[True]))
    own_ms = float(np.median(ms[False]))
    return {
        "ms_per_step_shared_order": round(shared_ms, 4),
        "ms_per_step_order_per_call": round(own_ms, 4),
        "block_steps_per_s_order_per_call": round(cfg.batch / (own_ms / 1e3), 1),
        "attention_calls_per_step": 2 + n_further,
    }


def paged_pool(kv, cu, page_size, seed):
    """The same prefix rows in shuffled pages of page_size tokens (one
    gather on the device). Returns pool, page_table, pages_per_seq."""
    lens = np.diff(cu)
    need = (lens + page_size - 1) // page_size
    pps = int(max(need.max(), 1))
    total = int(need.sum())
    perm = np.random.default_rng(seed).permutation(total).astype(np.int64)
    table = np.full((len(lens), pps), -1, dtype=np.int32)
    first = np.concatenate([[0], np.cumsum(need)[:-1]])
    dst = np.empty(int(lens.sum()), dtype=np.int64)
    for b, n in enumerate(lens):
        pages = perm[first[b]:first[b] + need[b]]
        table[b, :need[b]] = pages
        t = np.arange(n)
        dst[cu[b]:cu[b + 1]] = pages[t // page_size] * page_size + t % page_size
    pool = torch.zeros((total * page_size,) + tuple(kv.shape[1:]), dtype=kv.dtype,
                       device=kv.device)
    pool[torch.as_tensor(dst, device=kv.device)] = kv
    return pool, torch.as_tensor(table, device=kv.device), pps


def time_paged(cfg, inp, dims, args, plen, page_size=64):
    """Block attention of layer 0 over the same prefix KV held in shuffled
    pages of 64 tokens (focus_block_attn_importance_paged), timed like the
    packed call."""
    import attention_delta_token_focus_amd as F
    from attention_delta_token_focus_amd.step import FocusStep
    step = FocusStep(dims, inp.cu_prefix, inp.meta.k_keep, n_further=0)
    cu = np.asarray(inp.cu_prefix, dtype=np.int64)
    L = inp.layers[0]
    kp, table, pps = paged_pool(L["k_cache"], cu, page_size, 7)
    vp, _, _ = paged_pool(L["v_cache"], cu, page_size, 7)
    step.schedule()

    def call():
        F.focus_block_attn_importance_paged(
            F.dtype_code(dims.dtype), dims.batch, dims.block, dims.hq, dims.hkv,
            dims.head_dim, 0.0, L["q"], L["k_blk"], L["v_blk"], kp, vp, table,
            page_size, pps, step.cu_prefix, step.order, step.max_prefix,
            step.out[0], step.imp[0], None, step.ws, step.ws_bytes)

    for _ in range(max(1, args.warmup // 2)):
        call()
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        ev[s][0].record(stream)
        call()
        ev[s][1].record(stream)
    torch.cuda.synchronize()
    us = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e3
    b = attn_bytes(cfg, plen)
    del kp, vp
    return {"page_size": page_size, "block_attn_us": round(us, 2),
            "achieved_GBs": round(b / (us / 1e6) / 1e9, 1)}


def time_dynamic_select(cfg, inp, dims, args):
    """focus_select_dynamic (the labelled reading of the dynamic budget)
    with the same still-masked flags and both structural rules."""
    from attention_delta_token_focus_amd.step import FocusStep
    masked = workloads.draw_masked(cfg, args.seed)
    y = workloads.draw_yield(cfg, args.seed)
    step = FocusStep(dims, inp.cu_prefix, inp.meta.k_keep, n_further=0,
                     masked=masked, rules=3, yield_hist=y, alpha=1.5)
    step.run(inp.layers)
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        ev[s][0].record(stream)
        step.select()
        ev[s][1].record(stream)
    torch.cuda.synchronize()
    k = step.k_used.cpu().numpy()
    return {
        "select_dynamic_us": round(float(np.mean(
            [e[0].elapsed_time(e[1]) for e in ev])) * 1e3, 2),
        "alpha": 1.5, "mean_budget": round(float(k.mean()), 3),
        "retained_tokens": int(step.cu_ret[-1].item()),
    }


def time_masked_select(cfg, inp, dims, n_further, args):
    """focus_select_masked with seeded still-masked flags and both
    structural rules (selection + compaction), then the retained attention
    of the further layers on the constrained retained set; the block
    attention of layers 0 and 1 runs once beforehand."""
    from attention_delta_token_focus_amd.step import FocusStep
    masked = workloads.draw_masked(cfg, args.seed)
    step = FocusStep(dims, inp.cu_prefix, inp.meta.k_keep, n_further=n_further,
                     masked=masked, rules=3)
    layers = inp.layers
    step.run(layers)
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        ev[s][0].record(stream)
        step.select()
        ev[s][1].record(stream)
        for i, lay in enumerate(layers[2:2 + n_further]):
            step.retained(lay, i)
        ev[s][2].record(stream)
    torch.cuda.synchronize()
    sel = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e3
    ret = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) * 1e3
    n_ret = int(step.cu_ret[-1].item())
    return {
        "select_masked_us": round(sel, 2),
        "retained_attn_all_further_layers_us": round(ret, 2),
        "retained_tokens": n_ret,
        "masked_fraction": round(float(masked.mean()), 4),
        "rules": "predecessor + masked prefix",
    }


def stream_read_reference(args, gib=4):
    """Read bandwidth of a plain device reduction (torch row sums of a
    4 GiB float32 matrix of 8192 rows, one pass; the fastest torch read
    measured on this GPU), timed like the attention launches: the measured
    stream-read figure the block attention is also compared with."""
    x = torch.ones((8192, (gib << 30) // 4 // 8192), dtype=torch.float32, device="cuda")
    for _ in range(2):
        x.sum(dim=1)
    stream = torch.cuda.current_stream()
    n = max(3, min(10, args.steps))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
    torch.cuda.synchronize()
    for e in ev:
        e[0].record(stream)
        x.sum(dim=1)
        e[1].record(stream)
    torch.cuda.synchronize()
    us = float(np.median([e[0].elapsed_time(e[1]) for e in ev])) * 1e3
    del x
    return {"kernel": f"torch row sums of a {gib} GiB float32 matrix (8192 rows)",
            "GBs": round((gib << 30) / (us / 1e6) / 1e9, 1)}


def attn_kernel_name(cfg) -> str:
    """The block-attention kernel instantiation the workload runs: the
    tuned bf16 d = 128 kernel with 1, 2 or 4 block tiles of 32 keys and the
    K/V load cache policy the library picks (0, the default, from three
    head chunks of up to 128 query rows per KV head on; 2, nt, below),
    else the generic kernel."""
    if cfg.dtype != "bf16" or cfg.head_dim != 128:
        return "attn_kernel (generic)"
    nbt = 1 if cfg.block <= 32 else (2 if cfg.block <= 64 else 4)
    g = cfg.hq // cfg.hkv
    per = min(max(128 // cfg.block, 1), g)
    n_hc = -(-g // per)
    pol = 0 if n_hc >= 3 else 2
    return f"attn_bf16_kernel<false, {nbt}, true, false, {pol}>"


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c3", choices=sorted(workloads.CONFIGS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 1 GiB device copy first (PMC scale)")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the layer-1 importance-only variant timing")
    ap.add_argument("--replicas", type=int, default=None,
                    help="copies of the inputs cycled step by step (default: 4 "
                         "when one step's inputs are under 512 MB, so that the "
                         "256 MB MALL does not serve them, else 1)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only; the path shards "
              "by sequence with no exchange, so run it once per GPU.",
              file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2

    from attention_delta_token_focus_amd.step import Dims, FocusStep

    cfg = workloads.get(args.config)
    n_further = 1 if cfg.extra_layers == 0 else cfg.extra_layers
    print(f"[bench] generating {cfg.name} on the device", file=sys.stderr,
          flush=True)
    inp = workloads.make_inputs(cfg, args.seed, device="cuda",
                                n_layers=2 + n_further)
    plen = inp.meta.prefix_lens
    dims = Dims(cfg.batch, cfg.block, cfg.hq, cfg.hkv, cfg.head_dim,
                workloads.torch_dtype(cfg), cfg.pool_k)
    step = FocusStep(dims, inp.cu_prefix, inp.meta.k_keep, n_further=n_further)
    layers = inp.layers
    footprint = sum(t.numel() * t.element_size() for lay in layers for t in lay.values())
    n_rep = args.replicas if args.replicas else (4 if footprint < (512 << 20) else 1)
    reps = [layers] + [[{k: v.clone() for k, v in lay.items()} for lay in layers]
                       for _ in range(n_rep - 1)]

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for w in range(args.warmup):
        step.run(reps[w % n_rep])
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr,
          flush=True)

    stream = torch.cuda.current_stream()
    # Timed pass: K steps back to back, events only at its two ends (events
    # between the kernels of a step add about 40 us per step at c3).
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for s in range(args.steps):
        step.run(reps[s % n_rep])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)

    # Breakdown pass: K more steps with events around each call on the
    # launch stream, for the per-kernel times and the roofline.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        e = ev[s]
        lays = reps[s % n_rep]
        e[5].record(stream)
        step.schedule()
        e[0].record(stream)
        step.block_attn(lays[0], 0)
        e[1].record(stream)
        step.block_attn(lays[1], 1)
        e[2].record(stream)
        step.select()
        e[3].record(stream)
        for i, lay in enumerate(lays[2:2 + n_further]):
            step.retained(lay, i)
        e[4].record(stream)
    torch.cuda.synchronize()

    attn_ms = [ev[s][0].elapsed_time(ev[s][1]) for s in range(args.steps)] + \
              [ev[s][1].elapsed_time(ev[s][2]) for s in range(args.steps)]
    sel_ms = [ev[s][2].elapsed_time(ev[s][3]) for s in range(args.steps)]
    sched_ms = [ev[s][5].elapsed_time(ev[s][0]) for s in range(args.steps)]
    ret_ms = [ev[s][3].elapsed_time(ev[s][4]) for s in range(args.steps)]
    attn_avg_s = float(np.mean(attn_ms)) / 1e3
    a_bytes = attn_bytes(cfg, plen)
    achieved = a_bytes / attn_avg_s / 1e9
    # The launch is bound by whichever roof is lower: HBM below the ridge of
    # MFMA_BF16_PEAK / HBM_PEAK flops per byte, the matrix cores above it.
    a_flops = attn_flops(cfg, plen)
    mfma_bound = a_flops / a_bytes > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    ms_per_step = total_ms / args.steps
    value = cfg.batch * args.steps / (total_ms / 1e3)
    n_ret = step.n_ret
    step_bytes = 2 * a_bytes + select_bytes(cfg, n_ret) + \
        n_further * retained_bytes(cfg, plen, n_ret)
    imp_evict_ms = (float(np.mean(sched_ms)) + float(np.mean(attn_ms)) * 2
                    + float(np.mean(sel_ms)))

    variants = None
    if not args.no_variants:
        variants = {
            "layer1_importance_only": time_l1_importance_only(
                cfg, inp, dims, n_further, args, plen),
            "masked_candidates_structural_rules": time_masked_select(
                cfg, inp, dims, n_further, args),
            "paged_prefix_kv": time_paged(cfg, inp, dims, args, plen),
            "dynamic_budget_reading": time_dynamic_select(cfg, inp, dims, args),
            "order_per_attention_call": time_order_per_call(
                cfg, inp, dims, n_further, args),
        }

    stream_ref = stream_read_reference(args)
    traffic = load_traffic(cfg.name)
    attn_us = np.asarray(attn_ms) * 1e3
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "block-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) Q/K/V, lognormal prefix lengths; "
                "no model weights, no datasets)",
        "config": {
            "workload": cfg.name, "batch": cfg.batch, "block": cfg.block,
            "hq": cfg.hq, "hkv": cfg.hkv, "head_dim": cfg.head_dim,
            "prefix_tokens": int(plen.sum()),
            "prefix": (f"fixed {cfg.prefix_fixed}" if cfg.prefix_fixed else
                       "lognormal median %g sigma %g clipped [%d, %d]"
                       % cfg.prefix_lognormal),
            "retained_tokens": n_ret, "pool_k": cfg.pool_k,
            "further_layers": n_further, "seed": args.seed,
            "input_replicas": n_rep,
        },
        "roofline": {
            "bound": "mfma" if mfma_bound else "hbm",
            "achieved": round(a_flops / attn_avg_s / 1e12, 1) if mfma_bound else round(achieved, 1),
            "peak": MFMA_BF16_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBS,
            "unit": "TFLOP/s" if mfma_bound else "GB/s",
            "frac": round((a_flops / attn_avg_s / 1e12 / MFMA_BF16_PEAK_TFLOPS) if mfma_bound
                          else achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "hbm_GBs": round(achieved, 1),
            "flops_per_launch": a_flops,
            "flops_per_byte": round(a_flops / a_bytes, 1),
            "kernel": "block attention + importance (%s)" % attn_kernel_name(cfg),
            "algorithmic_bytes_per_launch": a_bytes,
            "avg_launch_us": round(attn_avg_s * 1e6, 2),
            "launch_us_p10_p50_p90": [round(float(np.percentile(attn_us, q)), 2)
                                      for q in (10, 50, 90)],
            "stream_read_reference": dict(
                stream_ref, attn_frac_of_it=round(achieved / stream_ref["GBs"], 4)),
        },
        "breakdown_us": {
            "schedule": round(float(np.mean(sched_ms)) * 1e3, 2),
            "block_attn_per_layer": round(float(np.mean(attn_ms)) * 1e3, 2),
            "delta_topk_compact": round(float(np.mean(sel_ms)) * 1e3, 2),
            "retained_attn_all_further_layers": round(float(np.mean(ret_ms)) * 1e3, 2),
        },
        "importance_evict_block_steps_per_s": round(
            cfg.batch / (imp_evict_ms / 1e3), 1),
        "step_hbm_fraction": round(step_bytes / (ms_per_step / 1e3) / 1e9
                                   / HBM_PEAK_GBS, 4),
        "wall_s": round(wall, 3),
        "variants": variants,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr,
              flush=True)
        result["cpu_baseline"] = cpu_baseline(inp, n_further, args.cpu_budget)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
