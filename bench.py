#!/usr/bin/env python3
"""Decode throughput of GQLA attention on one MI355X, both paths.

One step = one decode step of one DeepSeek-V3-shaped GQLA attention layer
(128 query heads, 8 groups, latent 512 + rope 64, nope/v 128) over a batch of
64 sequences at context 4096, on both decode paths of the same weights:
  * MQA-absorb, s_q = 1, over the paged latent cache (1152 B/token), and
  * GQA, s_q = 2 (one MTP row, causal between the two new tokens), over the
    cache expanded once by gqla_expand_cache (4224 B/token).
Tokens per step = 64 * 1 + 64 * 2.  Inputs are seeded synthetic tensors,
resident in HBM before timing.  The one-shot expansion is timed separately
and is not part of a step.

Prints ONE JSON line (see the keys below).  `--gpus N` with N > 1 exits: this
build runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/s per MI355X, both paths, B=64 ctx 4K; % of roofline"
WORKLOAD = ("DeepSeek-V3-shaped GQLA decode layer: 128 query heads, 8 groups, latent 512 + "
            "rope 64, nope/v 128, batch 64, context 4096, paged cache (64-token pages); "
            "MQA-absorb s_q=1 over the latent cache + GQA s_q=2 over the expanded cache")
SRC_FILES = ["decode_attention_gqla_amd/csrc/gqa_decode.hip",
             "decode_attention_gqla_amd/csrc/absorb_decode.hip",
             "decode_attention_gqla_amd/csrc/absorb_wide.hip",
             "decode_attention_gqla_amd/csrc/absorb_wide.hip.h",
             "decode_attention_gqla_amd/csrc/common.hip.h",
             "decode_attention_gqla_amd/csrc/combine.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in SRC_FILES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the steps take about 0.3 ms each: 200 warmup steps bring the GPU to its steady state (with 5,
    # the timed steps ran 15% slower)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--absorb-split", type=int, default=2048,
                    help="tokens per split-KV partition of the absorb path (0 = no split)")
    ap.add_argument("--gqa-split", type=int, default=0,
                    help="tokens per split-KV partition of the GQA path (0 = no split)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seqs", type=int, default=64,
                    help="sequences of the batch the CPU oracle decodes (bounded sample)")
    ap.add_argument("--only", choices=["absorb", "gqa"], default=None,
                    help="profiling aid: run only one path per step (not a valid bench line)")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the (g, s_q) = (4, 1) configuration measured after the main steps")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="run only a plain device copy of this many bytes (counter calibration)")
    return ap.parse_args()


def copy_probe(nbytes: int):
    import torch
    n = nbytes // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n * 4, "dispatches": 3}))


def cpu_baseline(case_abs, case_gqa, n_seqs: int, gpu_outs=None):
    """fp64 CPU oracle on a bounded sample: the literal decode of the first
    n_seqs sequences on both paths' row sets.  With gpu_outs ({path: (out, lse)}
    as CPU tensors from the timed run) it also returns their parity against
    these oracle outputs: error_stats of out and the largest lse error."""
    import numpy as np
    from oracle.gqla_ref import Dims, decode_literal, error_stats
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    f = lambda t: t.double().numpy()
    seqs = list(range(n_seqs))
    t0 = time.perf_counter()
    toks = 0
    refs = {}
    for name, case in (("mqa_absorb", case_abs), ("gqa", case_gqa)):
        d = Dims(h_q=case.h_q, g=case.g, r=case.r, d_R=case.d_R, d_nope=case.d_nope,
                 d_v=case.d_v, s_q=case.s_q, bs=case.bs)
        refs[name] = decode_literal(f(case.q_nope), f(case.q_rope), f(case.pages), case.block_table.numpy(),
                                    case.seqlens.numpy(), f(case.w_uk), f(case.w_uv), d, seqs=seqs)
        toks += n_seqs * case.s_q
    dt = time.perf_counter() - t0
    cpu = {"value": toks / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
           "sample": f"fp64 numpy literal decode (expand per group, then softmax attention) of "
                     f"{n_seqs} of the 64 sequences on both paths ({toks} tokens, {dt:.1f} s)"}
    parity = None
    if gpu_outs is not None:
        parity = {"bar": {"max_rel": 1e-2, "rel_l2": 5e-3, "lse_abs": 2e-2},
                  "sequences": n_seqs, "reference": "oracle decode_literal (fp64)"}
        ok = True
        for name, (out, lse) in gpu_outs.items():
            ref_out, ref_lse = refs[name]
            st = error_stats(f(out[:n_seqs]), ref_out)
            lse_err = float(np.max(np.abs(f(lse[:n_seqs]) - ref_lse)))
            good = bool(st["finite"] and st["max_rel"] <= 1e-2 and st["rel_l2"] <= 5e-3 and lse_err <= 2e-2)
            ok = ok and good
            parity[name] = {"max_rel": st["max_rel"], "rel_l2": st["rel_l2"], "lse_max_abs": lse_err,
                            "pass": good}
        parity["pass"] = ok
    return cpu, parity


def measure_append(G, d, pages, bt, sl, lens, w_uk, w_uv, E, steps: int, n_new: int = 2):
    """One step's incremental append: the last n_new tokens of every sequence written into the
    latent pages and their K/V/rope slots into the expanded cache (the rows are the ones already
    there, so the caches do not change)."""
    import torch
    B = len(lens)
    btc = bt.cpu()
    idx = []
    for b, L in enumerate(lens):
        for j in range(n_new):
            t = L - n_new + j
            idx.append((int(btc[b, t // 64]), t % 64))
    pg = torch.tensor([i for i, _ in idx], device="cuda")
    sl_ = torch.tensor([s for _, s in idx], device="cuda")
    rows = pages[pg, sl_].reshape(B, n_new, -1).contiguous()
    fn = lambda: G.gqla_append_tokens(d, rows, pages, bt, sl, w_uk, w_uv, expanded_pages=E)
    warm_up(fn)
    # back-to-back calls between two events (the host enqueues ahead, so launch overhead on the
    # host does not show), several repeats
    us = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        us.append(a.elapsed_time(b) * 1e3 / steps)
    us.sort()
    return {"workload": f"{n_new} new tokens for each of {B} sequences: latent rows plus their K, V and "
                        "rope slots in the expanded cache (g = 8)", "us_per_call_median": us[len(us) // 2]}


def measure_g4(G, rf, config_case, steps: int, absorb_split: int, gsplit: int = 0):
    """The pages' other ridge-optimal configuration, (g, s_q) = (4, 1): 32 heads per group,
    2176 B per token in the expanded cache; both paths over a 64 x 4096 batch, alternating
    (each path's cache flushes the other's from the 256 MB memory-side cache)."""
    import torch
    case = config_case("dsv3_g4", 1)
    d = G.Dims.of(case)
    dev = "cuda"
    pages, bt, sl = case.pages.to(dev), case.block_table.to(dev), case.seqlens.to(dev)
    w_uk, w_uv = case.w_uk.to(dev), case.w_uv.to(dev)
    qn, qr = case.q_nope.to(dev), case.q_rope.to(dev)
    B = case.batch
    lens = [int(x) for x in case.seqlens]
    E = G.expand_cache(d, pages, w_uk, w_uv)
    out = torch.empty(B, 1, case.h_q, case.d_v, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, 1, case.h_q, dtype=torch.float32, device=dev)
    sa = G.make_split_plan(lens, absorb_split) + (absorb_split,) if absorb_split else None
    ws = G.absorb_workspace(d, B, total_splits=sa[1] if sa else 0)
    og, tg = G.make_split_plan(lens, gsplit) if gsplit else (None, 0)
    po = torch.empty(tg, 1, case.h_q, case.d_v, dtype=torch.float32, device=dev) if gsplit else None
    pl = torch.empty(tg, 1, case.h_q, dtype=torch.float32, device=dev) if gsplit else None
    fns = {
        "mqa_absorb": lambda: G.gqla_decode_mqa_absorb(d, qn, qr, pages, bt, sl, w_uk, w_uv, out=out, lse=lse,
                                                       split_offsets=sa[0] if sa else None,
                                                       split_tokens=sa[2] if sa else 0,
                                                       total_splits=sa[1] if sa else 0, workspace=ws),
        "gqa": lambda: G.gqla_decode_gqa(d, qn, qr, E, bt, sl, out=out, lse=lse, split_offsets=og,
                                         split_tokens=gsplit, total_splits=tg, part_out=po, part_lse=pl),
    }
    us_med = time_alternating(fns, steps)
    works = {"mqa_absorb": rf.work_absorb(lens, 128, 4, 512, 64, 128, 128, 1),
             "gqa": rf.work_gqa(lens, 128, 4, 64, 128, 128, 1)}
    res = {}
    for k in fns:
        med = us_med[k]
        w = works[k]
        res[k] = {"us_median": med, "tok_s": B / (med * 1e-6), "roofline_us": w.roofline_us(),
                  "roofline_frac": w.roofline_us() / med, "bound": w.bound(), "alg_bytes": w.bytes}
    del E
    return {"workload": "(g, s_q) = (4, 1): 128 query heads in 4 groups of 32, latent 512 + rope 64, "
                        "batch 64, context 4096", "absorb_split_tokens": absorb_split,
            "gqa_split_tokens": gsplit, "paths": res}


def warm_up(fn, seconds: float = 0.05):
    """Call `fn` for about `seconds` of GPU time before timing it: the GPU reaches its steady
    clock only after some tens of milliseconds of work (the main loop's 200 warmup steps take
    about 50 ms), and a variant's calls follow seconds of host-side input generation."""
    import torch
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(3):
        fn()
    b.record()
    torch.cuda.synchronize()
    per_call = max(a.elapsed_time(b) * 1e-3 / 3, 1e-6)
    for _ in range(min(2000, int(seconds / per_call))):
        fn()
    torch.cuda.synchronize()


def time_alternating(fns: dict, steps: int) -> dict:
    """Median microseconds per call of each function, calling them in turn (each path's cache then
    flushes the other's from the 256 MB memory-side cache, as in a step).  One HIP event between
    consecutive calls: a call's time is the interval between the events around it, so it holds one
    event marker (about 3 us), as in the main loop's per-path pass."""
    import torch
    warm_up(lambda: [fn() for fn in fns.values()])
    evs = {k: [] for k in fns}
    marks = [torch.cuda.Event(enable_timing=True)]
    marks[0].record()
    for _ in range(steps):
        for k, fn in fns.items():
            fn()
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            evs[k].append((marks[-1], e))
            marks.append(e)
    torch.cuda.synchronize()
    res = {}
    for k in fns:
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs[k])
        res[k] = us[len(us) // 2]
    return res


def time_back_to_back(fn, steps: int, repeats: int = 5) -> float:
    """Microseconds per call of `fn` called `steps` times back to back between two HIP events (the
    host enqueues ahead of the GPU, so neither host launch gaps nor per-call markers show); the
    median over `repeats` such runs."""
    import torch
    warm_up(fn)
    us = []
    for _ in range(repeats):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        us.append(a.elapsed_time(b) * 1e3 / steps)
    us.sort()
    return us[len(us) // 2]


def path_entry(us: float, tokens: int, w) -> dict:
    return {"us_median": us, "tok_s": tokens / (us * 1e-6), "alg_bytes": w.bytes, "bound": w.bound(),
            "achieved_GBps": w.bytes / (us * 1e-6) / 1e9, "roofline_us": w.roofline_us(),
            "roofline_frac": w.roofline_us() / us}


def measure_dense(G, rf, config_case, name: str, steps: int, absorb_split: int, gqa_split: int,
                  sqs=((1, 2),), seed_base: int = 0) -> dict:
    """Both decode paths on one config of `inputs.CONFIGS`: for each (absorb s_q, GQA s_q) pair the
    MQA-absorb call over the latent cache and the GQA call over its expansion, split-KV by the
    given partition sizes (0 = unsplit), timed alternately; the roofline of each call from the drawn
    context lengths."""
    import torch
    res = {}
    E = None
    for sq_a, sq_g in sqs:
        # one seed for every pair, so the cache (and its expansion) is the same
        ca = config_case(name, sq_a, seed=seed_base + 10)
        cg = config_case(name, sq_g, seed=seed_base + 10)
        assert torch.equal(ca.pages, cg.pages) and torch.equal(ca.w_uv, cg.w_uv)
        dev = "cuda"
        da, dg = G.Dims.of(ca), G.Dims.of(cg)
        pages, bt, sl = ca.pages.to(dev), ca.block_table.to(dev), ca.seqlens.to(dev)
        w_uk, w_uv = ca.w_uk.to(dev), ca.w_uv.to(dev)
        if E is None:
            E = G.expand_cache(dg, pages, w_uk, w_uv)
        qa = (ca.q_nope.to(dev), ca.q_rope.to(dev))
        qg = (cg.q_nope.to(dev), cg.q_rope.to(dev))
        B, H = ca.batch, ca.h_q
        lens = [int(x) for x in ca.seqlens]
        out_a = torch.empty(B, sq_a, H, ca.d_v, dtype=torch.bfloat16, device=dev)
        lse_a = torch.empty(B, sq_a, H, dtype=torch.float32, device=dev)
        out_g = torch.empty(B, sq_g, H, cg.d_v, dtype=torch.bfloat16, device=dev)
        lse_g = torch.empty(B, sq_g, H, dtype=torch.float32, device=dev)
        sa = G.make_split_plan(lens, absorb_split) if absorb_split else (None, 0)
        sg = G.make_split_plan(lens, gqa_split) if gqa_split else (None, 0)
        ws = G.absorb_workspace(da, B, total_splits=sa[1])
        po = torch.empty(sg[1], sq_g, H, cg.d_v, dtype=torch.float32, device=dev) if gqa_split else None
        pl = torch.empty(sg[1], sq_g, H, dtype=torch.float32, device=dev) if gqa_split else None
        fns = {
            "mqa_absorb": lambda: G.gqla_decode_mqa_absorb(da, qa[0], qa[1], pages, bt, sl, w_uk, w_uv, out=out_a,
                                                           lse=lse_a, split_offsets=sa[0],
                                                           split_tokens=absorb_split if absorb_split else 0,
                                                           total_splits=sa[1], workspace=ws),
            "gqa": lambda: G.gqla_decode_gqa(dg, qg[0], qg[1], E, bt, sl, out=out_g, lse=lse_g, split_offsets=sg[0],
                                             split_tokens=gqa_split if gqa_split else 0, total_splits=sg[1],
                                             part_out=po, part_lse=pl),
        }
        us = time_alternating(fns, steps)
        wa = rf.work_absorb(lens, H, ca.g, ca.r, ca.d_R, ca.d_nope, ca.d_v, sq_a)
        wg = rf.work_gqa(lens, H, cg.g, cg.d_R, cg.d_nope, cg.d_v, sq_g)
        res[f"absorb_sq{sq_a}"] = path_entry(us["mqa_absorb"], B * sq_a, wa)
        res[f"gqa_sq{sq_g}"] = path_entry(us["gqa"], B * sq_g, wg)
        del pages
    del E
    return res


def measure_sparse(G, rf, d2, qn, qr, E, bt, sl, lens, steps: int, topks=(2048, 512)):
    """Sparse GQLA on the GQA path: each of the 8 groups of every sequence attends to its own
    seeded random selection of `topk` distinct positions (stand-in for an indexer's top-k),
    over the same expanded cache and s_q = 2 queries as the dense GQA path.  One call = the
    row-resolution kernel + the gathering decode."""
    import torch
    from decode_attention_gqla_amd.inputs import sparse_indices
    B = len(lens)
    res = {}
    for topk in topks:
        idx_h = sparse_indices(lens, d2.num_groups, topk, seed=topk)
        idx = idx_h.to("cuda")
        ws = G.sparse_workspace(d2, B, topk)
        out = torch.empty(B, 2, 128, 128, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(B, 2, 128, dtype=torch.float32, device="cuda")

        def fn():
            G.gqla_decode_gqa_sparse(d2, qn, qr, E, bt, sl, idx, out, lse=lse, workspace=ws)
        med = time_back_to_back(fn, steps)
        w = rf.work_gqa_sparse(idx_h.numpy(), lens, 128, 8, 64, 128, 128, 2)
        res[f"topk_{topk}"] = {"us_median": med, "tok_s": B * 2 / (med * 1e-6), "alg_bytes": w.bytes,
                               "bound": w.bound(), "achieved_GBps": w.bytes / (med * 1e-6) / 1e9,
                               "roofline_us": w.roofline_us(), "roofline_frac": w.roofline_us() / med}
    return {"workload": "sparse GQA, DeepSeek-V3 shape, batch 64, context 4096, s_q = 2, topk distinct "
                        "random positions per (sequence, group)", "calls": res}


def measure_sparse_ragged(G, rf, config_case, steps: int, topk: int = 2048, splits=(0, 512, 1024)):
    """Sparse GQA at small batch: the ragged long-context mix (16 sequences, contexts log-uniform
    in [1024, 32768]) with s_q = 2 and `topk` random positions per (sequence, group); one
    workgroup per (sequence, group) is only 128 workgroups, so the call is also measured split into
    ranges of entries merged by log-sum-exp."""
    import torch
    from decode_attention_gqla_amd.inputs import sparse_indices
    case = config_case("dsv3_ragged", 2)
    d = G.Dims.of(case)
    dev = "cuda"
    pages, bt, sl = case.pages.to(dev), case.block_table.to(dev), case.seqlens.to(dev)
    w_uk, w_uv = case.w_uk.to(dev), case.w_uv.to(dev)
    qn, qr = case.q_nope.to(dev), case.q_rope.to(dev)
    lens = [int(x) for x in case.seqlens]
    B = len(lens)
    E = G.expand_cache(d, pages, w_uk, w_uv)
    del pages
    idx_h = sparse_indices(lens, d.num_groups, topk, seed=topk + 1)
    idx = idx_h.to(dev)
    w = rf.work_gqa_sparse(idx_h.numpy(), lens, 128, 8, 64, 128, 128, 2)
    out = torch.empty(B, 2, 128, 128, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, 2, 128, dtype=torch.float32, device=dev)
    res = {}
    for split in splits:
        ws = G.sparse_workspace(d, B, topk, split)

        def fn():
            G.gqla_decode_gqa_sparse(d, qn, qr, E, bt, sl, idx, out, lse=lse, workspace=ws,
                                     split_entries=split)
        med = time_back_to_back(fn, steps)
        res[f"split_{split}" if split else "unsplit"] = {
            "us_median": med, "tok_s": B * 2 / (med * 1e-6), "achieved_GBps": w.bytes / (med * 1e-6) / 1e9,
            "roofline_us": w.roofline_us(), "roofline_frac": w.roofline_us() / med}
    del E
    return {"workload": f"sparse GQA, ragged long-context mix: 16 sequences, contexts log-uniform in "
                        f"[1024, 32768], s_q = 2, {topk} random positions per (sequence, group)",
            "alg_bytes": w.bytes, "calls": res}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported by this build "
              "(the GQA path would shard by KV group across GPUs, see DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    import decode_attention_gqla_amd as G
    from decode_attention_gqla_amd import roofline as rf
    from decode_attention_gqla_amd.inputs import config_case

    G.lib()
    log("generating inputs")
    case_abs = config_case("dsv3", 1)
    case_gqa = config_case("dsv3", 2, seed=1002 + 10)      # same weights and cache (same seed)
    assert torch.equal(case_abs.pages, case_gqa.pages) and torch.equal(case_abs.w_uv, case_gqa.w_uv)
    dev = "cuda"
    d1, d2 = G.Dims.of(case_abs), G.Dims.of(case_gqa)
    pages = case_abs.pages.to(dev)
    bt = case_abs.block_table.to(dev)
    sl = case_abs.seqlens.to(dev)
    w_uk, w_uv = case_abs.w_uk.to(dev), case_abs.w_uv.to(dev)
    qa_n, qa_r = case_abs.q_nope.to(dev), case_abs.q_rope.to(dev)
    qg_n, qg_r = case_gqa.q_nope.to(dev), case_gqa.q_rope.to(dev)
    B = case_abs.batch
    lens = [int(x) for x in case_abs.seqlens]

    # one-shot expansion (not part of a step; timed after the steps, see below)
    E = G.expand_cache(d2, pages, w_uk, w_uv)
    torch.cuda.synchronize()

    out_a = torch.empty(B, 1, 128, 128, dtype=torch.bfloat16, device=dev)
    lse_a = torch.empty(B, 1, 128, dtype=torch.float32, device=dev)
    out_g = torch.empty(B, 2, 128, 128, dtype=torch.bfloat16, device=dev)
    lse_g = torch.empty(B, 2, 128, dtype=torch.float32, device=dev)
    sa = G.make_split_plan(lens, args.absorb_split) + (args.absorb_split,) if args.absorb_split else None
    sg = G.make_split_plan(lens, args.gqa_split) + (args.gqa_split,) if args.gqa_split else None
    ws = G.absorb_workspace(d1, B, total_splits=sa[1] if sa else 0)
    pg = (torch.empty(sg[1], 2, 128, 128, dtype=torch.float32, device=dev),
          torch.empty(sg[1], 2, 128, dtype=torch.float32, device=dev)) if sg else (None, None)

    def run_absorb():
        G.gqla_decode_mqa_absorb(d1, qa_n, qa_r, pages, bt, sl, w_uk, w_uv, out=out_a, lse=lse_a,
                                 split_offsets=sa[0] if sa else None,
                                 split_tokens=sa[2] if sa else 0, total_splits=sa[1] if sa else 0,
                                 workspace=ws)

    def run_gqa():
        G.gqla_decode_gqa(d2, qg_n, qg_r, E, bt, sl, out=out_g, lse=lse_g,
                          split_offsets=sg[0] if sg else None, split_tokens=sg[2] if sg else 0,
                          total_splits=sg[1] if sg else 0, part_out=pg[0], part_lse=pg[1])

    paths = [("mqa_absorb", run_absorb), ("gqa", run_gqa)]
    if args.only:
        paths = [p for p in paths if p[0] == {"absorb": "mqa_absorb", "gqa": "gqa"}[args.only]]
    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        for _, fn in paths:
            fn()
    torch.cuda.synchronize()
    # timed region: K steps between two events on the launch stream, nothing in between (a
    # timing event between calls adds a marker packet that the queue waits on: about 3 us per
    # marker measured on this step)
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        for name, fn in paths:
            fn()
    t_end.record()
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    # per-path breakdown: the same K steps again, one event between consecutive calls (a call's
    # time is the interval between the events around it, so it includes one marker: these
    # per-path times, and the fractions of the roofline computed from them, are upper bounds)
    evs = {name: [] for name, _ in paths}
    marks = [torch.cuda.Event(enable_timing=True)]
    marks[0].record()
    for _ in range(args.steps):
        for name, fn in paths:
            fn()
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            evs[name].append((marks[-1], e))
            marks.append(e)
    torch.cuda.synchronize()
    ms_step_marked = marks[0].elapsed_time(marks[-1]) / args.steps
    # the one-shot expansion of the whole pool, timed now that the GPU is in its steady state:
    # median of 10 calls, each between its own two events
    ex_us = []
    if not args.only:
        for _ in range(10):
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record()
            G.gqla_expand_cache(d2, pages, w_uk, w_uv, E)
            ev1.record()
            torch.cuda.synchronize()
            ex_us.append(ev0.elapsed_time(ev1) * 1e3)
    t_expand_us = sorted(ex_us)[len(ex_us) // 2] if ex_us else None
    per_path = {}
    for name, _ in paths:
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs[name])
        per_path[name] = {"us_mean": sum(us) / len(us), "us_median": us[len(us) // 2],
                          "us_p10": us[len(us) // 10], "us_p90": us[(9 * len(us)) // 10]}
    w_abs = rf.work_absorb(lens, 128, 8, 512, 64, 128, 128, 1)
    w_gqa = rf.work_gqa(lens, 128, 8, 64, 128, 128, 2)
    works = {"mqa_absorb": (w_abs, B * 1), "gqa": (w_gqa, B * 2)}
    tokens = sum(works[n][1] for n, _ in paths)
    for name, _ in paths:
        w, tk = works[name]
        t = per_path[name]["us_mean"]
        per_path[name].update({
            "tokens": tk, "tok_s": tk / (t * 1e-6),
            "alg_bytes": w.bytes, "alg_flops": w.flops, "bound": w.bound(),
            "achieved_GBps": w.bytes / (t * 1e-6) / 1e9,
            "achieved_TFLOPs": w.flops / (t * 1e-6) / 1e12,
            "roofline_us": w.roofline_us(), "roofline_frac": w.roofline_us() / t,
        })
    dom = max(per_path, key=lambda n: per_path[n]["us_mean"])
    wd = works[dom][0]
    td = per_path[dom]["us_mean"]
    traffic = None
    src_hash = kernel_source_hash()
    if os.path.exists(TRAFFIC_FILE):
        try:
            tr = json.load(open(TRAFFIC_FILE))
            ent = tr.get(dom)
            if ent and ent.get("source_hash") == src_hash:
                traffic = ent.get("bytes_per_launch")
        except Exception:  # pragma: no cover
            traffic = None
    def roof_of(w, t):
        if w.bound() == "hbm":
            r = {"bound": "hbm", "achieved": w.bytes / (t * 1e-6) / 1e9, "peak": rf.MI355X_HBM_GBPS,
                 "unit": "GB/s"}
        else:
            r = {"bound": "mfma", "achieved": w.flops / (t * 1e-6) / 1e12,
                 "peak": rf.MI355X_BF16_TFLOPS, "unit": "TFLOP/s"}
        r["frac"] = r["achieved"] / r["peak"]
        return r
    roof = roof_of(wd, td)
    roof["traffic"] = traffic
    roof["kernel"] = dom
    # every path's own fraction, and whether each reaches 70% of its roofline
    roof["per_path"] = {n: roof_of(works[n][0], per_path[n]["us_mean"]) for n, _ in paths}
    roof["target_frac"] = 0.7
    roof["target_met"] = all(v["frac"] >= 0.7 for v in roof["per_path"].values())
    roof["worst_path"] = min(roof["per_path"], key=lambda n: roof["per_path"][n]["frac"])
    # the path selector on this batch: at the roofline, and with the fractions of it that
    # each path just reached here
    selector = None
    if not args.only:
        sel_d = G.Dims.make(128, 8, 512, 64, 128, 128, 1)
        names = {G.PATH_ABSORB: "mqa_absorb", G.PATH_GQA: "gqa"}
        at_roof, _, _ = G.gqla_select_path(sel_d, lens, 1, 2, G.Hw(rf.MI355X_HBM_GBPS, rf.MI355X_BF16_TFLOPS,
                                                                    1.0, 1.0, 0))
        fa = min(1.0, per_path["mqa_absorb"]["roofline_frac"])
        fg = min(1.0, per_path["gqa"]["roofline_frac"])
        measured, ea, eg = G.gqla_select_path(sel_d, lens, 1, 2, G.Hw(rf.MI355X_HBM_GBPS, rf.MI355X_BF16_TFLOPS,
                                                                       fa, fg, 0))
        selector = {"at_roofline": names[at_roof], "with_measured_fractions": names[measured],
                    "frac_absorb": fa, "frac_gqa": fg,
                    "tok_s_absorb": ea.tokens_per_s, "tok_s_gqa": eg.tokens_per_s}
    variants = None
    if not args.only and not args.no_variants:
        log("variants: append, sparse GQA, (g, s_q) = (4, 1)")
        variants = {"append_2_tokens": measure_append(G, d2, pages, bt, sl, lens, w_uk, w_uv, E, args.steps),
                    "sparse_gqa": measure_sparse(G, rf, d2, qg_n, qg_r, E, bt, sl, lens, args.steps),
                    "sparse_gqa_ragged": measure_sparse_ragged(G, rf, config_case, args.steps),
                    "g4_sq1": measure_g4(G, rf, config_case, args.steps, args.absorb_split)}
        log("variants: dense ragged long-context mix, LLaMA-3-8B shape")
        variants["dense_ragged"] = {
            "workload": "ragged long-context mix: DeepSeek-V3 shape, 16 sequences, contexts log-uniform in "
                        "[1024, 32768], random 64-token page table; absorb s_q = 1 and GQA s_q = 2, split-KV",
            "absorb_split_tokens": 1280, "gqa_split_tokens": 2560,
            "paths": measure_dense(G, rf, config_case, "dsv3_ragged", args.steps, 1280, 2560, ((1, 2),), 1004)}
        variants["llama3_8b"] = {
            "workload": "LLaMA-3-8B-shaped layer: 32 query heads, 8 groups, latent 512 + rope 64, nope/v 128, "
                        "batch 32, context 2048; both paths at s_q = 1 and s_q = 2",
            "absorb_split_tokens": 512, "gqa_split_tokens": 0,
            "paths": measure_dense(G, rf, config_case, "llama3_8b", args.steps, 512, 0, ((1, 1), (2, 2)), 1001)}
    cpu = None
    parity = None
    if not args.no_cpu and not args.only:
        log("cpu oracle baseline and parity of the timed outputs")
        gpu_outs = {"mqa_absorb": (out_a.cpu(), lse_a.cpu()), "gqa": (out_g.cpu(), lse_g.cpu())}
        cpu, parity = cpu_baseline(case_abs, case_gqa, args.cpu_seqs, gpu_outs)
    line = {
        "metric": METRIC,
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_with_call_markers": ms_step_marked,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": WORKLOAD, "global_batch": B, "seq_len": 4096,
                   "absorb_split_tokens": args.absorb_split, "gqa_split_tokens": args.gqa_split,
                   "only": args.only},
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity": parity,
        "paths": per_path,
        "expand_us": t_expand_us,
        "path_selector": selector,
        "variants": variants,
        "kernel_source_hash": src_hash,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
