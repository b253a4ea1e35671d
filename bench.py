#!/usr/bin/env python3
"""Benchmark one block-diffusion denoise step on one MI355X.

A step is one pass of the whole hot path over one 32-slot block:

    xn = RMSNorm(x)                                   bdm_rmsnorm
    x' = x + MoE(xn)   (Clover-shaped layer)          bdm_moe_block_forward
    stats = head(x')   (online-softmax partials)      bdm_lm_head_stats
    tokens = unmask(merge(stats))                     bdm_unmask_from_stats

with H 2048, 256 routed experts (SwiGLU 2048->512->2048, bf16) plus one
shared expert, top-8 with renormalised weights, the untied 248,320 x 2048
head, mask id 151669 and threshold 0.95.  Inputs are seeded synthetic
tensors already resident in HBM.  To keep the 256 MB Infinity Cache from
serving repeated weights, the timed steps rotate over --sets independent
weight sets (router, experts, shared expert, head) and token blocks.

The weights are packed once before the timed region (--layout 2, the
default: MFMA tiles with gate/up as interleaved pairs).

Output: one JSON line (rank 0).  `value` is block-tokens/s of the whole
step; the MoE layer alone (its launches back to back over the rotated sets)
and the head alone are reported beside it, each with its algorithmic HBM
bytes (touched experts x 6,291,456 B; head 1,017,118,720 B) and the fraction
of the 8 TB/s HBM peak, and so are the layer with the coreset selector, 16 /
32 / 64 blocks in one layer call, the load-skew batch, the head over many
rows, the verify epilogue and one step of the 40-layer loop.  The roofline
entry is the head GEMM kernel (one launch per step, the largest single
kernel): after the timed steps the same launches run back to back over the
rotated sets between two HIP events recorded on the stream they run on; its
HBM traffic comes from the committed rocprofv3 counter summary when that was
taken on the current kernel source, else it is null.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PMC_SUMMARY = os.path.join(HERE, "profiles", "all_kernels_bench_workloads.traffic.md")
EXPERT_BYTES = 3 * 2048 * 512 * 2        # gate + up + down, bf16
HEAD_BYTES = 248320 * 2048 * 2


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--sets", type=int, default=4, help="rotated weight sets / token blocks")
    p.add_argument("--cpu-blocks", type=int, default=4,
                   help="weight sets whose blocks the CPU oracle cycles over for cpu_baseline "
                        "(0: skip the CPU baseline)")
    p.add_argument("--cpu-runs", type=int, default=5,
                   help="timed oracle runs per workload after one warm-up (median reported)")
    p.add_argument("--stack-layers", type=int, default=40,
                   help="layers of the denoise-loop stack measured beside the step (0: skip)")
    p.add_argument("--layout", type=int, default=2,
                   help="weight layout (packed once, untimed): 2 = MFMA tiles with gate/up "
                        "packed as pairs, 1 = MFMA tiles, 0 = row-major")
    p.add_argument("--norm-in-router", action="store_true",
                   help="take the step's RMSNorm inside the router (x_norm) instead of its own "
                        "launch (the same bits; measured no faster: every router workgroup "
                        "reduces all 32 rows)")
    return p.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the single-GPU denoise step only: run it with --gpus 1 "
              "(the path is not built for several GPUs).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import block_diffusion_moe_amd as bdm

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bdm.load()
    L, HS = synth.LAYER, synth.HEAD
    print(f"[bench] generating {args.sets} weight sets on device", file=sys.stderr, flush=True)
    sets = []
    for r in range(args.sets):
        inp = synth.moe_inputs(L, seed=r, block_seed=r + 1, device=dev, with_residual=False)
        w_head = synth.head_weights(HS, r, device=dev)
        blk = synth.head_block(HS, w_head, block_seed=r + 1, n_boost=10)
        sets.append((inp, w_head, blk))
    torch.cuda.synchronize()
    # the weights the kernels read: packed once (not timed) or the row-major tensors
    if args.layout == 2:
        pk, pp = bdm.bdm_pack_weights, bdm.bdm_pack_gate_up
        kw_sets = []
        for i, _, _ in sets:
            g, u = pp(i.w_gate, i.w_up)
            sg, su = pp(i.ws_gate, i.ws_up)
            kw_sets.append(dict(w_gate=g, w_up=u, w_down=pk(i.w_down), ws_gate=sg, ws_up=su,
                                ws_down=pk(i.ws_down)))
        heads = [pk(w) for _, w, _ in sets]
    elif args.layout:
        pk = bdm.bdm_pack_weights
        kw_sets = [dict(w_gate=pk(i.w_gate), w_up=pk(i.w_up), w_down=pk(i.w_down),
                        ws_gate=pk(i.ws_gate), ws_up=pk(i.ws_up), ws_down=pk(i.ws_down))
                   for i, _, _ in sets]
        heads = [pk(w) for _, w, _ in sets]
    else:
        kw_sets = [dict(w_gate=i.w_gate, w_up=i.w_up, w_down=i.w_down, ws_gate=i.ws_gate,
                        ws_up=i.ws_up, ws_down=i.ws_down) for i, _, _ in sets]
        heads = [w for _, w, _ in sets]
    torch.cuda.synchronize()

    T, H = L.T, L.H
    moe_ws = bdm.workspace(bdm.bdm_moe_workspace_bytes(T, H, L.I, L.E, L.k, True), dev)
    parts = bdm.bdm_head_stat_parts()
    st_m = torch.empty((T, parts), dtype=torch.float32, device=dev)
    st_s = torch.empty_like(st_m)
    st_a = torch.empty((T, parts), dtype=torch.int32, device=dev)
    xn = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    xs = [s[0].x for s in sets]                  # per-set block input (residual stream)
    xo = [torch.empty_like(s[0].x) for s in sets]  # per-set layer output = head input
    tokens = [s[2].tokens.clone() for s in sets]
    idx = torch.empty((T, L.k), dtype=torch.int32, device=dev)
    nc = torch.zeros((1,), dtype=torch.int32, device=dev)

    def step(i, ev=None):
        r = i % args.sets
        inp, kw, w_head = sets[r][0], kw_sets[r], heads[r]
        x = xs[r]
        if ev is not None:
            ev[0].record()
        if args.norm_in_router:
            # the RMSNorm taken inside the router (x_norm)
            bdm.bdm_moe_block_forward(x, inp.w_router, kw["w_gate"], kw["w_up"], kw["w_down"],
                                      L.k, ws_gate=kw["ws_gate"], ws_up=kw["ws_up"],
                                      ws_down=kw["ws_down"], residual=x, y=xo[r], topk_idx=idx,
                                      ws=moe_ws, x_norm=xn)
            if ev is not None:
                ev[1].record()
        else:
            bdm.bdm_rmsnorm(x, xn, eps=1e-6)
            if ev is not None:
                ev[1].record()
            bdm.bdm_moe_block_forward(xn, inp.w_router, kw["w_gate"], kw["w_up"], kw["w_down"],
                                      L.k, ws_gate=kw["ws_gate"], ws_up=kw["ws_up"],
                                      ws_down=kw["ws_down"], residual=x, y=xo[r], topk_idx=idx,
                                      ws=moe_ws)
        if ev is not None:
            ev[2].record()
        bdm.bdm_lm_head_stats(xo[r], w_head, HS.mask_id, st_m, st_s, st_a)
        if ev is not None:
            ev[3].record()
        bdm.bdm_unmask_from_stats(st_m, st_s, st_a, HS.mask_id, 0.95, True, tokens[r],
                                  n_committed=nc)
        if ev is not None:
            ev[4].record()

    # touched experts per set (routing of each set's step input)
    touched, xns = [], []
    for r in range(args.sets):
        inp = sets[r][0]
        xns.append(torch.empty_like(xn))
        bdm.bdm_rmsnorm(xs[r], xns[r], eps=1e-6)
        y = torch.empty_like(xn)
        bdm.bdm_moe_block_forward(xns[r], inp.w_router, inp.w_gate, inp.w_up, inp.w_down, L.k,
                                  ws_gate=inp.ws_gate, ws_up=inp.ws_up, ws_down=inp.ws_down,
                                  y=y, topk_idx=idx, ws=moe_ws)
        torch.cuda.synchronize()
        touched.append(int(torch.unique(idx).numel()))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # per-call timing (events between the three calls of every step)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(i, evs[i])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / args.steps
    step_ms = np.array([e[0].elapsed_time(e[4]) for e in evs])
    # (with the RMSNorm inside the router, events 1 and 2 coincide)
    norm_us = 0.0 if args.norm_in_router else \
        1e3 * float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    moe_us = 1e3 * float(np.mean([e[0 if args.norm_in_router else 1].elapsed_time(e[2])
                                  for e in evs]))
    gemm_us = 1e3 * float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    merge_us = 1e3 * float(np.mean([e[3].elapsed_time(e[4]) for e in evs]))
    head_us = gemm_us + merge_us

    # untimed-by-events replay of the same steps (no event records in between)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(i)
    stop.record()
    torch.cuda.synchronize()
    ms_step_plain = start.elapsed_time(stop) / args.steps

    # the same steps replayed from HIP graphs (one captured step per weight
    # set; no call in the step allocates, synchronises or records a memset)
    graphs = []
    for r in range(args.sets):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(r)
        graphs.append(g)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        graphs[i % args.sets].replay()
    stop.record()
    torch.cuda.synchronize()
    ms_step_graph = start.elapsed_time(stop) / args.steps
    # and once more with an event pair around every replay (percentiles)
    evg = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        evg[i][0].record()
        graphs[i % args.sets].replay()
        evg[i][1].record()
    torch.cuda.synchronize()
    graph_ms = np.array([e[0].elapsed_time(e[1]) for e in evg])
    del graphs

    # the head GEMM kernel alone: the same launches back to back over the
    # rotated sets, two events on the stream they run on around all of them
    # (per-call events inside a step add their own overhead to each call)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        r = i % args.sets
        bdm.bdm_lm_head_stats(xo[r], heads[r], HS.mask_id, st_m, st_s, st_a)
    stop.record()
    torch.cuda.synchronize()
    gemm_loop_us = start.elapsed_time(stop) * 1e3 / args.steps
    # the MoE layer alone, the same way (each set's own normalised input)
    ylay = torch.empty_like(xn)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        r = i % args.sets
        kw = kw_sets[r]
        bdm.bdm_moe_block_forward(xns[r], sets[r][0].w_router, kw["w_gate"], kw["w_up"],
                                  kw["w_down"], L.k, ws_gate=kw["ws_gate"], ws_up=kw["ws_up"],
                                  ws_down=kw["ws_down"], residual=xs[r], y=ylay, topk_idx=idx,
                                  ws=moe_ws)
    stop.record()
    torch.cuda.synchronize()
    moe_loop_us = start.elapsed_time(stop) * 1e3 / args.steps
    # the same layer with the block coreset expert selector (top_p 0.9 over
    # the 32-slot block), timed the same way; its bytes are the kept experts'
    nk = torch.zeros((1,), dtype=torch.int32, device=dev)
    kept = []
    for r in range(args.sets):
        kw = kw_sets[r]
        bdm.bdm_moe_block_forward(xns[r], sets[r][0].w_router, kw["w_gate"], kw["w_up"],
                                  kw["w_down"], L.k, ws_gate=kw["ws_gate"], ws_up=kw["ws_up"],
                                  ws_down=kw["ws_down"], residual=xs[r], y=ylay, ws=moe_ws,
                                  coreset_top_p=0.9, coreset_block=T, n_kept=nk)
        torch.cuda.synchronize()
        kept.append(int(nk.item()))
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        r = i % args.sets
        kw = kw_sets[r]
        bdm.bdm_moe_block_forward(xns[r], sets[r][0].w_router, kw["w_gate"], kw["w_up"],
                                  kw["w_down"], L.k, ws_gate=kw["ws_gate"], ws_up=kw["ws_up"],
                                  ws_down=kw["ws_down"], residual=xs[r], y=ylay, ws=moe_ws,
                                  coreset_top_p=0.9, coreset_block=T, n_kept=nk)
    stop.record()
    torch.cuda.synchronize()
    cs_us = start.elapsed_time(stop) * 1e3 / args.steps
    kept_mean = float(np.mean([kept[i % args.sets] for i in range(args.steps)]))
    cs_bytes = (kept_mean + 1) * EXPERT_BYTES

    # the self-speculative verify epilogue over the same head: 32 candidates +
    # the boundary row, threshold rule (0.9, 0.6), back to back like the GEMM
    hv = [torch.cat([xo[r], xo[r][:1]]).contiguous() for r in range(args.sets)]
    cv = [tokens[r].clone() for r in range(args.sets)]
    vws = bdm.workspace(bdm.bdm_head_verify_workspace_bytes(T + 1, H, HS.V), dev)
    vtok = torch.empty((T + 1,), dtype=torch.int32, device=dev)
    vna = torch.empty((1,), dtype=torch.int32, device=dev)
    for r in range(args.sets):
        bdm.bdm_lm_head_verify(hv[r], heads[r], cv[r], "threshold", 0.9, 0.6, tokens_out=vtok,
                               n_accepted=vna, ws=vws)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        r = i % args.sets
        bdm.bdm_lm_head_verify(hv[r], heads[r], cv[r], "threshold", 0.9, 0.6, tokens_out=vtok,
                               n_accepted=vna, ws=vws)
    stop.record()
    torch.cuda.synchronize()
    verify_us = start.elapsed_time(stop) * 1e3 / args.steps
    verify_gbs = HEAD_BYTES / (verify_us * 1e-6) / 1e9

    # multi-block batching: 16, 32 and 64 blocks of 32 tokens in one MoE
    # call (one pass over the touched experts), timed back to back the same way
    multi = {}
    for nb in (16, 32, 64):
        TB = nb * T
        shp = synth.MoEShape(T=TB, H=H, E=L.E, I=L.I, k=L.k)
        xb = [synth.moe_tokens(shp, 500 + 10 * nb + r, dev)[0] for r in range(args.sets)]
        wsb = bdm.workspace(bdm.bdm_moe_workspace_bytes(TB, H, L.I, L.E, L.k, True), dev)
        yb = torch.empty((TB, H), dtype=torch.bfloat16, device=dev)
        ib = torch.empty((TB, L.k), dtype=torch.int32, device=dev)
        ub = []
        for r in range(args.sets):
            kw = kw_sets[r]
            bdm.bdm_moe_block_forward(xb[r], sets[r][0].w_router, kw["w_gate"], kw["w_up"],
                                      kw["w_down"], L.k, ws_gate=kw["ws_gate"], ws_up=kw["ws_up"],
                                      ws_down=kw["ws_down"], y=yb, topk_idx=ib, ws=wsb)
            torch.cuda.synchronize()
            ub.append(int(torch.unique(ib).numel()))
        nrep = max(8, args.steps // 4)
        torch.cuda.synchronize()
        start.record()
        for i in range(nrep):
            r = i % args.sets
            kw = kw_sets[r]
            bdm.bdm_moe_block_forward(xb[r], sets[r][0].w_router, kw["w_gate"], kw["w_up"],
                                      kw["w_down"], L.k, ws_gate=kw["ws_gate"], ws_up=kw["ws_up"],
                                      ws_down=kw["ws_down"], y=yb, ws=wsb)
        stop.record()
        torch.cuda.synchronize()
        us = start.elapsed_time(stop) * 1e3 / nrep
        ubm = float(np.mean([ub[i % args.sets] for i in range(nrep)]))
        nbytes = (ubm + 1) * EXPERT_BYTES
        flops = TB * (L.k + 1) * 6.0 * H * L.I
        multi[f"{nb}_blocks"] = {
            "tokens": TB, "us": round(us, 2), "block_tokens_per_s": round(TB / (us * 1e-6), 1),
            "unique_experts": round(ubm, 2), "bytes": int(nbytes),
            "GB_s": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_of_peak": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "mfma_TFLOP_s": round(flops / (us * 1e-6) / 1e12, 1),
            "mfma_frac_of_bf16_peak": round(flops / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del xb, wsb, yb, ib

    # the load-skew batch: 8 blocks (256 tokens) through the same layers
    # with a log-Zipf router bias (s = 1.1), so a few experts take most tokens
    skew_x = [synth.moe_tokens(synth.SKEW, 700 + r, dev)[0] for r in range(args.sets)]
    skew_b = [synth.zipf_router_bias(L.E, r, 1.1, dev) for r in range(args.sets)]
    wsk = bdm.workspace(bdm.bdm_moe_workspace_bytes(256, H, L.I, L.E, L.k, True), dev)
    yk = torch.empty((256, H), dtype=torch.bfloat16, device=dev)
    ik = torch.empty((256, L.k), dtype=torch.int32, device=dev)
    uk, hot = [], []

    def skew_call(r, topk=None):
        kw = kw_sets[r]
        bdm.bdm_moe_block_forward(skew_x[r], sets[r][0].w_router, kw["w_gate"], kw["w_up"],
                                  kw["w_down"], L.k, router_bias=skew_b[r], ws_gate=kw["ws_gate"],
                                  ws_up=kw["ws_up"], ws_down=kw["ws_down"], y=yk, topk_idx=topk,
                                  ws=wsk)
    for r in range(args.sets):
        skew_call(r, ik)
        torch.cuda.synchronize()
        cnt = torch.bincount(ik.reshape(-1).long(), minlength=L.E)
        uk.append(int((cnt > 0).sum()))
        hot.append(int(cnt.max()))
    nrep = max(8, args.steps // 4)
    torch.cuda.synchronize()
    start.record()
    for i in range(nrep):
        skew_call(i % args.sets)
    stop.record()
    torch.cuda.synchronize()
    sk_us = start.elapsed_time(stop) * 1e3 / nrep
    ukm = float(np.mean([uk[i % args.sets] for i in range(nrep)]))
    sk_bytes = (ukm + 1) * EXPERT_BYTES
    skew = {"tokens": 256, "us": round(sk_us, 2),
            "block_tokens_per_s": round(256 / (sk_us * 1e-6), 1),
            "unique_experts": round(ukm, 2), "busiest_expert_tokens": hot, "bytes": int(sk_bytes),
            "GB_s": round(sk_bytes / (sk_us * 1e-6) / 1e9, 1),
            "frac_of_peak": round(sk_bytes / (sk_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    skew_host = [(synth.bf16_bits(skew_x[r]), skew_b[r].cpu().numpy()) for r in range(args.sets)]
    del skew_x, skew_b, wsk, yk, ik

    # the head statistics over the same 16 / 32 / 64 blocks (all their rows
    # in one call: every 64-row pass in one launch), rotated head sets
    head_multi = {}
    P = bdm.bdm_head_stat_parts()
    g_h = torch.Generator(device=dev)
    g_h.manual_seed(4242)
    for nb in (16, 32, 64):
        TB = nb * T
        hb = torch.randn((TB, H), generator=g_h, device=dev).to(torch.bfloat16)
        st = [torch.empty((TB, P), dtype=dt, device=dev)
              for dt in (torch.float32, torch.float32, torch.int32)]
        for r in range(args.sets):
            bdm.bdm_lm_head_stats(hb, heads[r], HS.mask_id, *st)
        nrep = max(8, args.steps // 4)
        torch.cuda.synchronize()
        start.record()
        for i in range(nrep):
            bdm.bdm_lm_head_stats(hb, heads[i % args.sets], HS.mask_id, *st)
        stop.record()
        torch.cuda.synchronize()
        us = start.elapsed_time(stop) * 1e3 / nrep
        flops = 2.0 * TB * H * HS.V
        head_multi[f"{nb}_blocks"] = {
            "rows": TB, "us": round(us, 2), "rows_per_s": round(TB / (us * 1e-6), 1),
            "head_GB_s": round(HEAD_BYTES / (us * 1e-6) / 1e9, 1),
            "mfma_TFLOP_s": round(flops / (us * 1e-6) / 1e12, 1),
            "mfma_frac_of_bf16_peak": round(flops / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "us_if_one_launch_per_64_rows": round(gemm_loop_us * (TB // 64), 1)}
        del hb, st

    u_mean = float(np.mean([touched[i % args.sets] for i in range(args.steps)]))
    moe_bytes = (u_mean + 1) * EXPERT_BYTES
    moe_gbs = moe_bytes / (moe_loop_us * 1e-6) / 1e9
    head_gbs = HEAD_BYTES / (head_us * 1e-6) / 1e9
    value = T / (ms_step_plain * 1e-3)

    gemm_gbs = HEAD_BYTES / (gemm_loop_us * 1e-6) / 1e9
    stream_gbs, stream_pattern = stream_read_gbs(torch, dev, max(8, args.steps // 10))
    roof = {"bound": "hbm", "kernel": "head_coop_kernel (bdm_lm_head_stats)",
            "achieved": round(gemm_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gemm_gbs / PEAK_HBM_GBS, 4), "traffic": head_traffic(),
            "bytes_per_launch": HEAD_BYTES, "us_per_launch": round(gemm_loop_us, 2),
            "launches_timed": args.steps, "us_per_launch_in_step": round(gemm_us, 2),
            "measured_stream_read_GB_s": round(stream_gbs, 1),
            "measured_stream_read_pattern": stream_pattern,
            "frac_of_measured_stream_read": round(gemm_gbs / stream_gbs, 4)}

    stack = None
    if args.stack_layers > 0:
        stack = stack_step(bdm, synth, torch, np, dev, args, L, HS)

    cpu = None
    if args.cpu_blocks > 0:
        cpu = cpu_baseline(torch, dev, sets[:args.cpu_blocks], skew_host[:args.cpu_blocks],
                           args.stack_layers, args.cpu_runs)

    out = {
        "metric": "denoise-block tokens/s per MoE layer + achieved HBM GB/s (% of MI355X peak)",
        "value": round(value, 1),
        "unit": "block-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step_plain, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations; random init)",
        "config": {
            "workload": "one denoise step over a 32-slot block: RMSNorm + one Clover-shaped MoE "
                        "layer (H 2048, 256 experts SwiGLU 2048->512->2048 + 1 shared, top-8 "
                        "renormalised) + untied 248,320x2048 head with the 0.95 unmask rule",
            "rmsnorm": "inside the router (x_norm)" if args.norm_in_router else
                       "its own launch (bdm_rmsnorm)",
            "block_tokens": T, "hidden": H, "experts": L.E, "top_k": L.k, "inter": L.I,
            "vocab": HS.V, "weight_sets_rotated": args.sets, "parallelism": "single GPU",
            "weight_layout": {2: "mfma_tiles, gate/up as pairs (packed once at load)",
                              1: "mfma_tiles (packed once at load)",
                              0: "row_major"}[args.layout],
        },
        "moe_layer": {"us": round(moe_loop_us, 2), "us_in_step": round(moe_us, 2),
                      "block_tokens_per_s": round(T / (moe_loop_us * 1e-6), 1),
                      "unique_experts": round(u_mean, 2), "bytes": int(moe_bytes),
                      "traffic": moe_layer_traffic(),
                      "GB_s": round(moe_gbs, 1), "frac_of_peak": round(moe_gbs / PEAK_HBM_GBS, 4),
                      "frac_of_measured_stream_read": round(moe_gbs / stream_gbs, 4)},
        "moe_layer_coreset_top_p_0.9": {
            "us": round(cs_us, 2), "block_tokens_per_s": round(T / (cs_us * 1e-6), 1),
            "kept_experts": round(kept_mean, 2), "bytes": int(cs_bytes),
            "GB_s": round(cs_bytes / (cs_us * 1e-6) / 1e9, 1),
            "frac_of_peak": round(cs_bytes / (cs_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
        "head_unmask": {"us": round(head_us, 2), "gemm_us": round(gemm_us, 2),
                        "merge_us": round(merge_us, 2), "bytes": HEAD_BYTES,
                        "GB_s": round(head_gbs, 1), "frac_of_peak": round(head_gbs / PEAK_HBM_GBS, 4)},
        "moe_layer_multiblock": multi,
        "moe_layer_skew_8_blocks": skew,
        "head_stats_multiblock": head_multi,
        "head_verify_33_rows": {"us": round(verify_us, 2), "bytes": HEAD_BYTES,
                                "GB_s": round(verify_gbs, 1),
                                "frac_of_peak": round(verify_gbs / PEAK_HBM_GBS, 4)},
        "denoise_step_stack": stack,
        "rmsnorm_us": round(norm_us, 2),
        "ms_per_step_with_events": round(ms_step, 4),
        "ms_per_step_event_p10_p50_p90": [round(float(np.percentile(step_ms, q)), 4)
                                          for q in (10, 50, 90)],
        "ms_per_step_graph_replay": round(ms_step_graph, 4),
        "ms_per_step_graph_replay_p10_p50_p90": [round(float(np.percentile(graph_ms, q)), 4)
                                                 for q in (10, 50, 90)],
        "wall_s_timed": round(wall, 3),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def stack_step(bdm, synth, torch, np, dev, args, L, HS):
    """One denoise step of the loop driver over a stack of Clover-shaped
    layers (bdm_denoise_block with max_steps 1: embedding, per layer RMSNorm +
    MoE, final RMSNorm, head + unmask, and the per-step host read of the
    counters) from the same initial block, repeated; bytes = every layer's
    touched experts (this step's routing) + the head."""
    nl = args.stack_layers
    print(f"[bench] generating the {nl}-layer stack", file=sys.stderr, flush=True)
    layers = []
    for l in range(nl):
        wr, wg, wu, wd, sg, su, sd, _ = synth.moe_weights(L, 100 + l, dev)
        pk = bdm.bdm_pack_weights
        if args.layout == 2:
            g, u = bdm.bdm_pack_gate_up(wg, wu)
            sgp, sup = bdm.bdm_pack_gate_up(sg, su)
        else:
            g, u, sgp, sup = pk(wg), pk(wu), pk(sg), pk(su)
        layers.append({"w_router": wr, "w_gate": g, "w_up": u, "w_down": pk(wd),
                       "ws_gate": sgp, "ws_up": sup, "ws_down": pk(sd)})
        del wg, wu, wd, sg, su, sd
    emb = stack_embedding(torch, L, HS, dev)
    w_head = bdm.bdm_pack_weights(synth.head_weights(HS, 0, device=dev))
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    gt, tok0 = stack_block(torch, L, HS, dev)
    # this step's routing per layer (untimed), for the bytes
    x = emb[tok0.long()].contiguous()
    xn = torch.empty_like(x)
    idx = torch.empty((L.T, L.k), dtype=torch.int32, device=dev)
    ws = bdm.workspace(bdm.bdm_moe_workspace_bytes(L.T, L.H, L.I, L.E, L.k, True), dev)
    touched = 0
    for lw in layers:
        bdm.bdm_rmsnorm(x, xn, eps=1e-6)
        bdm.bdm_moe_block_forward(xn, lw["w_router"], lw["w_gate"], lw["w_up"], lw["w_down"],
                                  L.k, ws_gate=lw["ws_gate"], ws_up=lw["ws_up"],
                                  ws_down=lw["ws_down"], residual=x, y=x, topk_idx=idx, ws=ws)
        torch.cuda.synchronize()
        touched += int(torch.unique(idx).numel())
    dws = bdm.workspace(bdm.bdm_denoise_workspace_bytes(L.T, L.H, L.I, L.E, L.k, True), dev)
    stack = bdm.MoeStack(layers)                 # marshalled once, as a serving loop would
    tok = tok0.clone()
    bdm.bdm_denoise_block(tok, emb, stack, w_head, L.k, HS.mask_id, 0.95, max_steps=1, ws=dws)
    reps = 5
    times, gtimes = [], []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(reps):
        tok.copy_(tok0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        bdm.bdm_denoise_block(tok, emb, stack, w_head, L.k, HS.mask_id, 0.95, max_steps=1,
                              ws=dws)
        times.append(time.perf_counter() - t0)
        e1.record()
        torch.cuda.synchronize()
        gtimes.append(e0.elapsed_time(e1))
    ms = 1e3 * float(np.median(times))
    nbytes = (touched + nl) * EXPERT_BYTES + HEAD_BYTES
    # the same step with the block coreset selector in every layer (shipped
    # on at top_p 0.9); bytes from this step's kept experts per layer
    x = emb[tok0.long()].contiguous()
    nk = torch.zeros((1,), dtype=torch.int32, device=dev)
    kept = 0
    for lw in layers:
        bdm.bdm_rmsnorm(x, xn, eps=1e-6)
        bdm.bdm_moe_block_forward(xn, lw["w_router"], lw["w_gate"], lw["w_up"], lw["w_down"],
                                  L.k, ws_gate=lw["ws_gate"], ws_up=lw["ws_up"],
                                  ws_down=lw["ws_down"], residual=x, y=x, ws=ws,
                                  coreset_top_p=0.9, coreset_block=L.T, n_kept=nk)
        torch.cuda.synchronize()
        kept += int(nk.item())
    ctimes = []
    for _ in range(reps):
        tok.copy_(tok0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        bdm.bdm_denoise_block(tok, emb, stack, w_head, L.k, HS.mask_id, 0.95, max_steps=1,
                              ws=dws, coreset_top_p=0.9)
        ctimes.append(time.perf_counter() - t0)
    cms = 1e3 * float(np.median(ctimes))
    cbytes = (kept + nl) * EXPERT_BYTES + HEAD_BYTES
    # 16 such blocks (different seeded ids) denoised together: one call over
    # 512 slots, the commit rule per 32-slot block; every layer then touches
    # (nearly) all 256 experts
    nb = 16
    TB = nb * L.T
    tb0 = []
    for b in range(nb):
        ids = torch.randperm(HS.V - 1, generator=gt)[:L.T]
        ids = ids + (ids >= HS.mask_id).long()
        t = ids.to(torch.int32)
        t[(b * 7) % L.T] = HS.mask_id
        tb0.append(t)
    tb0 = torch.cat(tb0).to(dev)
    xb = emb[tb0.long()].contiguous()
    xbn = torch.empty_like(xb)
    ib = torch.empty((TB, L.k), dtype=torch.int32, device=dev)
    wsb = bdm.workspace(bdm.bdm_moe_workspace_bytes(TB, L.H, L.I, L.E, L.k, True), dev)
    mtouched = 0
    for lw in layers:
        bdm.bdm_rmsnorm(xb, xbn, eps=1e-6)
        bdm.bdm_moe_block_forward(xbn, lw["w_router"], lw["w_gate"], lw["w_up"], lw["w_down"],
                                  L.k, ws_gate=lw["ws_gate"], ws_up=lw["ws_up"],
                                  ws_down=lw["ws_down"], residual=xb, y=xb, topk_idx=ib, ws=wsb)
        torch.cuda.synchronize()
        mtouched += int(torch.unique(ib).numel())
    del xb, xbn, ib, wsb
    dwsb = bdm.workspace(bdm.bdm_denoise_workspace_bytes(TB, L.H, L.I, L.E, L.k, True), dev)
    tb = tb0.clone()
    bdm.bdm_denoise_block(tb, emb, stack, w_head, L.k, HS.mask_id, 0.95, max_steps=1, ws=dwsb,
                          block_tokens=L.T)
    mtimes = []
    for _ in range(3):
        tb.copy_(tb0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        bdm.bdm_denoise_block(tb, emb, stack, w_head, L.k, HS.mask_id, 0.95, max_steps=1,
                              ws=dwsb, block_tokens=L.T)
        mtimes.append(time.perf_counter() - t0)
    mms = 1e3 * float(np.median(mtimes))
    mbytes = (mtouched + nl) * EXPERT_BYTES + HEAD_BYTES
    del dwsb
    out = {"layers": nl, "ms": round(ms, 3), "block_tokens_per_s": round(L.T / (ms * 1e-3), 1),
           "touched_experts_all_layers": touched, "bytes": int(nbytes),
           "GB_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
           "frac_of_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           "gpu_ms": round(float(np.median(gtimes)), 3),
           "coreset_top_p_0.9": {"ms": round(cms, 3),
                                 "block_tokens_per_s": round(L.T / (cms * 1e-3), 1),
                                 "kept_experts_all_layers": kept, "bytes": int(cbytes),
                                 "GB_s": round(cbytes / (cms * 1e-3) / 1e9, 1),
                                 "frac_of_peak": round(cbytes / (cms * 1e-3) / 1e9
                                                       / PEAK_HBM_GBS, 4)},
           "16_blocks": {"slots": TB, "ms": round(mms, 3),
                         "block_tokens_per_s": round(TB / (mms * 1e-3), 1),
                         "touched_experts_all_layers": mtouched, "bytes": int(mbytes),
                         "GB_s": round(mbytes / (mms * 1e-3) / 1e9, 1),
                         "frac_of_peak": round(mbytes / (mms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                         "timing": "host wall clock, median of 3; commit rule per 32-slot block"},
           "block": "31 committed tokens (distinct seeded ids) + 1 masked slot",
           "timing": f"host wall clock of bdm_denoise_block(max_steps=1) (its per-step host "
                     f"read included), median of {reps}; gpu_ms: events on the stream around "
                     f"the call"}
    del stack, layers, emb, w_head
    torch.cuda.empty_cache()
    return out


def stack_embedding(torch, L, HS, dev):
    """The stack step's embedding table [V][H] bf16 (seeded, N(0,1))."""
    g = torch.Generator(device=dev)
    g.manual_seed(902)
    return torch.randn((HS.V, L.H), generator=g, device=dev).to(torch.bfloat16)


def stack_block(torch, L, HS, dev):
    """The stack step's block: late in its loop, 31 committed tokens (distinct
    seeded ids) and one masked slot, so the 32 rows differ (an all-masked
    block has 32 identical rows and touches only k experts per layer).
    Returns (the generator, for further draws; the block on `dev`)."""
    gt = torch.Generator(device="cpu")
    gt.manual_seed(903)
    ids = torch.randperm(HS.V - 1, generator=gt)[:L.T]
    ids = ids + (ids >= HS.mask_id).long()                  # never the mask id
    tok0 = ids.to(torch.int32).to(dev)
    tok0[L.T // 2] = HS.mask_id
    return gt, tok0


def stream_read_gbs(torch, dev, reps, nbytes=None):
    """Read bandwidth of a plain stream of the head's size (so that its fixed
    launch, ramp and tail costs weigh as much as the head's) with the weight
    kernels' access (16-byte non-temporal loads, libbdmcal.so), in two
    orders: a grid-stride loop of 1,024 workgroups, and one contiguous region
    per workgroup (256 and 512 workgroups, the persistent kernels' order).
    The best of them is the box's achievable ceiling for this path, measured
    beside it.  Returns (GB/s, pattern)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                   "block_diffusion_moe_amd", "libbdmcal.so"))
    sig = [ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    for f in (lib.bdmcal_stream_read, lib.bdmcal_stream_read_region):
        f.restype = ctypes.c_int
        f.argtypes = sig
    nbytes = (nbytes or HEAD_BYTES) // 16 * 16
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(2)]
    out = torch.empty(1024 * 256, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream().cuda_stream
    best = (0.0, "")
    unit = 256 * 4 * 16                         # a region workgroup's batch, bytes
    for name, fn, blocks, region in (
            ("grid-stride, 1024 workgroups", lib.bdmcal_stream_read, 1024, False),
            ("one region per workgroup, 256", lib.bdmcal_stream_read_region, 256, True),
            ("one region per workgroup, 512", lib.bdmcal_stream_read_region, 512, True)):
        def launch(b):
            if fn(b.data_ptr(), nbytes, out.data_ptr(), blocks, st) != 0:
                raise RuntimeError("stream read probe failed")
        for b in bufs:
            launch(b)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(reps):
            launch(bufs[i % 2])
        e1.record()
        torch.cuda.synchronize()
        # a region workgroup reads whole batches only (the remainder is not read)
        nread = (nbytes // blocks) // unit * unit * blocks if region else nbytes
        gbs = nread / (e0.elapsed_time(e1) * 1e-3 / reps) / 1e9
        if gbs > best[0]:
            best = (gbs, name)
    del bufs, out
    torch.cuda.empty_cache()
    return best


def _summary_records():
    try:
        with open(PMC_SUMMARY) as fh:
            txt = fh.read()
    except OSError:
        return {}
    vals = {}
    for ln in txt.splitlines():
        if ln.startswith("<!--") and "=" in ln:
            k, v = ln.strip("<!-> \n").split("=", 1)
            vals[k.strip()] = v.strip()
    return vals


def head_traffic():
    """HBM bytes per head GEMM launch from the committed counter summary
    (calibrated FETCH_SIZE + WRITE_SIZE), or None when the summary is missing or
    was taken on other kernel sources."""
    vals = _summary_records()
    from block_diffusion_moe_amd.traffic import kernel_source_digest
    if vals.get("source_sha256") != kernel_source_digest() or "traffic_bytes" not in vals:
        return None
    return int(float(vals["traffic_bytes"]))


def moe_layer_traffic():
    """HBM bytes of one one-block MoE layer (all its launches) from the same
    summary, or None when missing or taken on other kernel sources."""
    vals = _summary_records()
    from block_diffusion_moe_amd.traffic import MOE_SOURCES, kernel_source_digest
    if (vals.get("moe_source_sha256") != kernel_source_digest(MOE_SOURCES)
            or "moe_layer_traffic_bytes" not in vals):
        return None
    return int(float(vals["moe_layer_traffic_bytes"]))


def cpu_baseline(torch, dev, blocks, skew_host, stack_layers, runs=5):
    """The CPU oracle (as it stands: numpy float64, per-token loops) on the
    host cores, beside the GPU run, on the same seeded inputs.

    * Thread count: numpy's BLAS runs the oracle's products.  The MoE layer's
      are per-token matrix-vector products over one expert (512 x 2,048),
      too small for BLAS threads to pay off; the head's are a real GEMM
      (32 rows x 248,320 x 2,048).  Each is timed with BLAS limited to one
      thread and with every host core, and each phase then uses its faster
      setting.
    * The one-block MoE layer (Clover shape, 32 tokens) and the head + unmask
      (32 rows, 248,320-row head): one warm-up, then the median of `runs`
      timed runs (rotating over the weight sets) at each thread setting.
    * The load-skew batch (256 tokens, log-Zipf router offset): one warm-up,
      median of `runs`, at the MoE layer's faster setting.
    * One step of the 40-layer stack from the GPU stack step's block
      (embedding rows, 40 x (RMSNorm + MoE layer), final RMSNorm, head +
      unmask): each layer's weights regenerated on the device from its seed
      and its touched experts copied to the host before that layer is timed
      (copy time excluded).
    Weights are copied to the host before the timed regions.  `value` is the
    same step the GPU's `value` times (RMSNorm + MoE layer + head + unmask
    over one 32-slot block), each phase at its faster thread setting."""
    import numpy as np
    import synth
    from oracle import head as ohead, moe as omoe, norm as onorm
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:
        threadpool_limits = None
    ncpu = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass

    def limits(n):
        if threadpool_limits is None:
            import contextlib
            return contextlib.nullcontext()
        return threadpool_limits(limits=n, user_api="blas")

    def median_of(fn, n_sets):
        fn(0)                                            # warm-up
        ts = []
        for i in range(runs):
            t0 = time.perf_counter()
            fn(i % n_sets)
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts)), [round(t, 4) for t in ts]

    host = []
    for inp, w_head, blk in blocks:
        host.append((synth.moe_host(inp, lazy=False), synth.bf16_bits(inp.x),
                     synth.bf16_bits(w_head), blk.tokens.cpu().numpy()))
    nsets = len(host)
    print(f"[bench] cpu baseline: {ncpu} host cores ({model})", file=sys.stderr, flush=True)

    def layer(r):
        h, xb, _, _ = host[r]
        xn = onorm.rmsnorm(xb, 1e-6)
        return omoe.moe_block(xn, h["w_router"], h["w_gate"], h["w_up"], h["w_down"], h["k"],
                              h["ws_gate"], h["ws_up"], h["ws_down"], residual=xb)["y"]

    ys = [layer(r) for r in range(nsets)]               # each set's head input

    def head(r):
        _, _, wh, tok = host[r]
        ohead.head_unmask(ys[r], wh, tok, synth.HEAD.mask_id, 0.95)

    def skew(r):
        h = host[r][0]
        xb, bias = skew_host[r]
        omoe.moe_block(xb, h["w_router"], h["w_gate"], h["w_up"], h["w_down"], h["k"],
                       h["ws_gate"], h["ws_up"], h["ws_down"], bias=bias)

    per = {}
    for name, fn in (("moe_layer", layer), ("head_unmask", head)):
        per[name] = {}
        for n in sorted({1, ncpu}):
            with limits(n):
                med, ts = median_of(fn, nsets)
            per[name][f"{n}_threads"] = {"median_s": round(med, 4), "runs_s": ts}
            print(f"[bench] cpu {name} {n} thread(s): median {med:.3f} s", file=sys.stderr,
                  flush=True)
    best = {k: min(((int(t.split("_")[0]), v["median_s"]) for t, v in d.items()),
                   key=lambda a: a[1]) for k, d in per.items()}
    with limits(best["moe_layer"][0]):
        sk_med, sk_ts = median_of(skew, len(skew_host))
    print(f"[bench] cpu skew batch: median {sk_med:.3f} s", file=sys.stderr, flush=True)
    step_s = best["moe_layer"][1] + best["head_unmask"][1]
    out = {"value": round(32 / step_s, 4), "unit": "block-tokens/s",
           "cores": max(best["moe_layer"][0], best["head_unmask"][0]), "kind": "oracle",
           "host_cores": ncpu, "cpu_model": model,
           "sample": f"one 32-slot block step = the one-block MoE layer (median of {runs} runs "
                     f"after one warm-up, {best['moe_layer'][0]} BLAS thread(s)) + the head and "
                     f"unmask (median of {runs}, {best['head_unmask'][0]} BLAS thread(s)); "
                     f"numpy float64 oracle, weights copied to the host before the timed "
                     f"region",
           "threads_used": {"moe_layer": best["moe_layer"][0],
                            "head_unmask": best["head_unmask"][0]},
           "per_thread_setting": per,
           "moe_layer_block_tokens_per_s": round(32 / best["moe_layer"][1], 4),
           "head_unmask_positions_per_s": round(32 / best["head_unmask"][1], 4),
           "skew_8_blocks": {"median_s": round(sk_med, 4), "runs_s": sk_ts,
                             "block_tokens_per_s": round(256 / sk_med, 4),
                             "threads": best["moe_layer"][0]}}
    del host, ys
    if stack_layers > 0:
        out["stack_step"] = cpu_stack_step(torch, dev, stack_layers, best, limits)
    return out


def cpu_stack_step(torch, dev, nl, best, limits):
    """One step of the stack on the CPU oracle from the GPU stack step's
    block; per layer the weights are regenerated on the device from their
    seed and the layer's touched experts (the oracle's own routing, taken
    untimed first) copied to the host before the layer is timed."""
    import numpy as np
    import synth
    from oracle import head as ohead, moe as omoe, norm as onorm
    L, HS = synth.LAYER, synth.HEAD
    emb = stack_embedding(torch, L, HS, dev)
    _, tok0 = stack_block(torch, L, HS, dev)
    x = synth.bf16_bits(emb[tok0.long()].contiguous())
    tok = tok0.cpu().numpy()
    del emb
    t_layers = 0.0
    for l in range(nl):
        wr, wg, wu, wd, sg, su, sd, _ = synth.moe_weights(L, 100 + l, dev)
        wr_h = wr.cpu().numpy()
        xn = onorm.rmsnorm(x, 1e-6)
        idx = omoe.route(xn, wr_h, L.k)[0]               # untimed: which experts to copy
        touched = np.unique(idx)
        W = {n: {int(e): synth.bf16_bits(t[int(e)]) for e in touched}
             for n, t in (("g", wg), ("u", wu), ("d", wd))}
        shared = (synth.bf16_bits(sg), synth.bf16_bits(su), synth.bf16_bits(sd))
        del wg, wu, wd, sg, su, sd
        with limits(best["moe_layer"][0]):
            t0 = time.perf_counter()
            xn = onorm.rmsnorm(x, 1e-6)
            x = omoe.moe_block(xn, wr_h, W["g"], W["u"], W["d"], L.k, *shared, residual=x)["y"]
            t_layers += time.perf_counter() - t0
        del W, shared
        if (l + 1) % 10 == 0:
            print(f"[bench] cpu stack step: {l + 1} layers, {t_layers:.1f} s", file=sys.stderr,
                  flush=True)
    wh = synth.bf16_bits(synth.head_weights(HS, 0, device=dev))
    torch.cuda.empty_cache()
    with limits(best["head_unmask"][0]):
        t0 = time.perf_counter()
        h = onorm.rmsnorm(x, 1e-6)
        ohead.head_unmask(h, wh, tok, HS.mask_id, 0.95)
        t_head = time.perf_counter() - t0
    del wh
    return {"layers": nl, "s": round(t_layers + t_head, 3), "layers_s": round(t_layers, 3),
            "head_s": round(t_head, 3),
            "block_tokens_per_s": round(L.T / (t_layers + t_head), 4),
            "sample": f"one step (embedding rows, {nl} x (RMSNorm + MoE layer), final "
                      f"RMSNorm, head + unmask) of the GPU stack step's block, each phase at "
                      f"its faster thread setting; touched experts copied to the host untimed"}


if __name__ == "__main__":
    main()
