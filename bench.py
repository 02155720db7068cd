#!/usr/bin/env python3
"""Benchmark of the gated-delta SSM layer core on one MI355X.

One timed step = one decode step of the whole layer core on the batched-decode
workload (64 sequences x 48 value heads, 128x128 fp32 state per head,
conv 10240 channels read from 20480-wide rows): conv1d + SiLU + L2 -> decay
gate -> recurrence -> gated RMSNorm in one launch (gdn_decode_step, whose
results are bit-identical to the separate entry points).  The same step as
four separate launches and as conv + gdn_decode_fused is timed beside it.
Inputs are resident in HBM before the timed region.  The state and conv
history live in one of several pools, rotated step by step, so the 192 MiB
state cannot stay in the 256 MB MALL between steps ("cold"); a same-pool
("MALL-hot") figure of the recurrence is reported beside it.

value = decode state GB/s of the whole step: (state bytes read + written) /
step time.  The prefill half of the metric (tokens/s of the 4096-token prompt
through gate, conv, chunked recurrence and norm) is timed in the same run and
reported under "prefill": as gdn_prefill_chunked (gate and conv inside the
chunked recurrence's first phase) + gdn_gated_rmsnorm, and as four launches.

Prints ONE JSON line.  --gpus N > 1 is refused: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
FP32_MATRIX_PEAK_TFLOPS = 157.3


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--pools", type=int, default=4, help="state pools rotated for cold timing")
    p.add_argument("--prefill-iters", type=int, default=10)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--burst-launches", type=int, default=50,
                   help="launches per back-to-back burst")
    p.add_argument("--burst-reps", type=int, default=10, help="bursts per figure (median)")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="run one device-to-device copy of this many MiB first (counter calibration)")
    return p.parse_args()


def decode_bytes(wl) -> dict:
    """Algorithmic HBM bytes of one decode step, per kernel (fp32 = 4 B)."""
    n, T, H, Hk, S, C, D = wl.n_seq, wl.n_tok, wl.H, wl.Hk, wl.S, wl.conv_dim, wl.d_conv
    state = n * H * S * S * 4
    recur = 2 * state + n * T * (2 * Hk * S + 2 * H * S + 2 * H) * 4
    conv = n * (2 * C * (D - 1) + T * 2 * C) * 4 + C * D * 4
    norm = n * T * 3 * H * wl.head_dim * 4 + wl.head_dim * 4
    gate = n * T * H * 2 * 4 + 2 * H * 4
    # the one-launch step: q, k, v, y and g stay on chip; z is read, out written
    step = (2 * state + conv - n * T * C * 4 + n * T * 2 * H * S * 4 + wl.head_dim * 4
            + n * T * H * 2 * 4 + 2 * H * 4)
    return {"state": 2 * state, "recurrence": recur, "conv": conv, "norm": norm, "gate": gate,
            "step": step}


def recorded_traffic(profile: str):
    """HBM bytes per launch measured by the FETCH_SIZE / WRITE_SIZE counter runs
    summarised in `profile`, or None when the kernel sources named there have
    changed since (their hash no longer matches) or the file is missing."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", profile)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", "|", "`")):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    try:
        h = hashlib.sha256()
        for f in kv["source_files"].split():
            h.update(open(os.path.join(root, f), "rb").read())
        if h.hexdigest()[:16] != kv["source_sha256_16"]:
            return None
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


def chunked_flops(T: int, H: int, S: int, C: int = 64) -> float:
    """Algorithmic flops of the chunked recurrence, per token-head 10*C*S + 6*S^2
    (2 flops a multiply-add; per chunk of C positions: K K^T and Q K^T on their
    lower halves, W, Ut, the intra-chunk output and its correction 2 C^2 S each;
    the three products with the state 2 C S^2 each).  The kernels form y as
    e^G Q S + M U, one C^2 S product fewer (8*C*S + 6*S^2); the figure is kept
    as the method's count so that rates stay comparable."""
    return float(T) * H * (10 * C * S + 6 * S * S)


# MFMA instructions the S = 128 chunked kernels issue per (sequence, head,
# 64-position chunk), counted from the kernels' code:
#   phase A, 16x16x32 bf16 (16384 flops each): K K^T and Q K^T on 20 lower
#     tiles x 4 k-steps x 3 (hi/lo split) = 240; W and U~: 8 waves x 2 k-steps
#     x 2 key tiles x 2 token tiles x 2 products x 3 = 384;
#   phase A, 16x16x4 fp32 (2048 flops each): the block inverse, 64;
#   phase B, 16x16x32 fp16 (16384 flops each) per 16-column value tile: 8 waves
#     x 4 k-steps x 2 (state hi/lo) = 64 for W S / Q S, 8 waves x 2 k-steps x 3
#     (U hi/lo, K hi/lo) = 48 for the state update, and 3 + 3 + 6 + 6 = 18 for
#     M U (U hi/lo, M hi/lo; token tiles 0 and 1 have one position k-step);
#     8 value tiles per head.
MFMA_FLOPS_PER_HEAD_CHUNK = (240 + 384) * 16384 + 64 * 2048 + 8 * (64 + 48 + 18) * 16384


def chunked_executed_flops(n_tok: int, H: int, n_seq: int = 1) -> float:
    """Flops of the MFMA instructions one chunked call issues (chunk count
    padded to even, as the kernels do)."""
    chunks = ((n_tok + 63) // 64 + 1) & ~1
    return float(n_seq) * H * chunks * MFMA_FLOPS_PER_HEAD_CHUNK


def chunked_attainable(T: int, H: int, Hk: int, S: int, ws_bytes: int, tflops: float) -> dict:
    """Roofline-attainable bf16 MFMA fraction of the chunked recurrence: its
    algorithmic flops over its HBM bytes give the arithmetic intensity, and
    min(peak, AI x 8 TB/s) / peak bounds the fraction any schedule reaches.
    Two byte counts: the path's own I/O (q, k read once, v read, y written, g,
    beta, state in and out) and that plus this two-pass design's workspace
    (written once by phase A, read back by phase B)."""
    fl = chunked_flops(T, H, S)
    io = (2 * T * Hk * S + 2 * T * H * S + 2 * T * H + 2 * H * S * S) * 4
    out = {}
    for name, b in (("single_pass_io", io), ("with_workspace_round_trip", io + 2 * ws_bytes)):
        ai = fl / b
        att = min(BF16_PEAK_TFLOPS, ai * HBM_PEAK_GBS / 1e3)
        out[name] = {"bytes": b, "flop_per_byte": ai, "attainable_tflops": att,
                     "attainable_frac_of_bf16_peak": att / BF16_PEAK_TFLOPS,
                     "measured_frac_of_attainable": tflops / att}
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: the gated-delta core has no cross-GPU "
              "step in this build (--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_delta_ssm_amd as gdn
    from gdn_inputs import WORKLOADS, Workload, make_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    if args.copy_probe_mib:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters give the
        # scale factor between counter readings and bytes moved
        n = args.copy_probe_mib * 2 ** 20 // 4
        src = torch.ones(n, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---------------------------------------------------------------- decode step
    wl = WORKLOADS["decode64"]
    inp = make_inputs(wl)
    cu = {k: v.to(dev) for k, v in inp.items() if isinstance(v, torch.Tensor)}
    n, H, Hk, S, C = wl.n_seq, wl.H, wl.Hk, wl.S, wl.conv_dim
    pools = [cu["state"].clone() for _ in range(args.pools)]
    hists = [cu["conv_hist"].clone() for _ in range(args.pools)]
    x = cu["x"][:, :, :C]                                   # rows 20480 apart
    conv_out = torch.empty(n, 1, C, device=dev)            # rows 10240 apart
    g = torch.empty(n, H, device=dev)
    y = torch.empty(n, 1, H, S, device=dev)
    nout = torch.empty(n, H, S, device=dev)
    qv = conv_out[:, :, :Hk * S].unflatten(-1, (Hk, S))
    kv = conv_out[:, :, Hk * S:2 * Hk * S].unflatten(-1, (Hk, S))
    vv = conv_out[:, :, 2 * Hk * S:].unflatten(-1, (H, S))
    z = cu["z"]                                             # [n][H][S]

    rec_ev = []

    def decode_step(i, timed=False):
        p = i % len(pools)
        gdn.gdn_decay_gate(cu["alpha"], cu["dt"], cu["a"], g)
        gdn.gdn_conv1d_silu_l2norm(x, cu["conv_w"], hists[p], conv_out,
                                   qk_channels=wl.qk_channels, head_dim=wl.head_dim,
                                   l2_eps=wl.l2_eps)
        if timed:
            e0 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        gdn.gdn_recurrence_decode(pools[p], qv, kv, vv, g.view(n, 1, H), cu["beta"], y,
                                  scale=wl.scale)
        if timed:
            e1 = torch.cuda.Event(enable_timing=True)
            e1.record(stream)
            rec_ev.append((e0, e1))
        gdn.gdn_gated_rmsnorm(y.view(n, H, S), cu["norm_w"], z, nout, eps=wl.norm_eps)

    def decode_step_fused(i):
        # the same step with gate, recurrence and norm in one launch
        p = i % len(pools)
        gdn.gdn_conv1d_silu_l2norm(x, cu["conv_w"], hists[p], conv_out,
                                   qk_channels=wl.qk_channels, head_dim=wl.head_dim,
                                   l2_eps=wl.l2_eps)
        gdn.gdn_decode_fused(pools[p], qv, kv, vv, cu["alpha"].view(n, 1, H), cu["dt"], cu["a"],
                             cu["beta"], cu["norm_w"], z.view(n, 1, H, S), nout.view(n, 1, H, S),
                             scale=wl.scale, norm_eps=wl.norm_eps)

    step_ws = torch.zeros(gdn.gdn_decode_step_workspace_bytes(n, Hk) // 4, dtype=torch.int32,
                          device=dev)

    def decode_step_one(i):
        # the whole step (conv, gate, recurrence, norm) in one launch
        p = i % len(pools)
        gdn.gdn_decode_step(pools[p], x, cu["conv_w"], hists[p], cu["alpha"].view(n, 1, H),
                            cu["dt"], cu["a"], cu["beta"], cu["norm_w"], z.view(n, 1, H, S),
                            nout.view(n, 1, H, S), scale=wl.scale, l2_eps=wl.l2_eps,
                            norm_eps=wl.norm_eps, workspace=step_ws)

    def time_steps(step):
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps

    fused_ms_per_step = time_steps(decode_step_fused)
    four_ms_per_step = time_steps(decode_step)

    for i in range(args.warmup):
        decode_step_one(i)
    torch.cuda.synchronize()
    # timed region: K whole steps, nothing else on the stream
    t0 = time.perf_counter()
    for i in range(args.steps):
        decode_step_one(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    # the same K steps again with HIP events around each recurrence launch (an
    # event pair adds about 5 us of dispatch gap on each side of the kernel,
    # so it is kept out of the timed region above)
    for i in range(args.steps):
        decode_step(i, timed=True)
    torch.cuda.synchronize()
    rec_ms = float(np.mean([a.elapsed_time(b) for a, b in rec_ev]))
    by = decode_bytes(wl)
    value = by["state"] / (ms_per_step * 1e-3) / 1e9

    # same-pool repeat: the state may stay in the MALL between launches
    hot_ev = []
    for i in range(args.warmup):
        gdn.gdn_recurrence_decode(pools[0], qv, kv, vv, g.view(n, 1, H), cu["beta"], y,
                                  scale=wl.scale)
    for i in range(args.steps):
        e0 = torch.cuda.Event(enable_timing=True); e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        gdn.gdn_recurrence_decode(pools[0], qv, kv, vv, g.view(n, 1, H), cu["beta"], y,
                                  scale=wl.scale)
        e1.record(stream)
        hot_ev.append((e0, e1))
    torch.cuda.synchronize()
    hot_ms = float(np.mean([a.elapsed_time(b) for a, b in hot_ev]))

    # back-to-back bursts: events around 50 launches, 10 bursts, median per launch
    def burst(launch, n_launch=args.burst_launches, reps=args.burst_reps):
        launch(0)
        torch.cuda.synchronize()
        per = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True); b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for i in range(n_launch):
                launch(i)
            b.record(stream)
            b.synchronize()
            per.append(a.elapsed_time(b) / n_launch)
        return float(np.median(per))

    bursts = {
        "step_one_launch_rotated": burst(decode_step_one),
        "recurrence_rotated_pools": burst(lambda i: gdn.gdn_recurrence_decode(
            pools[i % len(pools)], qv, kv, vv, g.view(n, 1, H), cu["beta"], y, scale=wl.scale)),
        "conv_step_rotated_hist": burst(lambda i: gdn.gdn_conv1d_silu_l2norm(
            x, cu["conv_w"], hists[i % len(hists)], conv_out, qk_channels=wl.qk_channels,
            head_dim=wl.head_dim, l2_eps=wl.l2_eps)),
        "norm": burst(lambda i: gdn.gdn_gated_rmsnorm(y.view(n, H, S), cu["norm_w"], z, nout,
                                                       eps=wl.norm_eps)),
        "gate": burst(lambda i: gdn.gdn_decay_gate(cu["alpha"], cu["dt"], cu["a"], g)),
    }
    del pools, hists
    torch.cuda.empty_cache()

    # achievable copy bandwidth: torch's device copy of the state's size (read +
    # write = the recurrence's state bytes), sources rotated like the state pools
    srcs = [torch.ones(n * H * S * S, device=dev) for _ in range(args.pools)]
    dst = torch.empty_like(srcs[0])
    torch_copy_ms = burst(lambda i: dst.copy_(srcs[i % len(srcs)]))
    # the library's non-temporal streaming copy: the state stream's access
    # pattern without its arithmetic
    copy_ms = burst(lambda i: gdn.gdn_stream_copy(dst, srcs[i % len(srcs)]))
    copy_gbs = by["state"] / (copy_ms * 1e-3) / 1e9
    # roofline of the timed step's one kernel: its launches back to back on
    # rotated (cold) state pools and histories, HIP events around 50 launches
    # on the launch stream
    burst_ms = bursts["step_one_launch_rotated"]
    achieved = by["step"] / (burst_ms * 1e-3) / 1e9
    rec_burst_gbs = by["recurrence"] / (bursts["recurrence_rotated_pools"] * 1e-3) / 1e9
    del srcs, dst
    torch.cuda.empty_cache()

    # launch-bound regime: one sequence x 32 heads, where the fused entry point
    # (gate + recurrence + norm in one launch) replaces three launches
    sw = WORKLOADS["decode"]
    si = make_inputs(sw)
    sc = {k: v.to(dev) for k, v in si.items() if isinstance(v, torch.Tensor)}
    sn, sT, sH, sS = sw.n_seq, sw.n_tok, sw.H, sw.S
    s_st = sc["state"].clone()
    s_g = torch.empty(sn * sT, sH, device=dev)
    s_y = torch.empty(sn, sT, sH, sS, device=dev)
    s_o = torch.empty(sn * sT, sH, sS, device=dev)

    def small_three(i):
        gdn.gdn_decay_gate(sc["alpha"], sc["dt"], sc["a"], s_g)
        gdn.gdn_recurrence_decode(s_st, sc["q"], sc["k"], sc["v"], s_g.view(sn, sT, sH),
                                  sc["beta"], s_y, scale=sw.scale)
        gdn.gdn_gated_rmsnorm(s_y.view(sn * sT, sH, sS), sc["norm_w"], sc["z"], s_o,
                              eps=sw.norm_eps)

    def small_fused(i):
        gdn.gdn_decode_fused(s_st, sc["q"], sc["k"], sc["v"], sc["alpha"].view(sn, sT, sH),
                             sc["dt"], sc["a"], sc["beta"], sc["norm_w"],
                             sc["z"].view(sn, sT, sH, sS), s_o.view(sn, sT, sH, sS),
                             scale=sw.scale, norm_eps=sw.norm_eps)

    # the whole one-sequence step (gate, conv, recurrence, norm), eager and
    # replayed from a HIP graph captured once (the launches then cost no host time)
    s_hist = sc["conv_hist"].clone()
    s_conv = torch.empty(sn, sT, sw.conv_dim, device=dev)
    s_q = s_conv[..., :sw.Hk * sS].unflatten(-1, (sw.Hk, sS))
    s_k = s_conv[..., sw.Hk * sS:2 * sw.Hk * sS].unflatten(-1, (sw.Hk, sS))
    s_v = s_conv[..., 2 * sw.Hk * sS:].unflatten(-1, (sH, sS))

    def small_step(i=0):
        gdn.gdn_decay_gate(sc["alpha"], sc["dt"], sc["a"], s_g)
        gdn.gdn_conv1d_silu_l2norm(sc["x"][..., :sw.conv_dim], sc["conv_w"], s_hist, s_conv,
                                   qk_channels=sw.qk_channels, head_dim=sw.head_dim,
                                   l2_eps=sw.l2_eps)
        gdn.gdn_recurrence_decode(s_st, s_q, s_k, s_v, s_g.view(sn, sT, sH), sc["beta"], s_y,
                                  scale=sw.scale)
        gdn.gdn_gated_rmsnorm(s_y.view(sn * sT, sH, sS), sc["norm_w"], sc["z"], s_o,
                              eps=sw.norm_eps)

    step_eager = burst(small_step)
    s_ws = torch.zeros(gdn.gdn_decode_step_workspace_bytes(sn, sw.Hk) // 4, dtype=torch.int32,
                       device=dev)

    def small_step_one(i=0):
        gdn.gdn_decode_step(s_st, sc["x"][..., :sw.conv_dim], sc["conv_w"], s_hist,
                            sc["alpha"].view(sn, sT, sH), sc["dt"], sc["a"], sc["beta"],
                            sc["norm_w"], sc["z"].view(sn, sT, sH, sS),
                            s_o.view(sn, sT, sH, sS), scale=sw.scale, l2_eps=sw.l2_eps,
                            norm_eps=sw.norm_eps, workspace=s_ws)

    step_one = burst(small_step_one)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        small_step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        small_step()
    step_graph = burst(lambda i: graph.replay())
    small = {"workload": "decode: 1 seq x 1 token, 32 value / 16 q-k heads, 128x128 state",
             "three_calls_ms": burst(small_three), "fused_ms": burst(small_fused),
             "step_eager_ms": step_eager, "step_graph_replay_ms": step_graph,
             "step_one_launch_ms": step_one}
    del graph, s_st, s_g, s_y, s_o, sc, s_hist, s_conv

    # ---------------------------------------------------------------- K-position verify
    # 16 sequences x K draft positions in one gdn_decode_step launch, with the
    # state and conv-history snapshots after every position but the last
    # written inline (K = 2 is the headline verify; 4 and 8 show the generic K)
    def verify_case(K, pools=6):
        # cold: `pools` disjoint sets of state, snapshots, conv history and
        # output rotated launch by launch (at K = 2 each set holds 64 MiB of
        # state and snapshots, six of them 384 MiB, beyond the 256 MB MALL);
        # MALL-hot: the same launch repeated on one set
        vw_ = WORKLOADS["verify2"]
        if K != vw_.n_tok:
            vw_ = Workload(**{**vw_.__dict__, "name": f"verify{K}", "n_tok": K})
        vi_ = make_inputs(vw_)
        vc = {k: v.to(dev) for k, v in vi_.items() if isinstance(v, torch.Tensor)}
        vn, vT, vH, vS, vC = vw_.n_seq, vw_.n_tok, vw_.H, vw_.S, vw_.conv_dim
        sets = []
        for _ in range(pools):
            sets.append(dict(st=vc["state"].clone(), hist=vc["conv_hist"].clone(),
                             out=torch.empty(vn, vT, vH, vS, device=dev),
                             snap=torch.empty(vn, vT - 1, vH, vS, vS, device=dev),
                             csnap=torch.empty(vn, vT - 1, vC, vw_.d_conv - 1, device=dev)))
        v_ws = torch.zeros(gdn.gdn_decode_step_workspace_bytes(vn, vw_.Hk) // 4,
                           dtype=torch.int32, device=dev)

        def verify_step(i=0, rotate=True):
            b = sets[i % pools] if rotate else sets[0]
            gdn.gdn_decode_step(b["st"], vc["x"][..., :vC], vc["conv_w"], b["hist"],
                                vc["alpha"].view(vn, vT, vH), vc["dt"], vc["a"], vc["beta"],
                                vc["norm_w"], vc["z"].view(vn, vT, vH, vS), b["out"],
                                scale=vw_.scale, l2_eps=vw_.l2_eps, norm_eps=vw_.norm_eps,
                                workspace=v_ws, snap=b["snap"], conv_snap=b["csnap"])
        cold_ms = burst(verify_step)
        hot_ms = burst(lambda i: verify_step(i, rotate=False))
        v_state_bytes = vn * vH * vS * vS * 4
        per_set = (K + 1) * v_state_bytes // 2 ** 20
        del sets
        return {"workload": f"verify{K}: 16 seq x {K} positions, 32 value / 16 q-k heads, "
                            "128x128 state, conv 8192 ch, state and conv-history snapshots "
                            "after every position but the last, one gdn_decode_step launch",
                "ms": cold_ms,
                "state_GBs": (K + 1) * v_state_bytes / (cold_ms * 1e-3) / 1e9,
                "cold_note": f"{pools} buffer sets rotated launch by launch (state + snapshots "
                             f"{per_set} MiB per set, {pools * per_set} MiB in all, beyond the "
                             "256 MB MALL)",
                "ms_mall_hot": hot_ms,
                "state_GBs_mall_hot": (K + 1) * v_state_bytes / (hot_ms * 1e-3) / 1e9,
                "hot_note": "the same buffers every launch: the state can stay in the MALL",
                "state_bytes_note": f"state read + final write + {K - 1} snapshot write(s)"}
    verify = verify_case(2)
    verify_more = {str(K): verify_case(K) for K in (4, 8)}

    # ---------------------------------------------------------------- prefill pass
    pw = WORKLOADS["prefill"]
    pin = make_inputs(pw)
    pc = {k: v.to(dev) for k, v in pin.items() if isinstance(v, torch.Tensor)}
    T, PH, PHk, PS, PC = pw.n_tok, pw.H, pw.Hk, pw.S, pw.conv_dim
    pg = torch.empty(T, PH, device=dev)
    pout = torch.empty(1, T, PC, device=dev)
    pst = torch.empty(1, PH, PS, PS, device=dev)
    phist = torch.empty_like(pc["conv_hist"])
    py = torch.empty(1, T, PH, PS, device=dev)
    pn = torch.empty(T, PH, PS, device=dev)
    pq = pout[:, :, :PHk * PS].unflatten(-1, (PHk, PS))
    pk = pout[:, :, PHk * PS:2 * PHk * PS].unflatten(-1, (PHk, PS))
    pv = pout[:, :, 2 * PHk * PS:].unflatten(-1, (PH, PS))
    ws = torch.empty(max(gdn.gdn_recurrence_chunked_workspace_bytes(1, T, PH, PHk, PS, 64), 1),
                     dtype=torch.uint8, device=dev)
    prefill = None
    ev = {}

    def prefill_pass(timed=False):
        pst.zero_()
        phist.copy_(pc["conv_hist"])
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(5)] if timed else None
        if timed: marks[0].record(stream)
        gdn.gdn_decay_gate(pc["alpha"], pc["dt"], pc["a"], pg)
        if timed: marks[1].record(stream)
        gdn.gdn_conv1d_silu_l2norm(pc["x"], pc["conv_w"], phist, pout,
                                   qk_channels=pw.qk_channels, head_dim=pw.head_dim,
                                   l2_eps=pw.l2_eps)
        if timed: marks[2].record(stream)
        gdn.gdn_recurrence_chunked(pst, pq, pk, pv, pg.view(1, T, PH), pc["beta"], py,
                                   scale=pw.scale, workspace=ws)
        if timed: marks[3].record(stream)
        gdn.gdn_gated_rmsnorm(py.view(T, PH, PS), pc["norm_w"], pc["z"], pn, eps=pw.norm_eps)
        if timed:
            marks[4].record(stream)
            ev.setdefault("marks", []).append(marks)

    def prefill_fused_launches():
        gdn.gdn_prefill_chunked(pst, pc["x"], pc["conv_w"], phist, pc["alpha"].view(1, T, PH),
                                pc["dt"], pc["a"], pc["beta"], py, scale=pw.scale,
                                l2_eps=pw.l2_eps, workspace=ws)
        gdn.gdn_gated_rmsnorm(py.view(T, PH, PS), pc["norm_w"], pc["z"], pn, eps=pw.norm_eps)

    def prefill_launches():
        gdn.gdn_decay_gate(pc["alpha"], pc["dt"], pc["a"], pg)
        gdn.gdn_conv1d_silu_l2norm(pc["x"], pc["conv_w"], phist, pout,
                                   qk_channels=pw.qk_channels, head_dim=pw.head_dim,
                                   l2_eps=pw.l2_eps)
        gdn.gdn_recurrence_chunked(pst, pq, pk, pv, pg.view(1, T, PH), pc["beta"], py,
                                   scale=pw.scale, workspace=ws)
        gdn.gdn_gated_rmsnorm(py.view(T, PH, PS), pc["norm_w"], pc["z"], pn, eps=pw.norm_eps)

    try:
        for _ in range(2):
            prefill_pass()
        torch.cuda.synchronize()
        # whole passes back to back between one event pair: the four launches
        # of every pass, with no event between them (the state and history
        # carry from pass to pass, which changes no kernel's work)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.prefill_iters):
            prefill_launches()
        e1.record(stream)
        e1.synchronize()
        pass_ms = e0.elapsed_time(e1) / args.prefill_iters
        # the same pass as gdn_prefill_chunked + norm (two launches)
        for _ in range(2):
            prefill_fused_launches()
        e0.record(stream)
        for _ in range(args.prefill_iters):
            prefill_fused_launches()
        e1.record(stream)
        e1.synchronize()
        fused_pass_ms = e0.elapsed_time(e1) / args.prefill_iters
        # the fused call alone (gate + conv + chunked recurrence)
        e0.record(stream)
        for _ in range(args.prefill_iters):
            gdn.gdn_prefill_chunked(pst, pc["x"], pc["conv_w"], phist, pc["alpha"].view(1, T, PH),
                                    pc["dt"], pc["a"], pc["beta"], py, scale=pw.scale,
                                    l2_eps=pw.l2_eps, workspace=ws)
        e1.record(stream)
        e1.synchronize()
        fused_call_ms = e0.elapsed_time(e1) / args.prefill_iters
        # the chunked call alone, back to back between one event pair
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(args.prefill_iters):
            gdn.gdn_recurrence_chunked(pst, pq, pk, pv, pg.view(1, T, PH), pc["beta"], py,
                                       scale=pw.scale, workspace=ws)
        c1.record(stream)
        c1.synchronize()
        chunk_call_ms = c0.elapsed_time(c1) / args.prefill_iters
        # per-op split: a second, instrumented run with events between launches
        for _ in range(args.prefill_iters):
            prefill_pass(timed=True)
        torch.cuda.synchronize()
        seg = np.array([[m[j].elapsed_time(m[j + 1]) for j in range(4)] for m in ev["marks"]])
        seg = seg.mean(axis=0)                           # ms: gate, conv, chunked, norm
        fl = chunked_flops(T, PH, PS)
        xfl = chunked_executed_flops(T, PH)
        prefill = {
            "workload": "prefill: 1 seq x 4096 tokens, 32 value / 16 q-k heads, 128x128 state, "
                        "conv 8192 ch, chunk 64",
            "tokens_per_s": T / (min(pass_ms, fused_pass_ms) * 1e-3),
            "pass_ms": min(pass_ms, fused_pass_ms),
            "pass_note": "the faster of the two forms of the layer pass below",
            "fused_pass_ms": fused_pass_ms,
            "fused_pass_tokens_per_s": T / (fused_pass_ms * 1e-3),
            "fused_pass_note": f"{args.prefill_iters} passes of gdn_prefill_chunked + "
                               "gdn_gated_rmsnorm back to back between one event pair",
            "fused_call_ms": fused_call_ms,
            "fused_call_note": "gdn_prefill_chunked alone: decay gate, conv1d + SiLU + L2 and "
                               "the chunked recurrence in two launches",
            "four_launch_pass_ms": pass_ms,
            "four_launch_pass_tokens_per_s": T / (pass_ms * 1e-3),
            "recurrence_tokens_per_s": T / (seg[2] * 1e-3),
            "chunked_call_ms": chunk_call_ms,
            "chunked_call_tokens_per_s": T / (chunk_call_ms * 1e-3),
            "chunked_call_note": f"{args.prefill_iters} gdn_recurrence_chunked calls back to "
                                 "back between one event pair (phase A and the scan)",
            "ms": {"gate": seg[0], "conv": seg[1], "chunked_recurrence": seg[2], "norm": seg[3]},
            "ms_note": "per-op split from a separate pass with events between launches; each "
                       "segment then carries the event pair's dispatch gaps, so the segments "
                       "sum to more than pass_ms",
            "chunked_algorithmic_tflops": fl / (seg[2] * 1e-3) / 1e12,
            "chunked_frac_of_bf16_peak": fl / (seg[2] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "chunked_executed_mfma_tflops": xfl / (seg[2] * 1e-3) / 1e12,
            "chunked_executed_frac_of_bf16_peak": xfl / (seg[2] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "chunked_fp32_equivalent_frac": fl / (seg[2] * 1e-3) / 1e12 / FP32_MATRIX_PEAK_TFLOPS,
            "chunked_peak_note": "frac_of_bf16_peak: algorithmic flops (one product each) over "
                                 "the dense bf16 MFMA peak (the fp16 MFMA peak is the same); "
                                 "executed: the flops of the MFMA instructions the kernels issue "
                                 "(bf16 hi/lo splits in phase A, fp16 with hi/lo state, U, K and M "
                                 "in phase B, fp32 16x16x4 in the block inverse), counted from the "
                                 "code; fp32_equivalent_frac divides the algorithmic rate by the "
                                 "fp32 matrix peak of an instruction the kernels do not issue, "
                                 "for comparison with an fp32 formulation only",
            "chunked_attainable": chunked_attainable(T, PH, PHk, PS, ws.numel(),
                                                     fl / (seg[2] * 1e-3) / 1e12),
        }
    except gdn.GdnError as e:
        prefill = {"error": str(e)}

    # ------------------------------------------------- packed batch of prompts (varlen)
    # eight prompts of different lengths in one chunked call, each from its own
    # state: the recurrence's throughput at batch > 1
    try:
        lens = [4096, 3000, 2048, 1500, 1024, 700, 300, 100]
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(int).tolist()
        total, n_p = cu[-1], len(lens)
        vin = make_inputs(pw, seed=5, n_tok=total, n_seq=1)
        vq = vin["q"][0].to(dev)
        vk = vin["k"][0].to(dev)
        vv = vin["v"][0].to(dev)
        vbeta = vin["beta"][0].to(dev)
        vg = torch.empty(total, PH, device=dev)
        gdn.gdn_decay_gate(vin["alpha"].to(dev), vin["dt"].to(dev), vin["a"].to(dev), vg)
        vst = torch.zeros(n_p, PH, PS, PS, device=dev)
        vy = torch.empty(total, PH, PS, device=dev)
        vws = torch.empty(max(gdn.gdn_recurrence_chunked_varlen_workspace_bytes(
            n_p, total, PH, PHk, PS, 64), 1), dtype=torch.uint8, device=dev)

        def varlen_call():
            gdn.gdn_recurrence_chunked_varlen(vst, vq, vk, vv, vg, vbeta, vy, cu,
                                              scale=pw.scale, workspace=vws)
        for _ in range(2):
            varlen_call()
        torch.cuda.synchronize()
        v0 = torch.cuda.Event(enable_timing=True)
        v1 = torch.cuda.Event(enable_timing=True)
        v0.record(stream)
        for _ in range(args.prefill_iters):
            varlen_call()
        v1.record(stream)
        v1.synchronize()
        vms = v0.elapsed_time(v1) / args.prefill_iters
        vfl = sum(chunked_flops(n, PH, PS) for n in lens)
        prefill_varlen = {
            "workload": f"{n_p} prompts of {lens} positions ({total} in all), 32 value / 16 q-k "
                        "heads, 128x128 state each, one gdn_recurrence_chunked_varlen call",
            "ms": vms, "recurrence_tokens_per_s": total / (vms * 1e-3),
            "chunked_algorithmic_tflops": vfl / (vms * 1e-3) / 1e12,
            "chunked_executed_frac_of_bf16_peak":
                sum(chunked_executed_flops(n, PH) for n in lens) / (vms * 1e-3) / 1e12
                / BF16_PEAK_TFLOPS,
            "note": "the chunked recurrence only (gate, conv, norm are per-token kernels); "
                    f"{args.prefill_iters} calls back to back between one event pair"}
        del vq, vk, vv, vg, vbeta, vst, vy, vws
    except gdn.GdnError as e:
        prefill_varlen = {"error": str(e)}

    # ------------------------------------------------- Mamba-2 SSD chunked scan
    try:
        from gdn_inputs import make_mamba2_inputs
        mT, mH, mG, mP, mN = 4096, 32, 1, 64, 128
        mi = make_mamba2_inputs(1, mT, mH, mG, mP, mN, seed=7)
        mx, mB, mC, mdt = (mi[k].to(dev) for k in ("x", "B", "C", "dt_raw"))
        mAl, mD, mbias = (mi[k].to(dev) for k in ("A_log", "D", "dt_bias"))
        mst = torch.zeros(1, mH, mP, mN, device=dev)
        my = torch.empty_like(mx)
        mws = torch.empty(gdn.gdn_mamba2_ssd_workspace_bytes(1, mT, mH, mP, mN, 64),
                          dtype=torch.uint8, device=dev)

        def ssd_call():
            gdn.gdn_mamba2_ssd_chunked(mst, mx, mB, mC, mdt, mAl, mD, mbias, my,
                                       dt_min=mi["dt_min"], dt_max=mi["dt_max"], workspace=mws)
        for _ in range(2):
            ssd_call()
        torch.cuda.synchronize()
        m0 = torch.cuda.Event(enable_timing=True)
        m1 = torch.cuda.Event(enable_timing=True)
        m0.record(stream)
        for _ in range(args.prefill_iters):
            ssd_call()
        m1.record(stream)
        m1.synchronize()
        mms = m0.elapsed_time(m1) / args.prefill_iters
        nch = (mT + 63) // 64
        # multiply-adds per (head, chunk): C B^T 64x64x N, M x 64x64x P, state 64 x P x N,
        # inter-chunk output 64 x P x N
        ssd_flops = 2.0 * mH * nch * (64 * 64 * mN + 64 * 64 * mP + 2 * 64 * mP * mN)
        mamba2 = {
            "workload": f"Mamba-2 selective scan, 1 seq x {mT} tokens, {mH} heads x head_dim {mP}, "
                        f"state {mN}, {mG} group, chunk 64, fp32",
            "ms": mms, "tokens_per_s": mT / (mms * 1e-3),
            "algorithmic_tflops": ssd_flops / (mms * 1e-3) / 1e12,
            "frac_of_fp32_peak": ssd_flops / (mms * 1e-3) / 1e12 / FP32_MATRIX_PEAK_TFLOPS,
            "executed_bf16_frac": 3 * ssd_flops / (mms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "note": "three launches (chunk outputs and states, state link, inter-chunk "
                    "outputs); the products on bf16 MFMA with each fp32 operand split into hi "
                    "+ lo (three MFMAs per product), hence executed = 3 x algorithmic"}
        del mx, mB, mC, mdt, mst, my, mws
    except gdn.GdnError as e:
        mamba2 = {"error": str(e)}

    # ---------------------------------------------------------------- CPU baseline (oracle)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, inp, args.cpu_seconds)

    out = {
        "metric": "decode state GB/s (% HBM roof) + chunked-prefill tokens/s per GDN layer",
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "decode64: 64 seq x 1 token, 48 value / 16 q-k heads, 128x128 fp32 "
                        "state per head (192 MiB), conv 10240 ch from 20480-wide rows; "
                        "conv+gate+recurrence+norm per step in one launch (gdn_decode_step), "
                        "state pools and conv histories rotated (cold)",
            "state_pools": args.pools,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "k_decode_step",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": recorded_traffic("k_decode_step_decode64.md"),
            "bytes_per_launch": by["step"],
            "avg_launch_ms": burst_ms,
            "timing": "HIP events around 50 back-to-back launches on rotated state pools and "
                      "conv histories, median of 10 bursts",
        },
        "decode": {
            "recurrence_state_GBs_cold": by["state"] / (rec_ms * 1e-3) / 1e9,
            "recurrence_ms_cold": rec_ms,
            "recurrence_ms_cold_note": "events around each launch inside the step sequence "
                                       "(includes the event pair's dispatch gap)",
            "recurrence_ms_mall_hot": hot_ms,
            "recurrence_state_GBs_mall_hot": by["state"] / (hot_ms * 1e-3) / 1e9,
            "step_frac_of_hbm": value / HBM_PEAK_GBS,
            "four_launch_ms_per_step": four_ms_per_step,
            "four_launch_state_GBs": by["state"] / (four_ms_per_step * 1e-3) / 1e9,
            "four_launch_note": "gate, conv, recurrence, norm as four launches",
            "fused_ms_per_step": fused_ms_per_step,
            "fused_state_GBs": by["state"] / (fused_ms_per_step * 1e-3) / 1e9,
            "fused_note": "conv + gdn_decode_fused (two launches) per step",
            "step_bytes_per_launch": by["step"],
            "conv_bytes_in_step": by["conv"] - n * C * 4,
            "conv_note": "inside the one-launch step the conv's bytes stream at the step "
                         "kernel's rate (roofline.achieved); on its own the conv launch is "
                         "bound by its ramp and drain (burst_ms_per_launch.conv_step_rotated_hist)",
            "conv_alone_GBs": by["conv"] / (bursts["conv_step_rotated_hist"] * 1e-3) / 1e9,
            "small_batch_gate_recurrence_norm": small,
            "verify2_step": verify,
            "verify_k_steps": verify_more,
            "burst_ms_per_launch": bursts,
            "recurrence_burst_GBs": rec_burst_gbs,
            "copy_peak": {"what": "gdn_stream_copy (16-byte non-temporal loads and stores), "
                                  "192 MiB per launch, sources rotated, 50-launch bursts",
                          "ms": copy_ms, "GBs": copy_gbs, "frac_of_hbm": copy_gbs / HBM_PEAK_GBS,
                          "torch_copy_ms": torch_copy_ms,
                          "torch_copy_GBs": by["state"] / (torch_copy_ms * 1e-3) / 1e9},
            "recurrence_frac_of_copy_peak": rec_burst_gbs / copy_gbs,
            "step_frac_of_copy_peak": achieved / copy_gbs,
        },
        "prefill": prefill,
        "prefill_varlen": prefill_varlen,
        "mamba2_ssd": mamba2,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out, default=float))


def cpu_baseline(wl, inp, seconds: float) -> dict:
    """The fp64 oracle's decode step (gate, conv, sequential recurrence, norm) on
    the same decode64 inputs, repeated for about `seconds` of host time."""
    import numpy as np

    import oracle
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    n, H, S, C = wl.n_seq, wl.H, wl.S, wl.conv_dim
    x = inp["x"][:, :, :C]
    def step():
        g = oracle.decay_gate(inp["alpha"], inp["dt"], inp["a"])
        out, _, _ = oracle.conv1d_silu_l2norm(x, inp["conv_w"], inp["conv_hist"],
                                              wl.qk_channels, wl.head_dim, wl.l2_eps)
        Hk = wl.Hk
        q = out[:, :, :Hk * S].reshape(n, 1, Hk, S)
        k = out[:, :, Hk * S:2 * Hk * S].reshape(n, 1, Hk, S)
        v = out[:, :, 2 * Hk * S:].reshape(n, 1, H, S)
        y, _, _ = oracle.recurrence_seq(inp["state"], q, k, v, g.reshape(n, 1, H), inp["beta"],
                                        wl.scale)
        oracle.gated_rmsnorm(y.reshape(n, H, S), inp["norm_w"], inp["z"], wl.norm_eps)

    times = []
    t_end = time.perf_counter() + seconds
    while True:
        t0 = time.perf_counter()
        step()
        times.append(time.perf_counter() - t0)
        if time.perf_counter() > t_end and len(times) >= 3:
            break
    med = float(np.median(times))
    threads = oracle.max_threads()
    # the same step on one thread, fewer repetitions
    oracle.set_threads(1)
    one = []
    try:
        t_end = time.perf_counter() + seconds / 2
        while len(one) < 3 or time.perf_counter() < t_end:
            t0 = time.perf_counter()
            step()
            one.append(time.perf_counter() - t0)
    finally:
        oracle.set_threads(threads)
    model = next((l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo")
                  if l.startswith("model name")), "unknown")
    state_bytes = 2 * n * H * S * S * 4
    return {"value": state_bytes / med / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"whole decode64 step (gate, conv, sequential fp64 recurrence, norm), "
                      f"median of {len(times)} runs over ~{seconds:.0f} s; state bytes of the "
                      f"fp32 step divided by the oracle's time",
            "ms_per_step": med * 1e3,
            "one_thread": {"value": state_bytes / float(np.median(one)) / 1e9,
                           "ms_per_step": float(np.median(one)) * 1e3, "runs": len(one)},
            "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": model}


if __name__ == "__main__":
    main()
