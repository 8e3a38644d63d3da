"""Benchmark: one rank's share of a 128K-token causal attention layer through
both context-parallel schedules, on one MI355X.

A step is one pass of the whole hot path over resident synthetic inputs:

* ring share -- ``cp_ring_fwd`` for one rank of an 8-rank zigzag ring over
  q, k, v bf16 [131072, 32, 128] (16 chunks of 8192; the rank's two query
  chunks against all 8 KV blocks over 8 steps, masked blocks skipped,
  log-sum-exp merged);
* Ulysses share -- ``cp_seq_to_head`` of q [131072, 32, 128] and of k, v
  [131072, 8, 128] for one rank of 8, full-sequence causal attention of its
  4 query heads over its 1 KV head (``cp_attn_block_fwd``), and
  ``cp_head_to_seq`` of the float32 output back into the sequence layout.

Throughput is causal-adjusted FLOP: 4*D*Hq per visible (query, key) pair
with a diagonal chunk counted as half (the handbook's work model, section
"之字形切分"): 2^44 for each share.  The attention kernel's own rate is timed
with HIP events recorded by the library around every launch on the launch
stream; its fraction of the bf16 dense MFMA peak is the roofline figure.
The CPU oracle is timed on a bounded sample of the ring share's rows.

``--layout striped`` (or contiguous) times the ring share with that split
instead (striped: q, k, v permuted to striped order once, before timing);
``--part ring|ulysses|bwd|usp|usp_bwd`` times one share, the backward pass,
or one rank of the USP hybrid (8-way Ulysses x 2-way ring), forward or
backward; ``--part block`` the whole sequence as one causal block
(``cp_attn_block_fwd`` on [131072, 32, 128]); ``--part merge|repack`` times the bandwidth-bound kernels alone
(the log-sum-exp merges of a ring rank run as separate kernels, the Ulysses
repacks of a rank) in GB/s against the HBM peak.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--part both|ring|ulysses|bwd|usp|usp_bwd|merge|repack|block]
                    [--merge-in-place]
                    [--layout zigzag|striped|contiguous]
                    [--rank r]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

S, HQ, HKV_ULY, D, P = 131072, 32, 8, 128, 8
RING_RANK, ULY_RANK = 0, 0
PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 4096 FLOP/clk x 2.4 GHz, dense
PEAK_HBM_GBS = 8000.0
METRIC = "causal block-attn fwd TFLOP/s + % bf16 MFMA peak, S=128K H=32 D=128"


def ring_share_flop(S, H, D, P, layout="zigzag", rank=0):
    """Causal-adjusted FLOP of one ring rank, a diagonal block counted half:
    zigzag 2P chunk units of (S/2P)^2; striped P causal blocks of (S/P)^2,
    each half; contiguous rank r (r + 1/2) units of (S/P)^2."""
    if layout == "zigzag":
        C = S // (2 * P)
        return 4.0 * D * H * (2 * P) * C * C
    C = S // P
    if layout == "striped":
        return 4.0 * D * H * P * C * C / 2.0
    return 4.0 * D * H * (rank + 0.5) * C * C


def plan_flop(cp, S, H, D, P, layout, rank):
    """The same convention counted over the library's ring plan: 4*D*H per
    pair of real rows, FULL pairs whole, DIAG pairs half (exact for padded
    lengths too)."""
    units = 0.0
    for (_r, _t, _qc, _kc, _qo, _ko, lq, lk, kind) in cp.cp_ring_plan(S, P, layout, rank, True):
        units += lq * lk if kind == cp.CP_PAIR_FULL else (lq * lk / 2.0 if kind == cp.CP_PAIR_DIAG
                                                         else 0.0)
    return 4.0 * D * H * units


def plan_flop_exact(cp, S, H, D, P, layout, rank):
    """4*D*H per visible (q, k) pair counted exactly: a diagonal pair of
    lq query and lk key rows starting at the same position has
    sum_i min(i + 1, lk) visible pairs (C(C+1)/2 for C x C) instead of
    half.  None for the striped split, whose diagonal pairs sit at local
    offsets."""
    if layout == "striped":
        return None
    units = 0.0
    for (_r, _t, _qc, _kc, _qo, _ko, lq, lk, kind) in cp.cp_ring_plan(S, P, layout, rank, True):
        if kind == cp.CP_PAIR_FULL:
            units += lq * lk
        elif kind == cp.CP_PAIR_DIAG:
            m = min(lq, lk)
            units += m * (m + 1) / 2.0 + (lq - m) * lk
    return 4.0 * D * H * units


def ulysses_share_flop(S, H_local, D):
    """Full-sequence causal attention of H_local heads, diagonal counted half."""
    return 4.0 * D * H_local * S * S / 2.0


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "attn_bf16_128k_rank_share_hbm_traffic.md")
KERNEL_SOURCE = os.path.join(ROOT, "context_parallelism_cp_amd", "csrc", "attn_bf16.hip")
BWD_TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "attn_bwd_128k_rank_share_hbm_traffic.md")
BLOCK_TRAFFIC_PROFILE = os.path.join(ROOT, "profiles",
                                     "attn_bf16_128k_single_block_32h_hbm_traffic.md")
BWD_KERNEL_SOURCE = os.path.join(ROOT, "context_parallelism_cp_amd", "csrc", "bwd_bf16.hip")


def recorded_traffic(profile=TRAFFIC_PROFILE, source=KERNEL_SOURCE, workload=None):
    """HBM bytes per launch (or launch pair) from a committed FETCH_SIZE /
    WRITE_SIZE summary, or None when the kernel source changed since it was
    taken or the summary is of another workload (its ``workload_key`` line
    must equal ``workload``)."""
    import hashlib
    try:
        fields = {}
        with open(profile, encoding="utf-8") as f:
            for line in f:
                if ":" in line and not line.startswith(("|", "#", "`")):
                    key, _, val = line.partition(":")
                    fields[key.strip()] = val.strip()
        with open(source, "rb") as f:
            current = hashlib.sha256(f.read()).hexdigest()
        if fields.get("kernel_source_sha256") != current:
            return None
        if workload is None or fields.get("workload_key") != workload:
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def workload_key(part, layout, rank, seq, ring_p):
    """The bench workload a traffic summary belongs to."""
    return f"part={part} layout={layout} rank={rank} seq={seq} P={ring_p}"


def cpu_baseline(q, k, v, budget_s=12.0, max_rows=512):
    """Time the float64 oracle on seeded rows of the ring rank's share."""
    import numpy as np

    from oracle import native
    from oracle import schedules as OS
    from seeded_inputs import sample_rows

    positions = OS.layout_index(OS.ZIGZAG, S, P, RING_RANK)
    order = sample_rows(len(positions), max_rows, seed=7).numpy()
    rng = np.random.default_rng(7)
    rng.shuffle(order)
    threads = len(os.sched_getaffinity(0))
    done_rows, flop, t_total = [], 0.0, 0.0
    for b in range(0, len(order), 16):
        rows = positions[order[b:b + 16]]
        t0 = time.perf_counter()
        native.attention_rows(q, k, v, rows=rows, n_threads=threads)
        t_total += time.perf_counter() - t0
        flop += sum(4.0 * D * HQ * (int(p) + 1) for p in rows)
        done_rows.extend(int(p) for p in rows)
        if t_total >= budget_s:
            break
    cpu_model = None
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    full = ring_share_flop(S, HQ, D, P, "zigzag", RING_RANK)
    return {
        "value": flop / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "full_ring_share_s_extrapolated": round(full / (flop / t_total), 1),
        "cpu_model": cpu_model,
        "kind": "oracle",
        "sample": (f"{len(done_rows)} seeded query rows of ring rank {RING_RANK}'s share "
                   f"(S={S}, P={P} zigzag) x all {HQ} heads against every visible key, "
                   f"float64 C oracle, {t_total:.1f} s, {flop / 1e12:.3f} TFLOP"),
    }


def backward(args, cp, torch, q_host, dq, dk, dv, dku, dvu, ql, kl, vl, uly_out_l, uly_lse,
             ring_out, ring_lse, stream, q_seq):
    """The backward pass of the same two shares (one JSON line).

    Ring share: cp_ring_bwd of rank 0 (zigzag: its 17 computed pairs; dq in
    the rank's local order, dk/dv over the whole sequence; dq, dk, dv here
    are the ring's inputs, in striped order for the striped layout).  Ulysses share:
    seq->head of dout, cp_attn_bwd_dvec, cp_attn_block_bwd of the 4 local
    query heads against their KV head, head->seq of dq, dk and dv.  The
    forward results (out, lse) are computed once before timing.
    FLOP: 2.5x the forward's causal-adjusted count (S, dP, dV, dK and dQ:
    10*D per visible pair and head, diagonal chunk counted half).
    """
    from seeded_inputs import make_qkv
    dev = "cuda:0"
    rows = S // P
    hp, hkp = HQ // P, HKV_ULY // P
    g = make_qkv(S=S, H=HQ, D=D, seed=1, dtype=torch.bfloat16)[0]
    dout_seq = g.to(dev)                              # upstream gradient, natural order
    idx = torch.from_numpy(cp.cp_layout_index(args.layout, S, P, args.rank).astype("int64"))
    dout_ring = g[idx].to(dev).contiguous()           # the ring rank's rows, local order
    del g
    # forward results
    cp.cp_ring_fwd(dq, dk, dv, P, args.layout, args.rank, out=ring_out, lse=ring_lse,
                   stream=stream)
    cp.cp_seq_to_head(q_seq, P, ULY_RANK, y=ql, stream=stream)
    cp.cp_seq_to_head(dku, P, ULY_RANK, y=kl, stream=stream)
    cp.cp_seq_to_head(dvu, P, ULY_RANK, y=vl, stream=stream)
    cp.cp_attn_block_fwd(ql, kl, vl, uly_out_l, uly_lse, stream=stream)
    f32 = dict(device=dev, dtype=torch.float32)
    g_q_ring, g_k_ring, g_v_ring = (torch.empty(rows, HQ, D, **f32), torch.empty(S, HQ, D, **f32),
                                    torch.empty(S, HQ, D, **f32))
    dvec_ring = torch.empty(HQ, rows, **f32)
    dout_l = torch.empty(S, hp, D, device=dev, dtype=torch.bfloat16)
    dvec_l = torch.empty(hp, S, **f32)
    g_ql, g_kl, g_vl = (torch.empty(S, hp, D, **f32), torch.empty(S, hkp, D, **f32),
                        torch.empty(S, hkp, D, **f32))
    g_q_seq = torch.zeros(S, HQ, D, **f32)
    g_k_seq = torch.zeros(S, HKV_ULY, D, **f32)
    g_v_seq = torch.zeros(S, HKV_ULY, D, **f32)

    def step():
        cp.cp_ring_bwd(dq, dk, dv, ring_out, ring_lse, dout_ring, P, args.layout, args.rank,
                       dq=g_q_ring, dk=g_k_ring, dv=g_v_ring, dvec=dvec_ring, stream=stream)
        cp.cp_seq_to_head(dout_seq, P, ULY_RANK, y=dout_l, stream=stream)
        cp.cp_attn_bwd_dvec(uly_out_l, dout_l, dvec_l, stream=stream)
        cp.cp_attn_block_bwd(ql, kl, vl, dout_l, uly_lse, dvec_l, g_ql, g_kl, g_vl, stream=stream)
        cp.cp_head_to_seq(g_ql, g_q_seq, P, ULY_RANK, stream=stream)
        cp.cp_head_to_seq(g_kl, g_k_seq, P, ULY_RANK, stream=stream)
        cp.cp_head_to_seq(g_vl, g_v_seq, P, ULY_RANK, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    cp.cp_timing_enable(True)
    cp.cp_timing_reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    bwd_ms, bwd_n = cp.cp_timing_read(cp.CP_KERNEL_BWD_BF16)
    dvec_ms, _ = cp.cp_timing_read(cp.CP_KERNEL_BWD_DVEC)
    perm_ms, _ = cp.cp_timing_read(cp.CP_KERNEL_PERMUTE)
    cp.cp_timing_enable(False)
    flop_step = 2.5 * (ring_share_flop(S, HQ, D, P, args.layout, args.rank)
                       + ulysses_share_flop(S, hp, D))
    kern_tflops = flop_step * args.steps / (bwd_ms * 1e-3) / 1e12 if bwd_ms > 0 else None
    result = {
        "metric": "causal block-attn bwd TFLOP/s + % bf16 MFMA peak, S=128K H=32 D=128",
        "value": round(flop_step * args.steps / elapsed / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": ("backward pass of one rank's share of a 128K-token causal attention "
                         f"layer: {args.layout} ring rank {args.rank} (S=131072, Hq=Hkv=32, "
                         "D=128, P=8) plus the Ulysses GQA rank (4 q heads on 1 KV head over "
                         "131072 tokens); bf16 q, k, v, dout; fp32 gradients"),
            "parts": "bwd",
            "ring_layout": args.layout,
            "ring_rank": args.rank,
            "flop_per_step": flop_step,
            "flop_convention": "2.5 x (4*D*Hq per visible (q,k) pair, diagonal chunk half)",
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "bwd_dq_kernel + bwd_dkdv_kernel",
            "achieved": round(kern_tflops, 2) if kern_tflops else None,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(kern_tflops / PEAK_BF16_TFLOPS, 4) if kern_tflops else None,
            "traffic": recorded_traffic(BWD_TRAFFIC_PROFILE, BWD_KERNEL_SOURCE,
                                        workload_key("bwd", args.layout, args.rank, S, P)),
            "traffic_unit": "bytes per dq + dk/dv launch pair (HBM read + write, calibrated)",
            "launches": bwd_n,
            "avg_launch_ms": round(bwd_ms / max(bwd_n, 1), 4),
        },
        "breakdown": {
            "bwd_kernels_ms_per_step": round(bwd_ms / args.steps, 3),
            "dvec_ms_per_step": round(dvec_ms / args.steps, 3),
            "repack_ms_per_step": round(perm_ms / args.steps, 3),
        },
    }
    print(json.dumps(result))


def usp_bwd(args, cp, torch, dq, dku, dvu, stream):
    """Backward of one rank's USP share (one JSON line): the forward of the
    rank's whole ring group once, untimed (its out and lse), then per step
    cp_usp_bwd of the rank (head-share copies, the ring backward on 4 query
    heads and 1 KV head, the gradients copied back).  FLOP: 2.5x the
    forward share's."""
    from seeded_inputs import make_qkv
    P_u, P_r = 8, 2
    rank = args.rank
    u, r = rank % P_u, rank // P_u
    hp = HQ // P_u
    rows = S // P_r
    dev = "cuda:0"
    qx, kx, vx = dq, dku, dvu
    if args.layout == "striped":
        order = torch.cat([torch.from_numpy(cp.cp_layout_index("striped", S, P_r, g).astype("int64"))
                           for g in range(P_r)]).to(dev)
        qx, kx, vx = (x[order].contiguous() for x in (dq, dku, dvu))
        del order
    out = torch.empty(rows, HQ, D, device=dev, dtype=torch.float32)
    lse = torch.empty(HQ, rows, device=dev, dtype=torch.float32)
    ws_f = torch.empty(cp.cp_usp_fwd_workspace(S, HQ, HKV_ULY, D, P_u, P_r, args.layout, rank,
                                               cp.CP_BF16), device=dev, dtype=torch.uint8)
    for uu in range(P_u):
        cp.cp_usp_fwd(qx, kx, vx, P_u, P_r, args.layout, r * P_u + uu, out=out, lse=lse,
                      workspace=ws_f, stream=stream)
    del ws_f
    idx = torch.from_numpy(cp.cp_layout_index(args.layout, S, P_r, r).astype("int64"))
    dout = make_qkv(S=S, H=HQ, D=D, seed=1, dtype=torch.bfloat16)[0][idx].to(dev).contiguous()
    f32 = dict(device=dev, dtype=torch.float32)
    g_q, g_k, g_v = (torch.empty(rows, HQ, D, **f32), torch.empty(S, HKV_ULY, D, **f32),
                     torch.empty(S, HKV_ULY, D, **f32))
    ws = torch.empty(cp.cp_usp_bwd_workspace(S, HQ, HKV_ULY, D, P_u, P_r, args.layout, rank,
                                             cp.CP_BF16), device=dev, dtype=torch.uint8)

    def step():
        cp.cp_usp_bwd(qx, kx, vx, out, lse, dout, P_u, P_r, args.layout, rank, dq=g_q, dk=g_k,
                      dv=g_v, workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    cp.cp_timing_enable(True)
    cp.cp_timing_reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    bwd_ms, bwd_n = cp.cp_timing_read(cp.CP_KERNEL_BWD_BF16)
    perm_ms, perm_n = cp.cp_timing_read(cp.CP_KERNEL_PERMUTE)
    dvec_ms, _ = cp.cp_timing_read(cp.CP_KERNEL_BWD_DVEC)
    cp.cp_timing_enable(False)
    flop_step = 2.5 * plan_flop(cp, S, hp, D, P_r, args.layout, r)
    kern = flop_step * args.steps / (bwd_ms * 1e-3) / 1e12 if bwd_ms > 0 else None
    print(json.dumps({
        "metric": "causal block-attn bwd TFLOP/s + % bf16 MFMA peak, USP 8x2, S=128K H=32/8 D=128",
        "value": round(flop_step * args.steps / elapsed / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"backward of one rank's USP share: rank {rank} (u={u}, r={r}) of 8-way "
                         f"Ulysses x 2-way {args.layout} ring, S=131072, Hq=32, Hkv=8, D=128; "
                         "bf16 q, k, v, dout; fp32 gradients"),
            "parts": "usp_bwd",
            "ring_layout": args.layout,
            "usp_rank": rank,
            "flop_per_step": flop_step,
            "flop_convention": "2.5 x (4*D*Hq_share per visible (q,k) pair, diagonal chunk half)",
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "bwd_dq_kernel + bwd_dkdv_kernel",
            "achieved": round(kern, 2) if kern else None,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(kern / PEAK_BF16_TFLOPS, 4) if kern else None,
            "traffic": None,
            "launches": bwd_n,
            "avg_launch_ms": round(bwd_ms / max(bwd_n, 1), 4),
        },
        "breakdown": {
            "bwd_kernels_ms_per_step": round(bwd_ms / args.steps, 3),
            "dvec_ms_per_step": round(dvec_ms / args.steps, 3),
            "repack_ms_per_step": round(perm_ms / args.steps, 3),
            "repack_launches_per_step": perm_n // max(args.steps, 1),
        },
    }))


def usp(args, cp, torch, dq, dku, dvu, stream):
    """One rank's share of the USP hybrid (one JSON line): 32 query heads on
    8 KV heads over 16 ranks as 8-way Ulysses x 2-way ring (the handbook's
    GQA exercise), S = 131072.  The share: seq->head of its ring group's
    query rows and of the key/value rows (head share u), the 2-step ring on
    4 query heads and 1 KV head, head->seq of the output rows.  FLOP: the
    ring share of the head share (diagonal chunk half), 2^43 per step."""
    P_u, P_r = 8, 2
    rank = args.rank
    u, r = rank % P_u, rank // P_u
    hp, hkp = HQ // P_u, HKV_ULY // P_u
    rows = S // P_r
    dev = "cuda:0"
    qx, kx, vx = dq, dku, dvu
    if args.layout == "striped":
        order = torch.cat([torch.from_numpy(cp.cp_layout_index("striped", S, P_r, g).astype("int64"))
                           for g in range(P_r)]).to(dev)
        qx, kx, vx = (x[order].contiguous() for x in (dq, dku, dvu))
        del order
    out = torch.empty(rows, HQ, D, device=dev, dtype=torch.float32)
    lse = torch.empty(HQ, rows, device=dev, dtype=torch.float32)
    ws = torch.empty(cp.cp_usp_fwd_workspace(S, HQ, HKV_ULY, D, P_u, P_r, args.layout, rank,
                                             cp.CP_BF16), device=dev, dtype=torch.uint8)

    def step():
        cp.cp_usp_fwd(qx, kx, vx, P_u, P_r, args.layout, rank, out=out, lse=lse, workspace=ws,
                      stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    cp.cp_timing_enable(True)
    cp.cp_timing_reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    attn_ms, attn_n = cp.cp_timing_read(cp.CP_KERNEL_ATTN_BF16)
    perm_ms, perm_n = cp.cp_timing_read(cp.CP_KERNEL_PERMUTE)
    cp.cp_timing_enable(False)
    flop_step = ring_share_flop(S, hp, D, P_r, args.layout, r)
    # each head-share copy reads and writes its bytes once
    perm_bytes = 2 * (rows * hp * D * 2 + 2 * S * hkp * D * 2 + rows * hp * D * 4)
    kern = flop_step * args.steps / (attn_ms * 1e-3) / 1e12 if attn_ms > 0 else None
    result = {
        "metric": "causal block-attn fwd TFLOP/s + % bf16 MFMA peak, USP 8x2, S=128K H=32/8 D=128",
        "value": round(flop_step * args.steps / elapsed / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"one rank's share of the USP hybrid: rank {rank} (u={u}, r={r}) of "
                         f"8-way Ulysses x 2-way {args.layout} ring, S=131072, Hq=32, Hkv=8, "
                         "D=128; bf16 inputs, fp32 out + lse"),
            "parts": "usp",
            "ring_layout": args.layout,
            "usp_rank": rank,
            "flop_per_step": flop_step,
            "flop_convention": "4*D*Hq_share per visible (q,k) pair, diagonal chunk counted half",
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_bf16_kernel",
            "achieved": round(kern, 2) if kern else None,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(kern / PEAK_BF16_TFLOPS, 4) if kern else None,
            "traffic": None,
            "launches": attn_n,
            "avg_launch_ms": round(attn_ms / max(attn_n, 1), 4),
        },
        "breakdown": {
            "attn_ms_per_step": round(attn_ms / args.steps, 3),
            "repack_ms_per_step": round(perm_ms / args.steps, 3),
            "repack_launches_per_step": perm_n // max(args.steps, 1),
            "repack_GBps": round(perm_bytes * args.steps / (perm_ms * 1e-3) / 1e9, 1)
            if perm_ms > 0 else None,
        },
    }
    print(json.dumps(result))


def block(args, cp, torch, dq, dk, dv, stream):
    """The whole 128K-token layer as one causal block (one JSON line):
    cp_attn_block_fwd of q, k, v bf16 [131072, 32, 128] (32 query heads on
    32 KV heads) into float32 out and lse, the shape the single-GPU kernel
    target names.  FLOP: 4*D*H per visible pair with the diagonal block
    counted half, 2^47 per step."""
    dev = "cuda:0"
    out = torch.empty(S, HQ, D, device=dev, dtype=torch.float32)
    lse = torch.empty(HQ, S, device=dev, dtype=torch.float32)

    def step():
        cp.cp_attn_block_fwd(dq, dk, dv, out, lse, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    cp.cp_timing_enable(True)
    cp.cp_timing_reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    attn_ms, attn_n = cp.cp_timing_read(cp.CP_KERNEL_ATTN_BF16)
    cp.cp_timing_enable(False)
    flop_step = 4.0 * D * HQ * S * S / 2.0
    kern = flop_step * args.steps / (attn_ms * 1e-3) / 1e12 if attn_ms > 0 else None
    result = {
        "metric": "causal block-attn fwd TFLOP/s + % bf16 MFMA peak, one block S=128K H=32 D=128",
        "value": round(flop_step * args.steps / elapsed / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": ("one causal block over the whole sequence: cp_attn_block_fwd of "
                         "q, k, v bf16 [131072, 32, 128] (Hq=Hkv=32, D=128), fp32 out + lse"),
            "parts": "block",
            "S": S, "Hq": HQ, "Hkv": HQ, "D": D,
            "flop_per_step": flop_step,
            "flop_convention": "4*D*Hq per visible (q,k) pair, diagonal block counted half",
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_bf16_kernel",
            "achieved": round(kern, 2) if kern else None,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(kern / PEAK_BF16_TFLOPS, 4) if kern else None,
            "traffic": recorded_traffic(BLOCK_TRAFFIC_PROFILE, KERNEL_SOURCE,
                                        workload_key("block", args.layout, args.rank, args.seq,
                                                     args.ring_p)),
            "traffic_unit": "bytes per launch (HBM read + write, calibrated)",
            "launches": attn_n,
            "avg_launch_ms": round(attn_ms / max(attn_n, 1), 4),
        },
    }
    print(json.dumps(result))


def rank_sweep(args, cp, torch, dq, dk, dv, stream, seq, RP):
    """Every rank's share of one ring, timed rank by rank (one JSON line):
    q, k, v bf16 [seq, 32, 128] (the first seq rows of the inputs; default
    65536 over P = 4 ranks), the contiguous and the zigzag split.  Per rank:
    its work in the handbook's units ("之字形切分": C x C chunk pairs of the
    2P-way split, C = seq / 2P, a diagonal pair counted half -- contiguous
    [2, 6, 10, 14] and zigzag [8, 8, 8, 8] at P = 4), its FLOP, the median
    ms of its cp_ring_fwd and the attention kernel's rate.  On a synchronous
    ring every step waits for the slowest rank, so a split's ring time is its
    largest rank time.  value: the zigzag split's FLOP over all ranks per
    second of rank time."""
    dev = "cuda:0"
    C = seq // (2 * RP)
    q, k, v = dq[:seq], dk[:seq], dv[:seq]
    rows = seq // RP
    out = torch.empty(rows, HQ, D, device=dev, dtype=torch.float32)
    lse = torch.empty(HQ, rows, device=dev, dtype=torch.float32)
    table = {}
    for layout in ("contiguous", "zigzag"):
        per = []
        for rank in range(RP):
            def step():
                cp.cp_ring_fwd(q, k, v, RP, layout, rank, out=out, lse=lse, stream=stream)
            for _ in range(args.warmup):
                step()
            torch.cuda.synchronize()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
            cp.cp_timing_enable(True)
            cp.cp_timing_reset()
            ev[0].record(stream)
            for i in range(args.steps):
                step()
                ev[i + 1].record(stream)
            torch.cuda.synchronize()
            ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
            attn_ms, attn_n = cp.cp_timing_read(cp.CP_KERNEL_ATTN_BF16)
            cp.cp_timing_enable(False)
            flop = plan_flop(cp, seq, HQ, D, RP, layout, rank)
            kern = flop * args.steps / (attn_ms * 1e-3) / 1e12
            per.append({"rank": rank, "units": flop / (4.0 * D * HQ * C * C), "flop": flop,
                        "launches": attn_n // args.steps,
                        "ms_median": round(ms[len(ms) // 2], 3),
                        "kernel_tflops": round(kern, 2),
                        "kernel_frac": round(kern / PEAK_BF16_TFLOPS, 4)})
        table[layout] = {"ranks": per,
                         "ring_time_ms": max(r["ms_median"] for r in per),
                         "flop_all_ranks": sum(r["flop"] for r in per)}
    zz = table["zigzag"]
    value = zz["flop_all_ranks"] / (sum(r["ms_median"] for r in zz["ranks"]) * 1e-3) / 1e12
    kern_ms = sum(r["flop"] / (r["kernel_tflops"] * 1e12) for r in zz["ranks"])
    print(json.dumps({
        "metric": f"causal ring per-rank shares TFLOP/s, S={seq} P={RP} H=32 D=128",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sum(r["ms_median"] for r in zz["ranks"]), 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"every rank of a {RP}-rank ring over {seq} tokens (Hq=Hkv=32, D=128, "
                         "bf16 inputs, fp32 out + lse), timed rank by rank; contiguous and "
                         "zigzag splits"),
            "parts": "ranks", "seq": seq, "P": RP, "chunk": C,
            "flop_convention": "4*D*Hq per visible (q,k) pair, diagonal chunk counted half",
            "per_rank": table,
            "ring_time_ratio_contiguous_over_zigzag": round(
                table["contiguous"]["ring_time_ms"] / zz["ring_time_ms"], 3),
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_bf16_kernel",
            "achieved": round(zz["flop_all_ranks"] / kern_ms / 1e12, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(zz["flop_all_ranks"] / kern_ms / 1e12 / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
        },
    }))


def merge_repack(args, cp, torch, dq, dku, dvu, stream):
    """The bandwidth-bound kernels alone (one JSON line each run).

    merge: the log-sum-exp merges of one ring rank at 128K (P = 8, zigzag)
    when they run as separate kernels: 15 per step (17 computed chunk
    pairs, the first result of each of the 2 query chunks is stored), each
    folding an [8192, 32, 128] float32 block result and its [32, 8192] lse
    into the running ones, out of place (or in place with --merge-in-place).
    Algorithmic bytes: 12 per output element + 12 per (row, head).

    repack: the Ulysses repacks of one rank at 128K (seq->head of q
    [131072, 32, 128] and of k, v [131072, 8, 128] bf16, head->seq of the
    float32 output), each reading and writing its rank's share once."""
    from seeded_inputs import make_qkv
    dev = "cuda:0"
    if args.part == "merge":
        rows, n_merge = S // (2 * P), 15
        o1, o2, _ = make_qkv(S=rows, H=HQ, D=D, seed=11)
        l1, l2, _ = make_qkv(S=HQ, H=rows, D=1, seed=12)
        l1, l2 = 3.0 * l1[..., 0], 3.0 * l2[..., 0]
        l1[:, ::97] = float("-inf")          # rows with no visible key on one side
        l2[:, ::89] = float("-inf")
        o1, o2, l1, l2 = (x.to(dev).contiguous() for x in (o1, o2, l1, l2))
        if args.merge_in_place:
            o, lse = o1, l1
        else:
            o, lse = torch.empty_like(o1), torch.empty_like(l1)

        def step():
            for _ in range(n_merge):
                cp.cp_lse_merge(o1, l1, o2, l2, o, lse, stream=stream)

        kind = cp.CP_KERNEL_MERGE
        bytes_step = n_merge * (rows * HQ * D * 12 + rows * HQ * 12)
        kernel = "lse_merge_kernel"
        workload = (f"log-sum-exp merges of one zigzag ring rank at S=131072, P=8: {n_merge} "
                    f"per step, each [{rows}, {HQ}, {D}] float32 + lse [{HQ}, {rows}], "
                    + ("in place" if args.merge_in_place else "out of place"))
        metric = "lse merge HBM GB/s + % of HBM peak, 8192x32x128 fp32 chunk"
    else:
        hp, hkp = HQ // P, HKV_ULY // P
        ql = torch.empty(S, hp, D, device=dev, dtype=torch.bfloat16)
        kl = torch.empty(S, hkp, D, device=dev, dtype=torch.bfloat16)
        vl = torch.empty(S, hkp, D, device=dev, dtype=torch.bfloat16)
        ol = torch.randn(S, hp, D, device=dev, dtype=torch.float32,
                         generator=torch.Generator(device=dev).manual_seed(13))
        out = torch.zeros(S, HQ, D, device=dev, dtype=torch.float32)   # head slice 0 written

        def step():
            cp.cp_seq_to_head(dq, P, ULY_RANK, y=ql, stream=stream)
            cp.cp_seq_to_head(dku, P, ULY_RANK, y=kl, stream=stream)
            cp.cp_seq_to_head(dvu, P, ULY_RANK, y=vl, stream=stream)
            cp.cp_head_to_seq(ol, out, P, ULY_RANK, stream=stream)

        kind = cp.CP_KERNEL_PERMUTE
        bytes_step = 2 * (S * hp * D * 2 + 2 * S * hkp * D * 2 + S * hp * D * 4)
        kernel = "unit_copy_kernel"
        workload = ("Ulysses repacks of one rank at S=131072, P=8: seq->head of q "
                    "[131072, 32, 128] and k, v [131072, 8, 128] bf16, head->seq of the "
                    "float32 output [131072, 4, 128] into its head slice of [131072, 32, 128]")
        metric = "Ulysses repack HBM GB/s + % of HBM peak, S=128K H=32/8 D=128"

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    cp.cp_timing_enable(True)
    cp.cp_timing_reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    k_ms, k_n = cp.cp_timing_read(kind)
    cp.cp_timing_enable(False)
    gbs = bytes_step * args.steps / (k_ms * 1e-3) / 1e9 if k_ms > 0 else None
    result = {
        "metric": metric,
        "value": round(bytes_step * args.steps / elapsed / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if args.part == "merge" else "bf16+f32",
        "data": "synthetic",
        "config": {"workload": workload, "parts": args.part, "bytes_per_step": bytes_step},
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "achieved": round(gbs, 1) if gbs else None,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4) if gbs else None,
            "traffic": None,
            "launches": k_n,
            "avg_launch_ms": round(k_ms / max(k_n, 1), 4),
            "bytes_per_launch": bytes_step * args.steps / max(k_n, 1),
        },
    }
    print(json.dumps(result))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--part", choices=["both", "ring", "ulysses", "bwd", "usp", "usp_bwd",
                                       "merge", "repack", "ranks", "block"],
                    default="both",
                    help="bwd: time the backward pass of both shares instead; usp: one rank "
                         "of the 8-way Ulysses x 2-way ring hybrid; merge / repack: the "
                         "bandwidth-bound kernels alone (GB/s against the HBM peak); block: "
                         "the whole sequence as one causal block on one GPU")
    ap.add_argument("--merge-in-place", action="store_true",
                    help="--part merge: fold into the running output in place")
    ap.add_argument("--layout", choices=["zigzag", "striped", "contiguous"], default="zigzag",
                    help="split of the ring share (striped: inputs permuted to striped order "
                         "once, before timing)")
    ap.add_argument("--seq", type=int, default=None,
                    help="sequence length of the ring share (--part ring only; lengths the "
                         "split does not divide are padded)")
    ap.add_argument("--rank", type=int, default=RING_RANK, choices=range(-1, 2 * P),
                    help="the virtual rank whose share is timed (ring: 0..P-1 or -1 for "
                         "every rank at once, usp: 0..15)")
    ap.add_argument("--ring-p", type=int, default=None,
                    help="ranks of the ring (--part ring and --part ranks only)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="before warm-up, copy 1 GiB device to device once (a plain copy "
                         "kernel of known size that scales HBM byte counters)")
    args = ap.parse_args()
    if args.part == "ranks":       # the 64K per-rank comparison: 4 ranks over 65536 tokens
        args.seq = 65536 if args.seq is None else args.seq
        args.ring_p = 4 if args.ring_p is None else args.ring_p
    args.seq = S if args.seq is None else args.seq
    args.ring_p = P if args.ring_p is None else args.ring_p
    RP = args.ring_p
    if RP != P and args.part not in ("ring", "ranks"):
        ap.error("--ring-p applies to --part ring and --part ranks only")
    if not 1 <= RP <= 64:
        ap.error("--ring-p must be in [1, 64]")
    if args.part not in ("usp", "usp_bwd") and args.rank >= RP:
        ap.error(f"--rank must be below {RP} for the ring share")
    if args.rank < 0 and args.part != "ring":
        ap.error("--rank -1 (every rank) applies to --part ring only")
    if args.seq != S and args.part not in ("ring", "ranks"):
        ap.error("--seq applies to --part ring and --part ranks only")
    if not 1 <= args.seq <= S:
        ap.error(f"--seq must be in [1, {S}]")
    if args.part == "ranks" and args.seq % (2 * RP) != 0:
        ap.error("--part ranks needs a length that 2 * --ring-p divides")
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the ring and Ulysses ranks are virtual and "
              "played on a single MI355X; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import context_parallelism_cp_amd as cp
    from seeded_inputs import make_qkv, sha256_of

    dev = "cuda:0"
    torch.cuda.set_device(0)
    t_gen = time.perf_counter()
    q, k, v = make_qkv(S=S, H=HQ, D=D, seed=0, dtype=torch.bfloat16)
    _, ku, vu = make_qkv(S=S, H=HQ, D=D, seed=0, dtype=torch.bfloat16, Hkv=HKV_ULY)
    dq, dk, dv = q.to(dev), k.to(dev), v.to(dev)
    dku, dvu = ku.to(dev), vu.to(dev)
    print(f"# inputs generated and resident in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr)

    seq = args.seq
    if args.layout == "striped":
        # a striped rank holds its shard in striped order: permute once (the
        # padding rows, if any, repeat the last row; they are never read)
        order = torch.cat([torch.from_numpy(cp.cp_layout_index("striped", seq, RP, r).astype("int64"))
                           for r in range(RP)]).clamp_(max=seq - 1).to(dev)
        rq, rk, rv = dq[order].contiguous(), dk[order].contiguous(), dv[order].contiguous()
        del order
    else:
        rq, rk, rv = dq[:seq], dk[:seq], dv[:seq]

    rows = cp._ring_rows(seq, RP, cp.LAYOUTS[args.layout], args.rank)[1]
    ring_out = torch.empty(rows, HQ, D, device=dev, dtype=torch.float32)
    ring_lse = torch.empty(HQ, rows, device=dev, dtype=torch.float32)
    hp, hkp = HQ // P, HKV_ULY // P
    ql = torch.empty(S, hp, D, device=dev, dtype=torch.bfloat16)
    kl = torch.empty(S, hkp, D, device=dev, dtype=torch.bfloat16)
    vl = torch.empty(S, hkp, D, device=dev, dtype=torch.bfloat16)
    uly_out_l = torch.empty(S, hp, D, device=dev, dtype=torch.float32)
    uly_lse = torch.empty(hp, S, device=dev, dtype=torch.float32)
    uly_out = torch.zeros(S, HQ, D, device=dev, dtype=torch.float32)
    stream = torch.cuda.current_stream()

    ring_done = []          # per timed step: an event after the ring share

    def step():
        if args.part in ("both", "ring"):
            cp.cp_ring_fwd(rq, rk, rv, RP, args.layout, args.rank, out=ring_out, lse=ring_lse,
                           stream=stream, seq_len=seq)
            if timing[0] and len(ring_done) < args.steps:
                ev = torch.cuda.Event(enable_timing=True)
                ev.record(stream)
                ring_done.append(ev)
        if args.part in ("both", "ulysses"):
            cp.cp_seq_to_head(dq, P, ULY_RANK, y=ql, stream=stream)
            cp.cp_seq_to_head(dku, P, ULY_RANK, y=kl, stream=stream)
            cp.cp_seq_to_head(dvu, P, ULY_RANK, y=vl, stream=stream)
            cp.cp_attn_block_fwd(ql, kl, vl, uly_out_l, uly_lse, stream=stream)
            cp.cp_head_to_seq(uly_out_l, uly_out, P, ULY_RANK, stream=stream)

    if args.calibration_copy:
        src = torch.empty(1 << 28, device=dev, dtype=torch.float32).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)          # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst

    if args.part == "usp":
        usp(args, cp, torch, dq, dku, dvu, stream)
        return
    if args.part == "block":
        block(args, cp, torch, dq, dk, dv, stream)
        return
    if args.part == "ranks":
        rank_sweep(args, cp, torch, dq, dk, dv, stream, args.seq, RP)
        return
    if args.part in ("merge", "repack"):
        merge_repack(args, cp, torch, dq, dku, dvu, stream)
        return
    if args.part == "usp_bwd":
        usp_bwd(args, cp, torch, dq, dku, dvu, stream)
        return
    if args.part == "bwd":
        backward(args, cp, torch, q, rq, rk, rv, dku, dvu, ql, kl, vl, uly_out_l, uly_lse,
                 ring_out, ring_lse, stream, dq)
        return

    timing = [False]
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # events on the launch stream around every step (no host synchronisation
    # inside the timed region) give the per-step median
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    timing[0] = True
    cp.cp_timing_enable(True)
    cp.cp_timing_reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step_ev[0].record(stream)
    for i in range(args.steps):
        step()
        step_ev[i + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = sorted(step_ev[i].elapsed_time(step_ev[i + 1]) for i in range(args.steps))
    ring_ms = (sorted(step_ev[i].elapsed_time(ring_done[i]) for i in range(args.steps))
               if len(ring_done) == args.steps else None)
    attn_ms, attn_n = cp.cp_timing_read(cp.CP_KERNEL_ATTN_BF16)
    perm_ms, perm_n = cp.cp_timing_read(cp.CP_KERNEL_PERMUTE)
    cp.cp_timing_enable(False)

    flop_ring = (plan_flop(cp, seq, HQ, D, RP, args.layout, args.rank)
                 if args.part in ("both", "ring") else 0.0)
    flop_uly = ulysses_share_flop(S, hp, D) if args.part in ("both", "ulysses") else 0.0
    flop_step = flop_ring + flop_uly
    ring_exact = (plan_flop_exact(cp, seq, HQ, D, RP, args.layout, args.rank)
                  if args.part in ("both", "ring") else 0.0)
    flop_exact = (None if ring_exact is None else ring_exact + (
        4.0 * D * hp * S * (S + 1) / 2.0 if args.part in ("both", "ulysses") else 0.0))
    ms_step = elapsed * 1e3 / args.steps
    value = flop_step * args.steps / elapsed / 1e12
    attn_tflops = flop_step * args.steps / (attn_ms * 1e-3) / 1e12 if attn_ms > 0 else None
    perm_bytes_step = 0
    if args.part in ("both", "ulysses"):
        # each repack reads and writes its rank's share once
        perm_bytes_step = 2 * (S * hp * D * 2 + 2 * S * hkp * D * 2 + S * hp * D * 4)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": ("one rank's share of a 128K-token causal attention layer: zigzag ring "
                         "rank (S=131072, Hq=Hkv=32, D=128, P=8, 16 chunks of 8192) plus "
                         "Ulysses GQA rank (Hq=32, Hkv=8, P=8 -> 4 q heads on 1 KV head over "
                         "all 131072 tokens); bf16 inputs, fp32 out + lse"
                         if (args.layout, args.rank, seq, RP) == ("zigzag", RING_RANK, S, P)
                         and args.part == "both" else
                         f"{args.part}: ring " + ("every rank" if args.rank < 0 else
                                                  f"rank {args.rank}")
                         + f" of the {RP}-rank {args.layout} split over {seq} tokens "
                         "(Hq=Hkv=32, D=128)"
                         + (" plus the Ulysses GQA rank" if args.part == "both" else "")),
            "parts": args.part,
            "ring_layout": args.layout,
            "ring_rank": args.rank,
            "ring_seq": seq,
            "S": S, "Hq": HQ, "Hkv_ring": HQ, "Hkv_ulysses": HKV_ULY, "D": D, "P": RP,
            "flop_per_step": flop_step,
            "flop_convention": "4*D*Hq per visible (q,k) pair, diagonal chunk counted half",
            "flop_per_step_exact": flop_exact,
            "inputs_sha256": sha256_of(q[:4096], k[:4096], v[:4096]),
        },
        "timing": {
            "ms_per_step_median": round(step_ms[len(step_ms) // 2], 3),
            "ms_per_step_min": round(step_ms[0], 3),
            "ring_ms_median": round(ring_ms[len(ring_ms) // 2], 3) if ring_ms else None,
            "value_exact_count": (round(flop_exact * args.steps / elapsed / 1e12, 2)
                                  if flop_exact else None),
            "source": "HIP events on the launch stream around each timed step (the ring "
                      "share: cp_ring_fwd with its fused merges)",
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_bf16_kernel",
            "achieved": round(attn_tflops, 2) if attn_tflops else None,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4) if attn_tflops else None,
            "traffic": recorded_traffic(workload=workload_key(args.part, args.layout, args.rank,
                                                              seq, RP)),
            "traffic_unit": "bytes per launch (HBM read + write, calibrated)",
            "launches": attn_n,
            "avg_launch_ms": round(attn_ms / max(attn_n, 1), 4),
            "flop_per_launch": flop_step * args.steps / max(attn_n, 1),
        },
        "breakdown": {
            "attn_ms_per_step": round(attn_ms / args.steps, 3),
            "repack_ms_per_step": round(perm_ms / args.steps, 3),
            "repack_launches_per_step": perm_n // max(args.steps, 1),
            "repack_GBps": round(perm_bytes_step * args.steps / (perm_ms * 1e-3) / 1e9, 1)
            if perm_ms > 0 else None,
            "repack_frac_hbm": round(perm_bytes_step * args.steps / (perm_ms * 1e-3) / 1e9
                                     / PEAK_HBM_GBS, 4) if perm_ms > 0 else None,
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(q, k, v)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
