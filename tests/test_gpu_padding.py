"""Padding (sequence lengths the split does not divide) through the C-ABI
against the oracle.

The real rows of every call must equal the single pass on the unpadded
sequence (oracle.schedules.ring_padded, pinned to it); the padding rows of
an output come back as (0, -inf), and padding rows of a striped-order input
are filled with NaN to show that they are never read.  Backward: per-rank
gradients against the oracle's composition over the padded plan, padding
rows of dq / dk / dv exactly 0.  Tolerances as the other parity tests.
"""
import numpy as np
import pytest
import torch

import context_parallelism_cp_amd as cp
from oracle import attention as OA
from oracle import schedules as OS
from seeded_inputs import make_qkv

from test_gpu_bwd import BF16_GRAD_REL, F32_GRAD_TOL, grads_compare
from test_gpu_parity import (BF16_LSE_TOL, BF16_OUT_TOL, DEV, F32_TOL, Guarded, announce,
                             chunk_edge_rows, compare, oracle_rows)

pytestmark = pytest.mark.gpu
LAYOUTS = ["contiguous", "zigzag", "striped"]


def input_positions(layout, S, P):
    """Position held by each row of the tensors a call takes (>= S: padding)."""
    lay = cp.LAYOUTS[layout]
    if lay != OS.STRIPED:
        return np.arange(S)
    return np.concatenate([OS.layout_index(lay, S, P, r) for r in range(P)])


def to_input(x, pos, S):
    """Rows of x at the given positions; padding rows NaN."""
    real = torch.from_numpy(np.minimum(pos, S - 1))
    y = x[real].clone()
    y[torch.from_numpy(pos >= S)] = float("nan")
    return y.to(DEV).contiguous()


def expected(ro, rl, pos, S):
    """Oracle rows at pos, padding rows (0, -inf)."""
    pos = np.asarray(pos)
    o = np.zeros((len(pos),) + ro.shape[1:])
    l = np.full((rl.shape[0], len(pos)), -np.inf)
    real = pos < S
    o[real] = ro[pos[real]]
    l[:, real] = rl[:, pos[real]]
    return o, l


def out_positions(layout, S, P, rank):
    lay = cp.LAYOUTS[layout]
    if rank < 0:
        return input_positions(layout, S, P)
    return OS.layout_index(lay, S, P, rank)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("S", [30, 29, 3])
def test_f32_padded_ring_page_inputs(layout, S):
    """The page's make_qkv() cut to S rows over 4 ranks (S = 3: a rank
    with no real row)."""
    P = 4
    announce(f"f32 padded ring S={S} P={P} {layout}")
    q, k, v = (x[:S] for x in make_qkv())
    ipos = input_positions(layout, S, P)
    qd, kd, vd = (to_input(x, ipos, S) for x in (q, k, v))
    lay = cp.LAYOUTS[layout]
    for causal in (True, False):
        ro, rl = OA.attention(q, k, v, causal=causal)
        po, pl, ppos = OS.ring_padded(q, k, v, P, lay, causal)
        for rank in [-1] + list(range(P)):
            opos = out_positions(layout, S, P, rank)
            rows = len(opos)
            out, lse = Guarded(rows, 8, 16), Guarded(8, rows)
            cp.cp_ring_fwd(qd, kd, vd, P, layout, rank, causal=causal, out=out.t, lse=lse.t,
                           seq_len=S)
            torch.cuda.synchronize()
            out.check(), lse.check()
            wo, wl = expected(ro, rl, opos, S)
            compare(out.t, lse.t, wo, wl, F32_TOL, F32_TOL, f"{layout} rank {rank}")
            assert bool((out.t[torch.from_numpy(opos >= S)] == 0).all())
            if rank >= 0:   # the padding oracle's own per-rank result
                real = torch.from_numpy(np.nonzero(opos < S)[0])
                compare(out.t[real], lse.t[:, real], po[rank], pl[rank], F32_TOL, F32_TOL,
                        f"{layout} rank {rank} vs ring_padded")
                assert np.array_equal(opos[opos < S], ppos[rank])


@pytest.mark.parametrize("layout", LAYOUTS)
def test_bf16_padded_ring_every_rank(layout):
    S, Hq, Hkv, P = 2000, 4, 2, 3
    announce(f"bf16 padded ring S={S} Hq={Hq} Hkv={Hkv} P={P} {layout}")
    q, k, v = make_qkv(S=S, H=Hq, D=128, seed=29, dtype=torch.bfloat16, Hkv=Hkv)
    ro, rl = oracle_rows(q, k, v, None)
    ipos = input_positions(layout, S, P)
    qd, kd, vd = (to_input(x, ipos, S) for x in (q, k, v))
    for rank in [-1] + list(range(P)):
        opos = out_positions(layout, S, P, rank)
        out, lse = cp.cp_ring_fwd(qd, kd, vd, P, layout, rank, seq_len=S)
        torch.cuda.synchronize()
        wo, wl = expected(ro, rl, opos, S)
        compare(out, lse, wo, wl, BF16_OUT_TOL, BF16_LSE_TOL, f"{layout} rank {rank}")


@pytest.mark.parametrize("layout,rank", [("zigzag", 0), ("zigzag", 7), ("striped", 7),
                                         ("contiguous", 7)])
def test_full_padded_rank_share_128k(layout, rank):
    """131071 tokens over 8 ranks (no split divides it): one rank's share
    in the benchmark's launch configuration, sampled rows and every padding
    row."""
    S, H, P = 131071, 32, 8
    announce(f"bf16 padded ring S={S} H={H} P={P} {layout} rank {rank} (sampled rows)")
    q, k, v = make_qkv(S=S, H=H, D=128, seed=0, dtype=torch.bfloat16)
    ipos = input_positions(layout, S, P)
    qd, kd, vd = (to_input(x, ipos, S) for x in (q, k, v))
    opos = out_positions(layout, S, P, rank)
    rows = len(opos)
    out, lse = Guarded(rows, H, 128), Guarded(H, rows)
    cp.cp_ring_fwd(qd, kd, vd, P, layout, rank, out=out.t, lse=lse.t, seq_len=S)
    torch.cuda.synchronize()
    out.check(), lse.check()
    del qd, kd, vd
    pad = np.nonzero(opos >= S)[0]
    pt = torch.from_numpy(pad).to(DEV)
    assert bool((out.t[pt] == 0).all()) and bool(torch.isneginf(lse.t[:, pt]).all())
    real = np.nonzero(opos < S)[0]
    local = chunk_edge_rows(len(real), max(len(real) // 2, 1), 8, seed=31 + rank)
    rows_sel = real[local[local < len(real)]]
    ro, rl = oracle_rows(q, k, v, opos[rows_sel])
    lt = torch.from_numpy(rows_sel).to(DEV)
    compare(out.t[lt], lse.t[:, lt], ro, rl, BF16_OUT_TOL, BF16_LSE_TOL,
            f"131071 {layout} rank {rank}")


# ------------------------------------------------------------- backward
def rank_bwd_oracle(q, k, v, dout, P, layout, rank, causal):
    """dq of the call's output rows and the call's dk / dv contributions,
    in the call's row order, from oracle.attention_bwd_at over the padded
    plan's pairs (padding rows 0)."""
    lay = cp.LAYOUTS[layout]
    qn, kn, vn, dn = (x.double().numpy() for x in (q, k, v, dout))
    S = qn.shape[0]
    out, lse = OA.attention(qn, kn, vn, causal=causal)
    dq, dk, dv = np.zeros_like(qn), np.zeros_like(kn), np.zeros_like(vn)
    for (r, _t, _qc, src, qo, ko, lq, lk, kind) in OS.ring_plan(S, P, lay, rank, causal):
        if kind == OS.SKIP:
            continue
        if lay == OS.STRIPED:
            qp = OS.layout_index(lay, S, P, r)[:lq]
            kp = OS.layout_index(lay, S, P, src)[:lk]
        else:
            qp, kp = np.arange(qo, qo + lq), np.arange(ko, ko + lk)
        gq, gk, gv = OA.attention_bwd_at(qn[qp], kn[kp], vn[kp], dn[qp], out[qp], lse[:, qp],
                                         qp, kp, causal=causal)
        dq[qp] += gq
        dk[kp] += gk
        dv[kp] += gv

    def rows_at(x, pos):
        y = np.zeros((len(pos),) + x.shape[1:])
        y[pos < S] = x[pos[pos < S]]
        return y

    opos = out_positions(layout, S, P, rank)
    ipos = input_positions(layout, S, P)
    return rows_at(dq, opos), rows_at(dk, ipos), rows_at(dv, ipos)


def run_padded_bwd(q, k, v, dout, P, layout, rank, causal, S):
    ipos = input_positions(layout, S, P)
    opos = out_positions(layout, S, P, rank)
    qd, kd, vd = (to_input(x, ipos, S) for x in (q, k, v))
    # dout rows of padding are finite: they multiply out = 0 in dvec only
    dd = dout[torch.from_numpy(np.minimum(opos, S - 1))].to(DEV).contiguous()
    out, lse = cp.cp_ring_fwd(qd, kd, vd, P, layout, rank, causal=causal, seq_len=S)
    Hq, D = q.shape[1], q.shape[2]
    Hkv = k.shape[1]
    dq, dk, dv = Guarded(len(opos), Hq, D), Guarded(len(ipos), Hkv, D), Guarded(len(ipos), Hkv, D)
    cp.cp_ring_bwd(qd, kd, vd, out, lse, dd, P, layout, rank, causal=causal, dq=dq.t, dk=dk.t,
                   dv=dv.t, seq_len=S)
    torch.cuda.synchronize()
    for g in (dq, dk, dv):
        g.check()
    return dq.t, dk.t, dv.t


@pytest.mark.parametrize("layout", LAYOUTS)
def test_f32_padded_ring_bwd_page_inputs(layout):
    S, P = 30, 4
    announce(f"f32 padded ring bwd S={S} P={P} {layout}")
    q, k, v = (x[:S] for x in make_qkv())
    dout = make_qkv(S=S, H=8, D=16, seed=78)[0]
    for causal in (True, False):
        for rank in [-1, 0, 1, 2, 3]:
            got = run_padded_bwd(q, k, v, dout, P, layout, rank, causal, S)
            want = rank_bwd_oracle(q, k, v, dout, P, layout, rank, causal)
            grads_compare(got, want, F32_GRAD_TOL, f"{layout} rank {rank} causal={causal}")


@pytest.mark.parametrize("layout", ["zigzag", "striped"])
def test_bf16_padded_ring_bwd(layout):
    S, Hq, Hkv, P = 2000, 4, 2, 3
    announce(f"bf16 padded ring bwd S={S} Hq={Hq} Hkv={Hkv} P={P} {layout}")
    q, k, v = make_qkv(S=S, H=Hq, D=128, seed=33, dtype=torch.bfloat16, Hkv=Hkv)
    dout = make_qkv(S=S, H=Hq, D=128, seed=34, dtype=torch.bfloat16)[0]
    for rank in [-1, 0, 2]:
        got = run_padded_bwd(q, k, v, dout, P, layout, rank, True, S)
        want = rank_bwd_oracle(q, k, v, dout, P, layout, rank, True)
        grads_compare(got, want, BF16_GRAD_REL, f"{layout} rank {rank}", rel=True)


@pytest.mark.parametrize("case", range(10))
def test_bf16_ring_random_shapes(case):
    """Seeded random ring calls: 2-5 ranks, any layout, one rank's share or
    every rank, lengths the split may or may not divide (200-3000 tokens),
    GQA ratios 1, 2, 4, causal or not; the forward against the single pass
    and the backward against the oracle's composition over the plan (the
    relative bound as in the random block sweep: against the largest
    gradient magnitude of the call when a tensor's own is smaller)."""
    rng = np.random.default_rng(7000 + case)
    P = int(rng.integers(2, 6))
    layout = str(rng.choice(LAYOUTS))
    S = int(rng.integers(200, 3001))
    Hkv = int(rng.choice([1, 2]))
    Hq = Hkv * int(rng.choice([1, 2, 4]))
    rank = int(rng.integers(-1, P))
    causal = bool(rng.integers(0, 2))
    announce(f"bf16 ring random case {case}: S={S} Hq={Hq} Hkv={Hkv} P={P} {layout} "
             f"rank {rank} causal={causal}")
    q, k, v = make_qkv(S=S, H=Hq, D=128, seed=8000 + case, dtype=torch.bfloat16, Hkv=Hkv)
    dout = make_qkv(S=S, H=Hq, D=128, seed=9000 + case, dtype=torch.bfloat16)[0]
    ro, rl = oracle_rows(q, k, v, None, causal=causal)
    ipos = input_positions(layout, S, P)
    opos = out_positions(layout, S, P, rank)
    qd, kd, vd = (to_input(x, ipos, S) for x in (q, k, v))
    out, lse = cp.cp_ring_fwd(qd, kd, vd, P, layout, rank, causal=causal, seq_len=S)
    torch.cuda.synchronize()
    wo, wl = expected(ro, rl, opos, S)
    compare(out, lse, wo, wl, BF16_OUT_TOL, BF16_LSE_TOL, f"ring random {case} fwd")
    got = run_padded_bwd(q, k, v, dout, P, layout, rank, causal, S)
    want = rank_bwd_oracle(q, k, v, dout, P, layout, rank, causal)
    floor = max(float(np.abs(w).max()) if w.size else 0.0 for w in want)
    grads_compare(got, want, BF16_GRAD_REL, f"ring random {case} bwd", rel=True,
                  scale_floor=floor)

