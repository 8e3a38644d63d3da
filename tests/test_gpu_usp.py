"""USP hybrid (Ulysses inside ring groups, ring across them) through the
C-ABI against the oracle.

Every rank of a group writes its head share of the group's rows; the P_u
ranks of a group together fill them, and the filled rows are compared with
the oracle's USP result for those ranks (oracle.schedules.usp_attention,
pinned to the single pass) and with the single pass at the rows'
positions.  Tolerances as the forward parity tests: float32 1e-5; bf16 out
1e-2, lse 1e-3.
"""
import numpy as np
import pytest
import torch

import context_parallelism_cp_amd as cp
from oracle import attention as OA
from oracle import schedules as OS
from seeded_inputs import make_qkv

from test_gpu_parity import (BF16_LSE_TOL, BF16_OUT_TOL, DEV, F32_TOL, Guarded, announce,
                             check_share, chunk_edge_rows, compare, dev, oracle_rows,
                             striped_order)

pytestmark = pytest.mark.gpu


def input_order(layout, S, P_r):
    return striped_order(S, P_r) if layout == "striped" else np.arange(S)


def run_group(qd, kd, vd, P_u, P_r, layout, r, causal=True):
    """All P_u ranks of ring group r into one guarded buffer."""
    S, Hq, D = qd.shape
    rows = S // P_r
    out, lse = Guarded(rows, Hq, D), Guarded(Hq, rows)
    for u in range(P_u):
        cp.cp_usp_fwd(qd, kd, vd, P_u, P_r, layout, r * P_u + u, causal=causal, out=out.t,
                      lse=lse.t)
    torch.cuda.synchronize()
    out.check(), lse.check()
    return out.t, lse.t


@pytest.mark.parametrize("layout", ["contiguous", "zigzag", "striped"])
@pytest.mark.parametrize("P_u,P_r", [(2, 2), (4, 2), (2, 4)])
def test_f32_usp_page_inputs(layout, P_u, P_r):
    """The page's make_qkv() with 8 heads on 4 KV heads (GQA)."""
    announce(f"f32 USP P_u={P_u} P_r={P_r} {layout} on make_qkv() (Hkv=4)")
    q, _, _ = make_qkv()
    _, k, v = make_qkv(H=4, seed=3)
    S = 32
    order = input_order(layout, S, P_r)
    ot = torch.from_numpy(order)
    qd, kd, vd = dev(q[ot], k[ot], v[ot])
    lay = cp.LAYOUTS[layout]
    for causal in (True, False):
        ro, rl = OA.attention(q, k, v, causal=causal)
        uo, ul, upos = OS.usp_attention(q, k, v, P_u, P_r, lay, causal=causal)
        out, lse = Guarded(S, 8, 16), Guarded(8, S)
        cp.cp_usp_fwd(qd, kd, vd, P_u, P_r, layout, -1, causal=causal, out=out.t, lse=lse.t)
        torch.cuda.synchronize()
        out.check(), lse.check()
        compare(out.t, lse.t, ro[order], rl[:, order], F32_TOL, F32_TOL, f"{layout} all ranks")
        for r in range(P_r):
            o, l = run_group(qd, kd, vd, P_u, P_r, layout, r, causal)
            ranks = range(r * P_u, (r + 1) * P_u)
            want_o = np.concatenate([uo[x] for x in ranks])
            want_l = np.concatenate([ul[x] for x in ranks], axis=1)
            compare(o, l, want_o, want_l, F32_TOL, F32_TOL, f"{layout} group {r}")
            pos = np.concatenate([upos[x] for x in ranks])
            assert np.array_equal(pos, OS.layout_index(lay, S, P_r, r))


@pytest.mark.parametrize("layout", ["zigzag", "striped"])
def test_bf16_usp_gqa_exercise_2k(layout):
    """The handbook's exercise shape: 32 query heads on 8 KV heads over 16
    ranks = 8-way Ulysses x 2-way ring, one KV head per rank, 2048 tokens;
    every rank, every row."""
    S, Hq, Hkv, P_u, P_r = 2048, 32, 8, 8, 2
    announce(f"bf16 USP S={S} Hq={Hq} Hkv={Hkv} P_u={P_u} P_r={P_r} {layout}")
    q, k, v = make_qkv(S=S, H=Hq, D=128, seed=17, dtype=torch.bfloat16, Hkv=Hkv)
    ro, rl = oracle_rows(q, k, v, None)
    order = input_order(layout, S, P_r)
    ot = torch.from_numpy(order)
    qd, kd, vd = dev(q[ot], k[ot], v[ot])
    out, lse = Guarded(S, Hq, 128), Guarded(Hq, S)
    cp.cp_usp_fwd(qd, kd, vd, P_u, P_r, layout, -1, out=out.t, lse=lse.t)
    torch.cuda.synchronize()
    out.check(), lse.check()
    compare(out.t, lse.t, ro[order], rl[:, order], BF16_OUT_TOL, BF16_LSE_TOL, "all ranks")
    lay = cp.LAYOUTS[layout]
    for r in range(P_r):
        o, l = run_group(qd, kd, vd, P_u, P_r, layout, r)
        idx = OS.layout_index(lay, S, P_r, r)
        compare(o, l, ro[idx], rl[:, idx], BF16_OUT_TOL, BF16_LSE_TOL, f"group {r}")


def test_bf16_usp_rank_writes_only_its_head_share():
    S, Hq, Hkv, P_u, P_r, rank = 512, 8, 4, 4, 2, 6     # u = 2, r = 1
    announce(f"bf16 USP S={S} rank {rank} head-share isolation")
    q, k, v = make_qkv(S=S, H=Hq, D=128, seed=19, dtype=torch.bfloat16, Hkv=Hkv)
    qd, kd, vd = dev(q, k, v)
    out = torch.full((S // P_r, Hq, 128), 7.0, device=DEV)
    lse = torch.full((Hq, S // P_r), 7.0, device=DEV)
    cp.cp_usp_fwd(qd, kd, vd, P_u, P_r, "zigzag", rank, out=out, lse=lse)
    torch.cuda.synchronize()
    keep = torch.ones(Hq, dtype=torch.bool)
    keep[4:6] = False
    assert bool((out[:, keep] == 7.0).all()) and bool((lse[keep] == 7.0).all())
    idx = OS.layout_index(OS.ZIGZAG, S, P_r, 1)
    ro, rl = oracle_rows(q, k, v, idx)
    compare(out[:, 4:6], lse[4:6], ro[:, 4:6], rl[4:6], BF16_OUT_TOL, BF16_LSE_TOL, "rank 6")


@pytest.mark.parametrize("layout,rank", [("zigzag", 13), ("striped", 2)])
def test_full_usp_rank_share_128k(layout, rank):
    """131072 tokens, 32 query heads on 8 KV heads, 8 x 2 ranks: one rank's
    share in the configuration the benchmark times, sampled rows."""
    S, Hq, Hkv, P_u, P_r = 131072, 32, 8, 8, 2
    u, r = rank % P_u, rank // P_u
    announce(f"bf16 USP S={S} Hq={Hq} Hkv={Hkv} {P_u}x{P_r} {layout} rank {rank} (sampled rows)")
    q, k, v = make_qkv(S=S, H=Hq, D=128, seed=0, dtype=torch.bfloat16, Hkv=Hkv)
    qd, kd, vd = dev(q, k, v)
    if layout == "striped":
        ot = torch.from_numpy(striped_order(S, P_r)).to(DEV)
        qd, kd, vd = (x[ot].contiguous() for x in (qd, kd, vd))
    rows = S // P_r
    out, lse = Guarded(rows, Hq, 128), Guarded(Hq, rows)
    cp.cp_usp_fwd(qd, kd, vd, P_u, P_r, layout, rank, out=out.t, lse=lse.t)
    torch.cuda.synchronize()
    out.check(), lse.check()
    del qd, kd, vd
    hs = slice(u * Hq // P_u, (u + 1) * Hq // P_u)
    local = chunk_edge_rows(rows, rows // 2, 10, seed=21 + rank)
    pos = OS.layout_index(cp.LAYOUTS[layout], S, P_r, r)
    ro, rl = oracle_rows(q, k, v, pos[local])
    lt = torch.from_numpy(local).to(DEV)
    o = out.t[lt][:, hs].double().cpu().numpy()
    lv = lse.t[hs][:, lt].double().cpu().numpy()
    compare(o, lv, ro[:, hs], rl[hs], BF16_OUT_TOL, BF16_LSE_TOL, f"128K USP {layout} rank {rank}")


# ------------------------------------------------------------- backward
from test_gpu_bwd import BF16_GRAD_REL, F32_GRAD_TOL, grads_compare, ring_rank_oracle  # noqa: E402


def usp_rank_bwd_oracle(q, k, v, dout, P_u, P_r, layout, rank):
    """dq of the rank's group rows (head share u) and its dk / dv (head share
    u), from the oracle ring backward on the head-sliced tensors."""
    Hq, Hkv = q.shape[1], k.shape[1]
    u, r = rank % P_u, rank // P_u
    hs = slice(u * Hq // P_u, (u + 1) * Hq // P_u)
    ks = slice(u * Hkv // P_u, (u + 1) * Hkv // P_u)
    gq, gk, gv = ring_rank_oracle(q[:, hs].contiguous(), k[:, ks].contiguous(),
                                  v[:, ks].contiguous(), dout[:, hs].contiguous(), P_r,
                                  cp.LAYOUTS[layout], r)
    return hs, ks, gq, gk, gv


@pytest.mark.parametrize("layout", ["contiguous", "zigzag", "striped"])
@pytest.mark.parametrize("P_u,P_r", [(2, 2), (4, 2)])
def test_f32_usp_bwd_page_inputs(layout, P_u, P_r):
    announce(f"f32 USP bwd P_u={P_u} P_r={P_r} {layout} on make_qkv() (Hkv=4)")
    q, _, _ = make_qkv()
    _, k, v = make_qkv(H=4, seed=3)
    dout = make_qkv(seed=5)[0]
    S = 32
    order = input_order(layout, S, P_r)
    ot = torch.from_numpy(order)
    qd, kd, vd = dev(q[ot], k[ot], v[ot])
    # every rank at once against the single-pass gradient
    out, lse = cp.cp_usp_fwd(qd, kd, vd, P_u, P_r, layout, -1)
    dq, dk, dv = Guarded(S, 8, 16), Guarded(S, 4, 16), Guarded(S, 4, 16)
    cp.cp_usp_bwd(qd, kd, vd, out, lse, dout[ot].to(DEV).contiguous(), P_u, P_r, layout, -1,
                  dq=dq.t, dk=dk.t, dv=dv.t)
    torch.cuda.synchronize()
    for g in (dq, dk, dv):
        g.check()
    qn, kn, vn, dn = (x.double().numpy() for x in (q, k, v, dout))
    ro, rl = OA.attention(qn, kn, vn)
    want = OA.attention_bwd(qn, kn, vn, dn, ro, rl)
    grads_compare((dq.t, dk.t, dv.t), [w[order] for w in want], F32_GRAD_TOL, f"{layout} all")
    np.testing.assert_allclose(OS.usp_bwd(q, k, v, dout, P_u, P_r, cp.LAYOUTS[layout])[0],
                               want[0], atol=1e-12)
    # each rank: its group's forward rows, its head share of the gradients
    lay = cp.LAYOUTS[layout]
    for rank in range(P_u * P_r):
        r = rank // P_u
        o, l = run_group(qd, kd, vd, P_u, P_r, layout, r)
        idx = torch.from_numpy(OS.layout_index(lay, S, P_r, r).astype(np.int64))
        gq = torch.full((S // P_r, 8, 16), 7.0, device=DEV)
        gk = torch.full((S, 4, 16), 7.0, device=DEV)
        gv = torch.full((S, 4, 16), 7.0, device=DEV)
        cp.cp_usp_bwd(qd, kd, vd, o, l, dout[idx].to(DEV).contiguous(), P_u, P_r, layout, rank,
                      dq=gq, dk=gk, dv=gv)
        torch.cuda.synchronize()
        hs, ks, wq, wk, wv = usp_rank_bwd_oracle(q, k, v, dout, P_u, P_r, layout, rank)
        grads_compare((gq[:, hs], gk[:, ks], gv[:, ks]), (wq, wk, wv), F32_GRAD_TOL,
                      f"{layout} rank {rank}")
        other = torch.ones(8, dtype=torch.bool)
        other[hs] = False
        assert bool((gq[:, other] == 7.0).all())


@pytest.mark.parametrize("layout", ["zigzag", "striped"])
def test_bf16_usp_bwd_gqa_exercise_2k(layout):
    """32 query heads on 8 KV heads, 8 x 2 ranks, 2048 tokens: every rank
    at once against the single-pass gradient, and rank 13 alone."""
    S, Hq, Hkv, P_u, P_r = 2048, 32, 8, 8, 2
    announce(f"bf16 USP bwd S={S} Hq={Hq} Hkv={Hkv} {P_u}x{P_r} {layout}")
    q, k, v = make_qkv(S=S, H=Hq, D=128, seed=41, dtype=torch.bfloat16, Hkv=Hkv)
    dout = make_qkv(S=S, H=Hq, D=128, seed=42, dtype=torch.bfloat16)[0]
    order = input_order(layout, S, P_r)
    ot = torch.from_numpy(order)
    qd, kd, vd = dev(q[ot], k[ot], v[ot])
    out, lse = cp.cp_usp_fwd(qd, kd, vd, P_u, P_r, layout, -1)
    dq, dk, dv = cp.cp_usp_bwd(qd, kd, vd, out, lse, dout[ot].to(DEV).contiguous(), P_u, P_r,
                               layout, -1)
    torch.cuda.synchronize()
    want = OS.usp_bwd(q, k, v, dout, P_u, P_r, cp.LAYOUTS[layout])
    grads_compare((dq, dk, dv), [w[order] for w in want], BF16_GRAD_REL, f"{layout} all",
                  rel=True)
    rank = 13
    r = rank // P_u
    o, l = run_group(qd, kd, vd, P_u, P_r, layout, r)
    idx = torch.from_numpy(OS.layout_index(cp.LAYOUTS[layout], S, P_r, r).astype(np.int64))
    gq, gk, gv = cp.cp_usp_bwd(qd, kd, vd, o, l, dout[idx].to(DEV).contiguous(), P_u, P_r,
                               layout, rank)
    torch.cuda.synchronize()
    hs, ks, wq, wk, wv = usp_rank_bwd_oracle(q, k, v, dout, P_u, P_r, layout, rank)
    grads_compare((gq[:, hs], gk[:, ks], gv[:, ks]), (wq, wk, wv), BF16_GRAD_REL,
                  f"{layout} rank {rank}", rel=True)


# ------------------------------------------------------------- padding
from test_gpu_padding import expected, input_positions, out_positions, to_input  # noqa: E402


@pytest.mark.parametrize("layout", ["contiguous", "zigzag", "striped"])
def test_f32_usp_padded_page_inputs(layout):
    """29 rows of the page's make_qkv() (8 query heads on 4 KV heads) over
    2 x 2 ranks: no ring split divides 29.  All ranks at once and every
    group, real rows against the single pass and the padded-USP oracle,
    padding rows (0, -inf); then the backward of all ranks."""
    S, P_u, P_r = 29, 2, 2
    announce(f"f32 USP padded S={S} P_u={P_u} P_r={P_r} {layout}")
    q, _, _ = (x[:S] for x in make_qkv())
    _, k, v = (x[:S] for x in make_qkv(H=4, seed=3))
    dout = make_qkv(seed=5)[0][:S]
    ipos = input_positions(layout, S, P_r)
    qd, kd, vd = (to_input(x, ipos, S) for x in (q, k, v))
    lay = cp.LAYOUTS[layout]
    ro, rl = OA.attention(q, k, v)
    po, pl, ppos = OS.usp_padded(q, k, v, P_u, P_r, lay)
    out, lse = cp.cp_usp_fwd(qd, kd, vd, P_u, P_r, layout, -1, seq_len=S)
    torch.cuda.synchronize()
    wo, wl = expected(ro, rl, ipos, S)
    compare(out, lse, wo, wl, F32_TOL, F32_TOL, f"{layout} all ranks")
    for r in range(P_r):
        opos = out_positions(layout, S, P_r, r)
        rows = len(opos)
        o, l = Guarded(rows, 8, 16), Guarded(8, rows)
        for u in range(P_u):
            cp.cp_usp_fwd(qd, kd, vd, P_u, P_r, layout, r * P_u + u, out=o.t, lse=l.t, seq_len=S)
        torch.cuda.synchronize()
        o.check(), l.check()
        wo, wl = expected(ro, rl, opos, S)
        compare(o.t, l.t, wo, wl, F32_TOL, F32_TOL, f"{layout} group {r}")
        real = torch.from_numpy(np.nonzero(opos < S)[0])
        compare(o.t[real], l.t[:, real], po[r], pl[r], F32_TOL, F32_TOL, f"{layout} group {r} oracle")
    # backward of every rank at once: the single-pass gradient on the real rows
    dd = to_input(dout, ipos, S)
    dd = torch.where(torch.isnan(dd), torch.zeros_like(dd), dd)
    gq, gk, gv = cp.cp_usp_bwd(qd, kd, vd, out, lse, dd, P_u, P_r, layout, -1, seq_len=S)
    torch.cuda.synchronize()
    qn, kn, vn, dn = (x.double().numpy() for x in (q, k, v, dout))
    want = OA.attention_bwd(qn, kn, vn, dn, ro, rl)
    real = np.nonzero(ipos < S)[0]
    rt = torch.from_numpy(real)
    grads_compare((gq[rt], gk[rt], gv[rt]), [w[ipos[real]] for w in want], F32_GRAD_TOL,
                  f"{layout} bwd")
    pad = torch.from_numpy(np.nonzero(ipos >= S)[0])
    for g in (gq, gk, gv):
        assert bool((g[pad] == 0).all())


@pytest.mark.parametrize("layout", ["zigzag", "striped"])
def test_bf16_usp_padded_gqa_exercise(layout):
    """1999 tokens, 32 query heads on 8 KV heads, 8 x 2 ranks (the ring
    split padded): every rank at once against the C oracle."""
    S, Hq, Hkv, P_u, P_r = 1999, 32, 8, 8, 2
    announce(f"bf16 USP padded S={S} Hq={Hq} Hkv={Hkv} {P_u}x{P_r} {layout}")
    q, k, v = make_qkv(S=S, H=Hq, D=128, seed=47, dtype=torch.bfloat16, Hkv=Hkv)
    ro, rl = oracle_rows(q, k, v, None)
    ipos = input_positions(layout, S, P_r)
    qd, kd, vd = (to_input(x, ipos, S) for x in (q, k, v))
    out, lse = cp.cp_usp_fwd(qd, kd, vd, P_u, P_r, layout, -1, seq_len=S)
    torch.cuda.synchronize()
    wo, wl = expected(ro, rl, ipos, S)
    compare(out, lse, wo, wl, BF16_OUT_TOL, BF16_LSE_TOL, f"{layout} all ranks")
