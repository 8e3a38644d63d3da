"""HIP path against the oracle, element by element, through the C-ABI.

Tolerances (max abs error against the float64 oracle on the same input
bytes): float32 path 1e-5 for out and lse; bf16 path (float32
accumulation) 1e-2 for out and 1e-3 for lse; repacks and index maps bit
exact.  Fully-masked rows must give exactly (0, -inf).

Small cases compare every output.  The full-size workloads (32K, 64K and
128K tokens, 32 heads, D = 128) run in the launch configuration the
benchmark times and compare a seeded sample of rows -- the first and last
row of every chunk plus uniform draws -- recomputed one by one by the C
oracle.  Every output buffer sits between guard regions filled with a
sentinel, checked after each call.
"""
import functools
import sys

import numpy as np
import pytest
import torch

import context_parallelism_cp_amd as cp
from oracle import attention as OA
from oracle import native
from oracle import schedules as OS
from seeded_inputs import make_qkv, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
F32_TOL = 1e-5
BF16_OUT_TOL = 1e-2
BF16_LSE_TOL = 1e-3
SENTINEL = 12345.0
GUARD = 1024  # floats on each side


def announce(msg):
    print(f"[gpu case] {msg}", flush=True)
    sys.stdout.flush()


class Guarded:
    """A float32 device tensor with sentinel-filled guard regions around it."""

    def __init__(self, *shape):
        n = int(np.prod(shape))
        self.buf = torch.full((n + 2 * GUARD,), SENTINEL, device=DEV, dtype=torch.float32)
        self.t = self.buf[GUARD:GUARD + n].view(*shape)

    def check(self):
        g = torch.cat([self.buf[:GUARD], self.buf[-GUARD:]])
        assert bool((g == SENTINEL).all()), "a kernel wrote outside its output buffer"


def compare(out, lse, ref_out, ref_lse, tol_out, tol_lse, what=""):
    o = out.detach().double().cpu().numpy() if torch.is_tensor(out) else out
    lv = lse.detach().double().cpu().numpy() if torch.is_tensor(lse) else lse
    assert np.array_equal(np.isneginf(lv), np.isneginf(ref_lse)), f"{what}: -inf pattern of lse"
    assert not np.isnan(o).any() and not np.isnan(lv).any(), f"{what}: NaN"
    fin = np.isfinite(ref_lse)
    err_l = float(np.abs(lv[fin] - ref_lse[fin]).max()) if fin.any() else 0.0
    err_o = float(np.abs(o - ref_out).max()) if o.size else 0.0
    print(f"    {what}: max|dout| = {err_o:.3e}, max|dlse| = {err_l:.3e}", flush=True)
    assert err_o <= tol_out, f"{what}: out error {err_o}"
    assert err_l <= tol_lse, f"{what}: lse error {err_l}"
    empty = np.isneginf(ref_lse).T  # [rows, H]
    assert np.all(o[empty] == 0.0), f"{what}: fully-masked rows must be 0"


def dev(*ts):
    return [t.to(DEV).contiguous() for t in ts]


# ----------------------------------------------------------------- float32
def test_f32_block_single_pass_page_inputs():
    announce("f32 block fwd, make_qkv() S=32 H=8 D=16")
    q, k, v = make_qkv()
    out, lse = Guarded(32, 8, 16), Guarded(8, 32)
    cp.cp_attn_block_fwd(*dev(q, k, v), out.t, lse.t)
    torch.cuda.synchronize()
    out.check(), lse.check()
    ro, rl = OA.attention(q, k, v)
    compare(out.t, lse.t, ro, rl, F32_TOL, F32_TOL, "page inputs")


@pytest.mark.parametrize("Sq,Sk,Hq,Hkv,D,qo,ko,causal", [
    (37, 53, 4, 2, 16, 20, 5, True),
    (37, 53, 4, 2, 16, 0, 0, False),
    (130, 70, 2, 1, 128, 100, 90, True),
    (65, 129, 3, 3, 40, 64, 0, True),
    (10, 10, 2, 2, 16, 0, 7, True),      # first rows see no key
    (5, 8, 2, 2, 16, 0, 100, True),      # no row sees a key
])
def test_f32_block_offsets_and_ragged(Sq, Sk, Hq, Hkv, D, qo, ko, causal):
    announce(f"f32 block fwd Sq={Sq} Sk={Sk} Hq={Hq} Hkv={Hkv} D={D} qo={qo} ko={ko} causal={causal}")
    q, _, _ = make_qkv(S=Sq, H=Hq, D=D, seed=Sq)
    _, k, v = make_qkv(S=Sk, H=Hkv, D=D, seed=Sk + 1)
    out, lse = Guarded(Sq, Hq, D), Guarded(Hq, Sq)
    cp.cp_attn_block_fwd(*dev(q, k, v), out.t, lse.t, q_offset=qo, k_offset=ko, causal=causal)
    torch.cuda.synchronize()
    out.check(), lse.check()
    ro, rl = OA.attention(q, k, v, causal=causal, q_offset=qo, k_offset=ko)
    compare(out.t, lse.t, ro, rl, F32_TOL, F32_TOL, "f32 block")


def test_f32_empty_kv():
    announce("f32 block fwd Sk=0")
    q, k, v = make_qkv(S=8, H=2, D=16)
    out, lse = Guarded(8, 2, 16), Guarded(2, 8)
    cp.cp_attn_block_fwd(q.to(DEV), k[:0].to(DEV), v[:0].to(DEV), out.t, lse.t)
    torch.cuda.synchronize()
    assert bool((out.t == 0).all()) and bool(torch.isneginf(lse.t).all())


@pytest.mark.parametrize("layout", ["contiguous", "zigzag"])
def test_f32_ring_page_inputs(layout):
    announce(f"f32 ring P=4 {layout} on make_qkv()")
    q, k, v = make_qkv()
    ro, rl = OA.attention(q, k, v)
    dq, dk, dv = dev(q, k, v)
    out, lse = Guarded(32, 8, 16), Guarded(8, 32)
    cp.cp_ring_fwd(dq, dk, dv, 4, layout, -1, out=out.t, lse=lse.t)
    torch.cuda.synchronize()
    out.check(), lse.check()
    compare(out.t, lse.t, ro, rl, F32_TOL, F32_TOL, f"{layout} all ranks")
    lay = cp.LAYOUTS[layout]
    for r in range(4):
        o2, l2 = Guarded(8, 8, 16), Guarded(8, 8)
        cp.cp_ring_fwd(dq, dk, dv, 4, layout, r, out=o2.t, lse=l2.t)
        torch.cuda.synchronize()
        o2.check(), l2.check()
        idx = OS.layout_index(lay, 32, 4, r)
        compare(o2.t, l2.t, ro[idx], rl[:, idx], F32_TOL, F32_TOL, f"{layout} rank {r}")


def striped_order(S, P):
    """Natural positions of the rows of a striped-order tensor: the ranks'
    shards back to back."""
    return np.concatenate([OS.layout_index(OS.STRIPED, S, P, r) for r in range(P)])


@pytest.mark.parametrize("causal", [True, False])
def test_f32_striped_ring_page_inputs(causal):
    announce(f"f32 ring P=4 striped causal={causal} on make_qkv()")
    q, k, v = make_qkv()
    ro, rl = OA.attention(q, k, v, causal=causal)
    perm = striped_order(32, 4)
    pt = torch.from_numpy(perm)
    dq, dk, dv = dev(q[pt], k[pt], v[pt])
    out, lse = Guarded(32, 8, 16), Guarded(8, 32)
    cp.cp_ring_fwd(dq, dk, dv, 4, "striped", -1, causal=causal, out=out.t, lse=lse.t)
    torch.cuda.synchronize()
    out.check(), lse.check()
    compare(out.t, lse.t, ro[perm], rl[:, perm], F32_TOL, F32_TOL, "striped all ranks")
    for r in range(4):
        o2, l2 = Guarded(8, 8, 16), Guarded(8, 8)
        cp.cp_ring_fwd(dq, dk, dv, 4, "striped", r, causal=causal, out=o2.t, lse=l2.t)
        torch.cuda.synchronize()
        o2.check(), l2.check()
        idx = OS.layout_index(OS.STRIPED, 32, 4, r)
        compare(o2.t, l2.t, ro[idx], rl[:, idx], F32_TOL, F32_TOL, f"striped rank {r}")


def test_f32_ring_noncausal():
    announce("f32 ring P=3 zigzag non-causal")
    q, k, v = make_qkv(S=48, H=2, D=16, seed=4)
    ro, rl = OA.attention(q, k, v, causal=False)
    out, lse = cp.cp_ring_fwd(*dev(q, k, v), 3, "zigzag", -1, causal=False)
    torch.cuda.synchronize()
    compare(out, lse, ro, rl, F32_TOL, F32_TOL, "non-causal ring")


def test_f32_ulysses_page_inputs():
    announce("f32 Ulysses P=4 on make_qkv()")
    q, k, v = make_qkv()
    P = 4
    dq, dk, dv = dev(q, k, v)
    heads = [cp.cp_seq_to_head(x, P, -1) for x in (dq, dk, dv)]
    torch.cuda.synchronize()
    ref_heads = [OS.seq_to_head([x.numpy()[r * 8:(r + 1) * 8] for r in range(P)], P)
                 for x in (q, k, v)]
    for got, want in zip(heads, ref_heads):
        for p in range(P):
            assert np.array_equal(got[p].cpu().numpy(), want[p])   # bit exact
    assert tuple(heads[0][0].shape) == (32, 2, 16)
    outs = torch.empty(P, 32, 2, 16, device=DEV)
    for p in range(P):
        o, _ = cp.cp_attn_block_fwd(heads[0][p], heads[1][p], heads[2][p])
        outs[p] = o
    y = torch.full((32, 8, 16), SENTINEL, device=DEV)
    cp.cp_head_to_seq(outs, y, P, -1)
    torch.cuda.synchronize()
    ro, _ = OA.attention(q, k, v)
    compare(y, np.zeros((8, 32)), ro, np.zeros((8, 32)), F32_TOL, F32_TOL, "Ulysses out")
    # one rank at a time gives the same bytes
    y2 = torch.full((32, 8, 16), SENTINEL, device=DEV)
    for p in range(P):
        hp = cp.cp_seq_to_head(dq, P, p)
        assert torch.equal(hp, heads[0][p])
        cp.cp_head_to_seq(outs[p].contiguous(), y2, P, p)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    back = torch.empty_like(dq)
    cp.cp_head_to_seq(heads[0], back, P, -1)
    torch.cuda.synchronize()
    assert torch.equal(back, dq)


# ------------------------------------------------------------------ merge
@pytest.mark.parametrize("Sq,H,D", [(33, 3, 128), (100, 8, 16), (7, 2, 256), (5, 1, 4)])
def test_merge_against_oracle(Sq, H, D):
    announce(f"lse merge Sq={Sq} H={H} D={D}")
    g = torch.Generator().manual_seed(Sq * H + D)
    o1, o2 = torch.randn(Sq, H, D, generator=g), torch.randn(Sq, H, D, generator=g)
    l1, l2 = torch.randn(H, Sq, generator=g) * 4, torch.randn(H, Sq, generator=g) * 4
    l1[0, 0] = -float("inf")                    # one side empty
    l2[-1, -1] = -float("inf")
    l1[0, -1] = l2[0, -1] = -float("inf")       # both empty
    o1[-1, 0] = 0.0
    o2[-1, 0] = 0.0
    ro, rl = OA.lse_merge(o1, l1, o2, l2)
    out, lse = Guarded(Sq, H, D), Guarded(H, Sq)
    cp.cp_lse_merge(*dev(o1, l1, o2, l2), out.t, lse.t)
    torch.cuda.synchronize()
    out.check(), lse.check()
    compare(out.t, lse.t, ro, rl, F32_TOL, F32_TOL, "merge")
    # in place: o, lse alias o1, lse1
    d1, dl1, d2, dl2 = dev(o1, l1, o2, l2)
    cp.cp_lse_merge(d1, dl1, d2, dl2, d1, dl1)
    torch.cuda.synchronize()
    compare(d1, dl1, ro, rl, F32_TOL, F32_TOL, "merge in place")


@pytest.mark.parametrize("Sq,H", [(8192, 32), (131072, 66)])
def test_merge_full_size_sampled(Sq, H):
    """The merge at the size a ring rank folds per step (8192 rows x 32
    heads, one loop trip per wavefront) and past the grid's cap (131072 x 66
    (row, head) groups, so wavefronts loop), out of place and in place;
    seeded sampled rows against the oracle's merge of the same rows (the
    merge is row-independent)."""
    D = 128
    announce(f"lse merge full size Sq={Sq} H={H} D={D} (sampled rows)")
    g = torch.Generator(device=DEV).manual_seed(Sq + H)
    o1 = torch.randn(Sq, H, D, device=DEV, generator=g)
    o2 = torch.randn(Sq, H, D, device=DEV, generator=g)
    l1 = torch.randn(H, Sq, device=DEV, generator=g) * 4
    l2 = torch.randn(H, Sq, device=DEV, generator=g) * 4
    l1[:, ::97] = -float("inf")
    l2[:, ::89] = -float("inf")
    rows = sample_rows(Sq, 48, seed=Sq).to(DEV)
    ref_in = [t.cpu() for t in (o1[rows], l1[:, rows], o2[rows], l2[:, rows])]
    ro, rl = OA.lse_merge(*ref_in)
    out, lse = torch.empty_like(o1), torch.empty_like(l1)
    cp.cp_lse_merge(o1, l1, o2, l2, out, lse)
    torch.cuda.synchronize()
    compare(out[rows], lse[:, rows], ro, rl, F32_TOL, F32_TOL, "merge full size")
    del out, lse
    cp.cp_lse_merge(o1, l1, o2, l2, o1, l1)     # in place
    torch.cuda.synchronize()
    compare(o1[rows], l1[:, rows], ro, rl, F32_TOL, F32_TOL, "merge full size in place")


# ------------------------------------------------------------------ bf16
def oracle_rows(q, k, v, rows, **kw):
    return native.attention_rows(q, k, v, rows=rows, **kw)


@pytest.mark.parametrize("Sq,Sk,Hq,Hkv,qo,ko,causal", [
    (300, 517, 4, 2, 400, 100, True),
    (300, 517, 4, 2, 0, 0, False),
    (128, 128, 2, 2, 0, 0, True),
    (257, 300, 2, 1, 0, 200, True),    # rows 0..198 see no key
    (64, 1000, 8, 2, 999, 0, True),
    (1, 1, 1, 1, 5, 5, True),
    # query heads per KV head 8 (one wavefront per head in a workgroup), 2,
    # and 16 (more than a workgroup's wavefronts: one head per workgroup)
    (300, 517, 8, 1, 400, 100, True),
    (130, 700, 16, 2, 50, 0, True),
    (97, 333, 6, 3, 0, 0, False),
    (257, 300, 16, 1, 0, 200, True),
])
def test_bf16_block_small(Sq, Sk, Hq, Hkv, qo, ko, causal):
    announce(f"bf16 block fwd Sq={Sq} Sk={Sk} Hq={Hq} Hkv={Hkv} qo={qo} ko={ko} causal={causal}")
    q, _, _ = make_qkv(S=Sq, H=Hq, D=128, seed=Sq, dtype=torch.bfloat16)
    _, k, v = make_qkv(S=Sk, H=Hkv, D=128, seed=Sk + 7, dtype=torch.bfloat16)
    out, lse = Guarded(Sq, Hq, 128), Guarded(Hq, Sq)
    cp.cp_attn_block_fwd(*dev(q, k, v), out.t, lse.t, q_offset=qo, k_offset=ko, causal=causal)
    torch.cuda.synchronize()
    out.check(), lse.check()
    ro, rl = oracle_rows(q, k, v, None, causal=causal, q_offset=qo, k_offset=ko)
    compare(out.t, lse.t, ro, rl, BF16_OUT_TOL, BF16_LSE_TOL, "bf16 block")


def random_block_case(case):
    """Seeded random block shape: lengths that need not fill a tile, GQA
    ratios that pack into a workgroup (1, 2, 4, 8) and ones that do not (3,
    16), offsets in either order, causal or not."""
    rng = np.random.default_rng(1000 + case)
    Hkv = int(rng.choice([1, 2]))
    group = int(rng.choice([1, 2, 3, 4, 8, 16 // Hkv]))
    Sq, Sk = int(rng.integers(1, 521)), int(rng.integers(1, 601))
    qo, ko = int(rng.integers(0, 1200)), int(rng.integers(0, 1200))
    return Sq, Sk, Hkv * group, Hkv, qo, ko, bool(rng.integers(0, 2))


@pytest.mark.parametrize("case", range(24))
def test_bf16_block_random_shapes(case):
    Sq, Sk, Hq, Hkv, qo, ko, causal = random_block_case(case)
    announce(f"bf16 block fwd random case {case}: Sq={Sq} Sk={Sk} Hq={Hq} Hkv={Hkv} "
             f"qo={qo} ko={ko} causal={causal}")
    q, _, _ = make_qkv(S=Sq, H=Hq, D=128, seed=2000 + case, dtype=torch.bfloat16)
    _, k, v = make_qkv(S=Sk, H=Hkv, D=128, seed=3000 + case, dtype=torch.bfloat16)
    out, lse = Guarded(Sq, Hq, 128), Guarded(Hq, Sq)
    cp.cp_attn_block_fwd(*dev(q, k, v), out.t, lse.t, q_offset=qo, k_offset=ko, causal=causal)
    torch.cuda.synchronize()
    out.check(), lse.check()
    ro, rl = oracle_rows(q, k, v, None, causal=causal, q_offset=qo, k_offset=ko)
    compare(out.t, lse.t, ro, rl, BF16_OUT_TOL, BF16_LSE_TOL, f"bf16 block random {case}")


def score_dynamics_inputs(kind, Sq, Sk, H, seed):
    """bf16 q, k, v whose scores stress the running max of the streaming
    softmax: "growing" -- key norms rise along the sequence, so a row's max
    climbs many times past the lazy-rescale threshold within one launch;
    "negative" -- every score near -100 nats (exponentials against a zero
    reference would underflow to 0); "sink" -- key 0 dominates every row by
    about 60 nats, the rest of the row is negligible beside it.  v is
    drawn at half scale: in a row dominated by one key the bf16 rounding of
    the probabilities alone moves the output by up to 2^-9 max|v|, which for
    unit-scale v (max about 5) is the whole 1e-2 tolerance; the stress is
    on the scores."""
    q, _, _ = make_qkv(S=Sq, H=H, D=128, seed=seed, dtype=torch.float32)
    _, k, v = make_qkv(S=Sk, H=H, D=128, seed=seed + 1, dtype=torch.float32)
    u = make_qkv(S=1, H=H, D=128, seed=seed + 2, dtype=torch.float32)[0]  # [1, H, D]
    if kind == "growing":
        q = 2.0 * q
        k = k * (1.0 + 8.0 * torch.arange(Sk, dtype=torch.float32) / Sk)[:, None, None]
    elif kind == "negative":
        q = 3.0 * u + 0.5 * q
        k = -3.0 * u + 0.5 * k
    elif kind == "sink":
        k = 0.3 * k
        k[0] = 6.0 * u[0]
        q = 0.3 * q + u
    v = 0.5 * v
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


@pytest.mark.parametrize("kind", ["growing", "negative", "sink"])
@pytest.mark.parametrize("qo,ko,causal", [(0, 0, True), (1500, 0, True), (0, 0, False),
                                          (0, 700, True)])
def test_bf16_block_score_dynamics(kind, qo, ko, causal):
    """Rows whose running max rises mid-launch (raise + rescale), rows far
    below zero, a dominant first key, and rows with no visible key for the
    first tiles (qo < ko) next to rows that have one."""
    Sq, Sk, H = 1000, 2000, 2
    announce(f"bf16 block fwd score dynamics {kind} qo={qo} ko={ko} causal={causal}")
    q, k, v = score_dynamics_inputs(kind, Sq, Sk, H, seed=31)
    out, lse = Guarded(Sq, H, 128), Guarded(H, Sq)
    cp.cp_attn_block_fwd(*dev(q, k, v), out.t, lse.t, q_offset=qo, k_offset=ko, causal=causal)
    torch.cuda.synchronize()
    out.check(), lse.check()
    ro, rl = oracle_rows(q, k, v, None, causal=causal, q_offset=qo, k_offset=ko)
    compare(out.t, lse.t, ro, rl, BF16_OUT_TOL, BF16_LSE_TOL, f"bf16 {kind}")


def test_bf16_block_empty_kv():
    announce("bf16 block fwd Sk=0")
    q, k, v = make_qkv(S=130, H=2, D=128, dtype=torch.bfloat16)
    out, lse = cp.cp_attn_block_fwd(q.to(DEV), k[:0].to(DEV), v[:0].to(DEV))
    torch.cuda.synchronize()
    assert bool((out == 0).all()) and bool(torch.isneginf(lse).all())


@pytest.mark.parametrize("layout", ["contiguous", "zigzag"])
def test_bf16_ring_small_every_rank(layout):
    S, H, P = 2048, 4, 4
    announce(f"bf16 ring S={S} H={H} P={P} {layout}")
    q, k, v = make_qkv(S=S, H=H, D=128, seed=11, dtype=torch.bfloat16)
    ro, rl = oracle_rows(q, k, v, None)
    dq, dk, dv = dev(q, k, v)
    out, lse = Guarded(S, H, 128), Guarded(H, S)
    cp.cp_ring_fwd(dq, dk, dv, P, layout, -1, out=out.t, lse=lse.t)
    torch.cuda.synchronize()
    out.check(), lse.check()
    compare(out.t, lse.t, ro, rl, BF16_OUT_TOL, BF16_LSE_TOL, f"{layout} all ranks")
    for r in range(P):
        o2, l2 = cp.cp_ring_fwd(dq, dk, dv, P, layout, r)
        torch.cuda.synchronize()
        idx = OS.layout_index(cp.LAYOUTS[layout], S, P, r)
        compare(o2, l2, ro[idx], rl[:, idx], BF16_OUT_TOL, BF16_LSE_TOL, f"{layout} rank {r}")


@pytest.mark.parametrize("S,Hq,Hkv,P", [(2048, 4, 4, 4), (3000, 8, 2, 8), (256, 2, 1, 2)])
def test_bf16_striped_ring_every_rank(S, Hq, Hkv, P):
    """Striped order in, striped order out; each rank's share in its local
    order.  S = 3000 over 8 ranks gives 375-row shards (ragged tiles)."""
    announce(f"bf16 ring S={S} Hq={Hq} Hkv={Hkv} P={P} striped")
    q, k, v = make_qkv(S=S, H=Hq, D=128, seed=13, dtype=torch.bfloat16, Hkv=Hkv)
    ro, rl = oracle_rows(q, k, v, None)
    perm = striped_order(S, P)
    pt = torch.from_numpy(perm)
    dq, dk, dv = dev(q[pt], k[pt], v[pt])
    out, lse = Guarded(S, Hq, 128), Guarded(Hq, S)
    cp.cp_ring_fwd(dq, dk, dv, P, "striped", -1, out=out.t, lse=lse.t)
    torch.cuda.synchronize()
    out.check(), lse.check()
    compare(out.t, lse.t, ro[perm], rl[:, perm], BF16_OUT_TOL, BF16_LSE_TOL, "striped all ranks")
    for r in range(P):
        o2, l2 = cp.cp_ring_fwd(dq, dk, dv, P, "striped", r)
        torch.cuda.synchronize()
        idx = OS.layout_index(OS.STRIPED, S, P, r)
        compare(o2, l2, ro[idx], rl[:, idx], BF16_OUT_TOL, BF16_LSE_TOL, f"striped rank {r}")


# ------------------------------------------------------- full-size workloads
@functools.lru_cache(maxsize=1)
def inputs_cached(S, H, Hkv):
    q, k, v = make_qkv(S=S, H=H, D=128, seed=0, dtype=torch.bfloat16, Hkv=Hkv)
    return q, k, v


def chunk_edge_rows(n_local, chunk, n_random, seed):
    edges = set()
    for c0 in range(0, n_local, chunk):
        edges.update({c0, c0 + chunk - 1})
    rnd = sample_rows(n_local, n_random + 2, seed=seed).tolist()
    return np.array(sorted(edges.union(rnd)), dtype=np.int64)


def check_share(out, lse, q, k, v, positions, local_rows, what):
    ro, rl = oracle_rows(q, k, v, positions[local_rows])
    o = out[torch.from_numpy(local_rows).to(DEV)].double().cpu().numpy()
    lv = lse[:, torch.from_numpy(local_rows).to(DEV)].double().cpu().numpy()
    compare(o, lv, ro, rl, BF16_OUT_TOL, BF16_LSE_TOL, what)


def test_full_ring_32k_all_ranks():
    S, H, P = 32768, 32, 8
    announce(f"bf16 ring S={S} H={H} P={P} zigzag, all ranks (sampled rows)")
    q, k, v = inputs_cached(S, H, H)
    dq, dk, dv = dev(q, k, v)
    out, lse = Guarded(S, H, 128), Guarded(H, S)
    cp.cp_ring_fwd(dq, dk, dv, P, "zigzag", -1, out=out.t, lse=lse.t)
    torch.cuda.synchronize()
    out.check(), lse.check()
    rows = chunk_edge_rows(S, S // (2 * P), 16, seed=2)
    check_share(out.t, lse.t, q, k, v, np.arange(S), rows, "32K all ranks")


@pytest.mark.parametrize("layout,rank", [("contiguous", 3), ("contiguous", 0), ("zigzag", 0),
                                         ("zigzag", 3)])
def test_full_rank_share_64k(layout, rank):
    S, H, P = 65536, 32, 4
    announce(f"bf16 ring S={S} H={H} P={P} {layout} rank {rank} (sampled rows)")
    q, k, v = inputs_cached(S, H, H)
    dq, dk, dv = dev(q, k, v)
    out, lse = Guarded(S // P, H, 128), Guarded(H, S // P)
    cp.cp_ring_fwd(dq, dk, dv, P, layout, rank, out=out.t, lse=lse.t)
    torch.cuda.synchronize()
    out.check(), lse.check()
    lay = cp.LAYOUTS[layout]
    chunk = S // P if layout == "contiguous" else S // (2 * P)
    rows = chunk_edge_rows(S // P, chunk, 8, seed=3 + rank)
    check_share(out.t, lse.t, q, k, v, OS.layout_index(lay, S, P, rank), rows,
                f"64K {layout} rank {rank}")


@pytest.mark.parametrize("rank", [0, 7])
def test_full_rank_share_128k(rank):
    S, H, P = 131072, 32, 8
    announce(f"bf16 ring S={S} H={H} P={P} zigzag rank {rank} (sampled rows)")
    q, k, v = inputs_cached(S, H, H)
    dq, dk, dv = dev(q, k, v)
    out, lse = Guarded(S // P, H, 128), Guarded(H, S // P)
    cp.cp_ring_fwd(dq, dk, dv, P, "zigzag", rank, out=out.t, lse=lse.t)
    torch.cuda.synchronize()
    out.check(), lse.check()
    rows = chunk_edge_rows(S // P, S // (2 * P), 8, seed=5 + rank)
    check_share(out.t, lse.t, q, k, v, OS.layout_index(cp.CP_LAYOUT_ZIGZAG, S, P, rank), rows,
                f"128K zigzag rank {rank}")


@pytest.mark.parametrize("rank", [0, 7])
def test_full_striped_rank_share_128k(rank):
    S, H, P = 131072, 32, 8
    announce(f"bf16 ring S={S} H={H} P={P} striped rank {rank} (sampled rows)")
    q, k, v = inputs_cached(S, H, H)
    pt = torch.from_numpy(striped_order(S, P)).to(DEV)
    dq, dk, dv = (x[pt].contiguous() for x in dev(q, k, v))
    out, lse = Guarded(S // P, H, 128), Guarded(H, S // P)
    cp.cp_ring_fwd(dq, dk, dv, P, "striped", rank, out=out.t, lse=lse.t)
    torch.cuda.synchronize()
    out.check(), lse.check()
    del dq, dk, dv
    rows = chunk_edge_rows(S // P, S // P, 12, seed=9 + rank)
    check_share(out.t, lse.t, q, k, v, OS.layout_index(OS.STRIPED, S, P, rank), rows,
                f"128K striped rank {rank}")


def test_full_ulysses_gqa_128k():
    S, Hq, Hkv, P, p = 131072, 32, 8, 8, 5
    announce(f"Ulysses GQA S={S} Hq={Hq} Hkv={Hkv} P={P} rank {p} (sampled rows)")
    q, k, v = inputs_cached(S, Hq, Hkv)
    dq, dk, dv = dev(q, k, v)
    ql = cp.cp_seq_to_head(dq, P, p)
    kl = cp.cp_seq_to_head(dk, P, p)
    vl = cp.cp_seq_to_head(dv, P, p)
    torch.cuda.synchronize()
    # bit-exact head-slice identity
    assert torch.equal(ql, dq[:, 4 * p:4 * p + 4]) and torch.equal(kl, dk[:, p:p + 1])
    out_l, lse_l = Guarded(S, 4, 128), Guarded(4, S)
    cp.cp_attn_block_fwd(ql, kl, vl, out_l.t, lse_l.t)
    y = torch.full((S, Hq, 128), SENTINEL, device=DEV)
    cp.cp_head_to_seq(out_l.t, y, P, p)
    torch.cuda.synchronize()
    out_l.check(), lse_l.check()
    untouched = torch.cat([y[:, :4 * p], y[:, 4 * p + 4:]], dim=1)
    assert bool((untouched == SENTINEL).all())
    assert torch.equal(y[:, 4 * p:4 * p + 4], out_l.t)
    rows = chunk_edge_rows(S, S // P, 16, seed=9)
    ro, rl = oracle_rows(q[:, 4 * p:4 * p + 4].contiguous(), k[:, p:p + 1].contiguous(),
                         v[:, p:p + 1].contiguous(), rows)
    idx = torch.from_numpy(rows).to(DEV)
    compare(y[idx][:, 4 * p:4 * p + 4].double().cpu().numpy(),
            lse_l.t[:, idx].double().cpu().numpy(), ro, rl, BF16_OUT_TOL, BF16_LSE_TOL,
            "Ulysses GQA 128K")
    # the same rows from the GQA definition over all 32 query heads (head h reads KV h // 4)
    ro_all, _ = oracle_rows(q, k, v, rows[:4])
    np.testing.assert_allclose(ro_all[:, 4 * p:4 * p + 4], ro[:4], atol=1e-12)


def test_full_block_128k_32_heads():
    """The whole 131072-token sequence as one causal block on 32 heads (the
    launch `bench.py --part block` times): sampled rows -- the edges of
    every 16384-row stretch and random ones -- against the C oracle."""
    S, H = 131072, 32
    announce(f"one causal block S={S} H={H} (sampled rows)")
    q, k, v = inputs_cached(S, H, H)
    dq, dk, dv = dev(q, k, v)
    out, lse = Guarded(S, H, 128), Guarded(H, S)
    cp.cp_attn_block_fwd(dq, dk, dv, out.t, lse.t)
    torch.cuda.synchronize()
    out.check(), lse.check()
    rows = chunk_edge_rows(S, 16384, 16, seed=11)
    ro, rl = oracle_rows(q, k, v, rows)
    idx = torch.from_numpy(rows).to(DEV)
    compare(out.t[idx].double().cpu().numpy(), lse.t[:, idx].double().cpu().numpy(), ro, rl,
            BF16_OUT_TOL, BF16_LSE_TOL, "one causal block 128K x 32 heads")


def test_ulysses_16way_with_kv_replication():
    """The handbook exercise's 16-way Ulysses on 32 query heads and 8 KV heads:
    KV heads copied to two ranks each (bit-exact), every rank's local
    attention, and head->seq back; equal to the single pass."""
    S, Hq, Hkv, P = 2048, 32, 8, 16
    announce(f"Ulysses {P}-way with KV replication S={S} Hq={Hq} Hkv={Hkv}")
    q, k, v = make_qkv(S=S, H=Hq, D=128, seed=23, dtype=torch.bfloat16, Hkv=Hkv)
    dq, dk, dv = dev(q, k, v)
    kr = cp.cp_kv_seq_to_head(dk, P, -1)
    torch.cuda.synchronize()
    for p in range(P):
        assert torch.equal(kr[p][:, 0], dk[:, p // 2])
    ro, rl = oracle_rows(q, k, v, None)
    out = Guarded(S, Hq, 128)
    for p in range(P):
        ql = cp.cp_seq_to_head(dq, P, p)
        kl = cp.cp_kv_seq_to_head(dk, P, p)
        vl = cp.cp_kv_seq_to_head(dv, P, p)
        assert torch.equal(kl, kr[p])
        o, l = cp.cp_attn_block_fwd(ql, kl, vl)
        cp.cp_head_to_seq(o, out.t, P, p)
        torch.cuda.synchronize()
        compare(o, l, ro[:, 2 * p:2 * p + 2], rl[2 * p:2 * p + 2], BF16_OUT_TOL, BF16_LSE_TOL,
                f"rank {p}")
    out.check()
    o = out.t.double().cpu().numpy()
    assert float(np.abs(o - ro).max()) <= BF16_OUT_TOL


def test_one_million_tokens_rank_share():
    """Large positions: 2^20 tokens, 4 heads, zigzag ring over 8 ranks, the
    last rank's share (chunks 7 and 8 of 16, positions up to 589823 seeing up
    to that many keys); sampled rows recomputed by the C oracle."""
    S, H, P, rank = 1 << 20, 4, 8, 7
    announce(f"bf16 ring S={S} H={H} P={P} zigzag rank {rank} (sampled rows)")
    q, k, v = make_qkv(S=S, H=H, D=128, seed=3, dtype=torch.bfloat16)
    dq, dk, dv = dev(q, k, v)
    out, lse = Guarded(S // P, H, 128), Guarded(H, S // P)
    cp.cp_ring_fwd(dq, dk, dv, P, "zigzag", rank, out=out.t, lse=lse.t)
    torch.cuda.synchronize()
    out.check(), lse.check()
    del dq, dk, dv
    rows = chunk_edge_rows(S // P, S // (2 * P), 6, seed=13)
    check_share(out.t, lse.t, q, k, v, OS.layout_index(cp.CP_LAYOUT_ZIGZAG, S, P, rank), rows,
                "1M zigzag rank 7")
