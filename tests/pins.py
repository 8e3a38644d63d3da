"""Pins: checks that tie the oracle to facts other than itself.

Each function takes the implementation under test (so that the mutation
tests can hand in deliberately broken copies) and raises AssertionError
when a fact fails.  Facts used:

* brute force over pure-Python loops, normalising exp(s_j) by their plain
  sum (no max shift, no log-sum-exp route);
* closed forms: with q = 0 every visible score is 0, so lse = ln(n) and
  out is the mean of the visible v rows; with one key, out = v_0 and
  lse = q.k/sqrt(D); with v = 1 every non-empty row's out is 1;
* a library special case: ``torch.nn.functional.scaled_dot_product_attention``
  (float64, CPU) for offsets 0, causal or not, with GQA heads;
* the merge identity over disjoint key sets and the global-max route of
  the "Sequence Parallel vs Context Parallel" blog, section 3.2;
* the values fixed by the handbook page "上下文并行：Ring Attention 与
  Ulysses": work per rank, KV blocks per rank, Ulysses shapes (text
  fixtures under tests/golden with their citations).
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name: str) -> dict[str, list[float]]:
    vals = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *nums = line.split()
            vals[key] = [float(x) for x in nums]
    return vals


# Set to np.float32 to round every random input to float32 first, so that an
# implementation that reads float32 inputs sees exactly the pins' numbers.
ROUND_INPUTS = None


def rand(shape, seed):
    x = np.random.default_rng(seed).standard_normal(shape)
    return x if ROUND_INPUTS is None else x.astype(ROUND_INPUTS).astype(np.float64)


# ----------------------------------------------------------- brute force
def brute_force(q, k, v, causal, q_offset, k_offset, qpos=None, kpos=None, kvalid=None):
    """Pure-Python loops: p_j = exp(s_j) / sum_j exp(s_j) over visible j.
    Positions are q_offset + i and k_offset + j unless given explicitly;
    keys with kvalid[j] False are never visible."""
    Sq, Hq, D = q.shape
    Sk, Hkv, _ = k.shape
    group = Hq // Hkv
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(Sq)]
    lse = [[-math.inf] * Sq for _ in range(Hq)]
    for h in range(Hq):
        g = h // group
        for i in range(Sq):
            e = []
            for j in range(Sk):
                pq = q_offset + i if qpos is None else int(qpos[i])
                pk = k_offset + j if kpos is None else int(kpos[j])
                if (causal and pk > pq) or (kvalid is not None and not kvalid[j]):
                    continue
                s = sum(float(q[i, h, d]) * float(k[j, g, d]) for d in range(D)) / math.sqrt(D)
                e.append((j, math.exp(s)))
            if not e:
                continue
            z = math.fsum(w for _, w in e)
            lse[h][i] = math.log(z)
            for d in range(D):
                out[i][h][d] = math.fsum(w / z * float(v[j, g, d]) for j, w in e)
    return np.array(out), np.array(lse)


def pin_brute_force(attn, cases=None):
    cases = cases or [
        # Sq, Sk, Hq, Hkv, D, causal, q_offset, k_offset
        (5, 7, 2, 1, 3, True, 4, 0),
        (6, 6, 2, 2, 4, True, 0, 0),
        (4, 9, 4, 2, 2, True, 3, 5),
        (3, 5, 1, 1, 5, False, 0, 0),
        (4, 4, 2, 1, 3, True, 0, 2),     # first rows see no key
    ]
    for n, (Sq, Sk, Hq, Hkv, D, causal, qo, ko) in enumerate(cases):
        q, k, v = rand((Sq, Hq, D), 3 * n), rand((Sk, Hkv, D), 3 * n + 1), rand((Sk, Hkv, D), 3 * n + 2)
        o, l = attn(q, k, v, causal=causal, q_offset=qo, k_offset=ko)
        ob, lb = brute_force(q, k, v, causal, qo, ko)
        np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
        assert np.array_equal(np.isinf(l), np.isinf(lb))
        np.testing.assert_allclose(np.where(np.isinf(lb), 0, l), np.where(np.isinf(lb), 0, lb),
                                   rtol=0, atol=1e-12)


def pin_attention_at(attn_at, attn):
    """Explicit positions: brute force on scattered positions (including
    rows that see no key), and offsets written as positions reduce to the
    offset form."""
    rng = np.random.default_rng(31)
    for n, (Sq, Sk, Hq, Hkv, D) in enumerate([(5, 7, 2, 1, 3), (6, 4, 4, 2, 2), (4, 6, 1, 1, 4)]):
        q, k, v = rand((Sq, Hq, D), 200 + n), rand((Sk, Hkv, D), 210 + n), rand((Sk, Hkv, D), 220 + n)
        qpos = rng.choice(np.arange(3, 40), Sq, replace=False)
        kpos = rng.choice(np.arange(0, 40), Sk, replace=False)
        kpos[0] = 0
        qpos[0] = 1                       # sees key 0 only if kpos holds 0 or 1
        qpos[-1] = -1                     # sees no key
        for causal in (True, False):
            o, l = attn_at(q, k, v, qpos, kpos, causal=causal)
            ob, lb = brute_force(q, k, v, causal, 0, 0, qpos=qpos, kpos=kpos)
            np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
            assert np.array_equal(np.isinf(l), np.isinf(lb))
            np.testing.assert_allclose(np.where(np.isinf(lb), 0, l), np.where(np.isinf(lb), 0, lb),
                                       rtol=0, atol=1e-12)
        kvalid = np.arange(Sk) % 3 != 1
        for causal in (True, False):
            o, l = attn_at(q, k, v, qpos, kpos, causal=causal, kvalid=kvalid)
            ob, lb = brute_force(q, k, v, causal, 0, 0, qpos=qpos, kpos=kpos, kvalid=kvalid)
            np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
            assert np.array_equal(np.isinf(l), np.isinf(lb))
        o, l = attn_at(q, k, v, np.arange(Sq) + 4, np.arange(Sk) + 2)
        o2, l2 = attn(q, k, v, causal=True, q_offset=4, k_offset=2)
        np.testing.assert_allclose(o, o2, atol=1e-14)
        np.testing.assert_allclose(l, l2, atol=1e-14)


def pin_striped(ring_striped, layout_index, striped, attn, cases=((4, 32), (8, 64), (3, 21), (2, 2))):
    """Striped split: every position owned once, rank r holding r, r+P, ...;
    the ring reproduces the single pass on every rank; the causal work of
    rank r is sum over its rows of (position + 1) visible keys, i.e.
    C*(r+1) + P*C*(C-1)/2, so ranks differ by C pairs at most."""
    for P, S in cases:
        C = S // P
        allpos = np.concatenate([layout_index(striped, S, P, r) for r in range(P)])
        assert sorted(allpos.tolist()) == list(range(S))
        for r in range(P):
            assert layout_index(striped, S, P, r).tolist() == [r + j * P for j in range(C)]
        q, k, v = (rand((S, 4, 8), 40 + P + i) for i in range(3))
        for causal in (True, False):
            ref_o, ref_l = attn(q, k, v, causal=causal)
            outs, lses, pairs = ring_striped(q, k, v, P, causal=causal)
            for r in range(P):
                idx = layout_index(striped, S, P, r)
                np.testing.assert_allclose(outs[r], ref_o[idx], rtol=0, atol=1e-12)
                np.testing.assert_allclose(lses[r], ref_l[:, idx], rtol=0, atol=1e-12)
                want = C * (r + 1) + P * C * (C - 1) // 2 if causal else C * S
                assert pairs[r] == want
            if causal:
                assert sum(pairs) == S * (S + 1) // 2


def pin_striped_plan(ring_plan, layout_index, striped, diag, full, attn, attn_at):
    """Every striped pair is computed, and in local coordinates it is the
    plain causal mask at the plan's offsets, q 0 and k 1 when the source rank
    comes after the query rank, 0 otherwise: rank r's row j is position
    r + jP, so key j' of rank s is visible iff s + j'P <= r + jP."""
    for P in (2, 4, 8):
        S = 8 * P
        plan = ring_plan(S, P, striped, -1)
        assert len(plan) == P * P and all(p[8] == diag for p in plan)
        assert all(p[8] == full for p in ring_plan(S, P, striped, -1, causal=False))
        q, k, v = (rand((S, 2, 4), 500 + i) for i in range(3))
        for (r, _t, _qc, src, qo, ko, *_rest) in plan:
            qi, ki = layout_index(striped, S, P, r), layout_index(striped, S, P, src)
            o, l = attn_at(q[qi], k[ki], v[ki], qi, ki)
            o2, l2 = attn(q[qi], k[ki], v[ki], q_offset=qo, k_offset=ko)
            np.testing.assert_allclose(o, o2, atol=1e-14)
            np.testing.assert_allclose(l, l2, atol=1e-14)


# ----------------------------------------------------------- closed forms
def pin_zero_query(attn):
    """q = 0: lse_i = ln n_i, out_i = mean of visible v_j, n_i = number visible."""
    for (Sq, Sk, qo, ko, Hq, Hkv) in [(6, 9, 3, 1, 2, 1), (8, 8, 0, 0, 4, 2), (5, 4, 0, 3, 2, 2)]:
        D = 3
        q = np.zeros((Sq, Hq, D))
        k, v = rand((Sk, Hkv, D), 11), rand((Sk, Hkv, D), 12)
        o, l = attn(q, k, v, causal=True, q_offset=qo, k_offset=ko)
        group = Hq // Hkv
        for i in range(Sq):
            n = min(max(qo + i - ko + 1, 0), Sk)
            for h in range(Hq):
                if n == 0:
                    assert l[h, i] == -np.inf and np.all(o[i, h] == 0)
                else:
                    assert abs(l[h, i] - math.log(n)) < 1e-12
                    np.testing.assert_allclose(o[i, h], v[:n, h // group].mean(axis=0), atol=1e-12)


def pin_ones_value(attn):
    Sq, Sk, D = 7, 10, 4
    q, k = rand((Sq, 2, D), 21), rand((Sk, 2, D), 22)
    o, l = attn(q, k, np.ones((Sk, 2, D)), causal=True, q_offset=2, k_offset=0)
    np.testing.assert_allclose(o, 1.0, atol=1e-12)


def pin_single_key(attn):
    D = 5
    q, k, v = rand((3, 2, D), 31), rand((1, 2, D), 32), rand((1, 2, D), 33)
    o, l = attn(q, k, v, causal=True, q_offset=7, k_offset=7)
    for h in range(2):
        for i in range(3):
            np.testing.assert_allclose(o[i, h], v[0, h], atol=1e-12)
            assert abs(l[h, i] - float(q[i, h] @ k[0, h]) / math.sqrt(D)) < 1e-12


def pin_sdpa(attn):
    """Offsets 0: torch's scaled_dot_product_attention in float64 on the CPU
    (its is_causal mask is the lower triangle including the diagonal; its
    enable_gqa maps query head h to KV head h // (Hq/Hkv))."""
    import torch.nn.functional as F
    for causal in (True, False):
        for (S, Hq, Hkv, D) in [(9, 4, 2, 8), (16, 2, 2, 16)]:
            q, k, v = rand((S, Hq, D), 41), rand((S, Hkv, D), 42), rand((S, Hkv, D), 43)
            o, _ = attn(q, k, v, causal=causal)
            tq, tk, tv = (torch.from_numpy(x).permute(1, 0, 2).unsqueeze(0) for x in (q, k, v))
            ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                 enable_gqa=(Hq != Hkv))
            np.testing.assert_allclose(o, ref[0].permute(1, 0, 2).numpy(), atol=1e-12)


# ----------------------------------------------------------------- merge
def pin_merge_identity(attn, merge):
    """attn over K1 u K2 == merge(attn over K1, attn over K2), both orders,
    and associativity over three parts; -inf parts are the identity."""
    Sq, Sk, H, D, qo = 6, 12, 2, 4, 8
    q, k, v = rand((Sq, H, D), 51), rand((Sk, H, D), 52), rand((Sk, H, D), 53)
    full = attn(q, k, v, causal=True, q_offset=qo, k_offset=0)
    cuts = [0, 4, 9, Sk]
    parts = [attn(q, k[a:b], v[a:b], causal=True, q_offset=qo, k_offset=a)
             for a, b in zip(cuts[:-1], cuts[1:])]
    for (x, y) in [(0, 1), (1, 0)]:
        m = merge(*parts[x], *parts[y])
        ref = attn(q, k[:9], v[:9], causal=True, q_offset=qo, k_offset=0)
        np.testing.assert_allclose(m[0], ref[0], atol=1e-12)
        np.testing.assert_allclose(m[1], ref[1], atol=1e-12)
    left = merge(*merge(*parts[0], *parts[1]), *parts[2])
    right = merge(*parts[0], *merge(*parts[1], *parts[2]))
    for res in (left, right):
        np.testing.assert_allclose(res[0], full[0], atol=1e-12)
        np.testing.assert_allclose(res[1], full[1], atol=1e-12)
    # a part whose keys all lie after every query: lse = -inf, identity of the merge
    empty = attn(q, k[:3], v[:3], causal=True, q_offset=0, k_offset=100)
    assert np.all(np.isneginf(empty[1])) and np.all(empty[0] == 0)
    res = merge(*empty, *full)
    np.testing.assert_allclose(res[0], full[0], atol=0)
    np.testing.assert_allclose(res[1], full[1], atol=0)
    both = merge(*empty, *empty)
    assert np.all(np.isneginf(both[1])) and np.all(both[0] == 0)


def pin_global_max_route(attn, global_max_attn):
    Sq, Sk, H, D = 7, 11, 2, 3
    q, k, v = rand((Sq, H, D), 61), rand((Sk, H, D), 62), rand((Sk, H, D), 63)
    parts = [np.arange(0, 3), np.arange(3, 8), np.arange(8, 11)]
    a = attn(q, k, v, causal=True, q_offset=4, k_offset=0)
    b = global_max_attn(q, k, v, parts, causal=True, q_offset=4, k_offset=0)
    np.testing.assert_allclose(a[0], b[0], atol=1e-12)
    np.testing.assert_allclose(a[1], b[1], atol=1e-12)


# ----------------------------------------------------------- schedules
def pin_work(rank_chunks, causal_units, CONTIGUOUS, ZIGZAG):
    """The zigzag section's printed work per rank for P = 4 (golden), every
    chunk owned exactly once, and the closed forms 4r + 2 (contiguous) and
    2P (zigzag) that summing the diagonal-half block grid gives."""
    g = load_golden("work_p4.txt")
    P = 4
    assert [causal_units(rank_chunks(CONTIGUOUS, P, r), 2 * P) for r in range(P)] == g["contiguous"]
    assert [causal_units(rank_chunks(ZIGZAG, P, r), 2 * P) for r in range(P)] == g["zigzag"]
    for layout in (CONTIGUOUS, ZIGZAG):
        for PP in (2, 4, 8):
            owned = sorted(c for r in range(PP) for c in rank_chunks(layout, PP, r))
            assert owned == list(range(2 * PP))
            for r in range(PP):
                want = 4 * r + 2 if layout == CONTIGUOUS else 2 * PP
                assert causal_units(rank_chunks(layout, PP, r), 2 * PP) == want


def make_qkv_page():
    """The handbook's make_qkv(): manual_seed(0), then randn(32, 8, 16) x3."""
    torch.manual_seed(0)
    return torch.randn(32, 8, 16), torch.randn(32, 8, 16), torch.randn(32, 8, 16)


# -------------------------------------------------------------- backward
BWD_CASES = [
    # (Sq, Sk, Hq, Hkv, D, causal, q_offset, k_offset)
    (5, 6, 2, 1, 4, True, 3, 1),      # GQA, offsets, causal
    (4, 4, 2, 2, 3, False, 0, 0),     # non-causal
    (4, 5, 1, 1, 2, True, 0, 2),      # rows 0 and 1 see no key
]


def _loss_grad_fd(attn, q, k, v, dout, causal, qo, ko, eps=1e-6):
    """Central finite differences of sum(dout * attn(q, k, v).out)."""
    def loss(q_, k_, v_):
        return float(np.sum(dout * attn(q_, k_, v_, causal=causal, q_offset=qo,
                                         k_offset=ko)[0]))
    grads = []
    for which in range(3):
        x = [q, k, v][which]
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += eps
            args_m[which][idx] -= eps
            g[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        grads.append(g)
    return grads


def pin_bwd_finite_differences(attn, attn_bwd):
    """The backward is the derivative of the (pinned) forward: central
    differences of sum(dout * out) agree to the difference formula's
    accuracy, on every case of BWD_CASES."""
    for n, (Sq, Sk, Hq, Hkv, D, causal, qo, ko) in enumerate(BWD_CASES):
        q, k, v = rand((Sq, Hq, D), 60 + n), rand((Sk, Hkv, D), 70 + n), rand((Sk, Hkv, D), 80 + n)
        dout = rand((Sq, Hq, D), 90 + n)
        out, lse = attn(q, k, v, causal=causal, q_offset=qo, k_offset=ko)
        got = attn_bwd(q, k, v, dout, out, lse, causal=causal, q_offset=qo, k_offset=ko)
        want = _loss_grad_fd(attn, q, k, v, dout, causal, qo, ko)
        for g, w in zip(got, want):
            np.testing.assert_allclose(g, w, atol=1e-7)


def pin_bwd_at_finite_differences(attn_at, attn_bwd_at):
    """Explicit-position backward against central differences of the
    explicit-position forward, on scattered positions with a row that sees
    no key."""
    Sq, Sk, Hq, Hkv, D = 5, 6, 2, 1, 3
    q, k, v = rand((Sq, Hq, D), 301), rand((Sk, Hkv, D), 302), rand((Sk, Hkv, D), 303)
    dout = rand((Sq, Hq, D), 304)
    qpos = np.array([7, 2, 11, -3, 5])
    kpos = np.array([4, 0, 9, 12, 1, 6])
    for causal in (True, False):
        out, lse = attn_at(q, k, v, qpos, kpos, causal=causal)
        got = attn_bwd_at(q, k, v, dout, out, lse, qpos, kpos, causal=causal)

        def fwd(q_, k_, v_, causal, q_offset, k_offset):
            return attn_at(q_, k_, v_, qpos, kpos, causal=causal)
        want = _loss_grad_fd(fwd, q, k, v, dout, causal, 0, 0)
        for g, w in zip(got, want):
            np.testing.assert_allclose(g, w, atol=1e-7)


def pin_bwd_autograd(attn, attn_bwd):
    """Offsets 0: torch autograd through scaled_dot_product_attention in
    float64 on the CPU (a library special case of the same gradient)."""
    import torch.nn.functional as F
    for causal in (True, False):
        for (S, Hq, Hkv, D) in [(9, 4, 2, 8), (7, 2, 2, 4)]:
            q, k, v = rand((S, Hq, D), 101), rand((S, Hkv, D), 102), rand((S, Hkv, D), 103)
            dout = rand((S, Hq, D), 104)
            out, lse = attn(q, k, v, causal=causal)
            got = attn_bwd(q, k, v, dout, out, lse, causal=causal)
            tq, tk, tv = (torch.from_numpy(x).permute(1, 0, 2).unsqueeze(0).requires_grad_()
                          for x in (q, k, v))
            o = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                               enable_gqa=(Hq != Hkv))
            o.backward(torch.from_numpy(dout).permute(1, 0, 2).unsqueeze(0))
            for g, t in zip(got, (tq, tk, tv)):
                np.testing.assert_allclose(g, t.grad[0].permute(1, 0, 2).numpy(), atol=1e-12)


def pin_bwd_closed_forms(attn, attn_bwd):
    """Closed forms.  Equal value rows make out constant in q and k, so
    dq = dk = 0.  Over a single block (full rows) the row sums of ds vanish,
    so sum_j dk_j = 0 for every KV head, and sum_j dv_j = sum over rows that
    see a key (and the heads of the group) of dout_i."""
    Sq, Sk, Hq, Hkv, D, qo, ko = 6, 7, 4, 2, 5, 2, 0
    q, k = rand((Sq, Hq, D), 111), rand((Sk, Hkv, D), 112)
    dout = rand((Sq, Hq, D), 113)
    v = np.broadcast_to(rand((1, Hkv, D), 114), (Sk, Hkv, D)).copy()
    out, lse = attn(q, k, v, causal=True, q_offset=qo, k_offset=ko)
    dq, dk, _ = attn_bwd(q, k, v, dout, out, lse, causal=True, q_offset=qo, k_offset=ko)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    v = rand((Sk, Hkv, D), 115)
    Sq, qo, ko = 6, 0, 2                          # rows 0 and 1 see no key
    q, dout = rand((Sq, Hq, D), 116), rand((Sq, Hq, D), 117)
    out, lse = attn(q, k, v, causal=True, q_offset=qo, k_offset=ko)
    _, dk, dv = attn_bwd(q, k, v, dout, out, lse, causal=True, q_offset=qo, k_offset=ko)
    group = Hq // Hkv
    for g in range(Hkv):
        np.testing.assert_allclose(dk[:, g, :].sum(axis=0), 0.0, atol=1e-12)
        want = sum(dout[i, h, :] for h in range(g * group, (g + 1) * group)
                   for i in range(Sq) if qo + i >= ko)
        np.testing.assert_allclose(dv[:, g, :].sum(axis=0), want, atol=1e-12)


def pin_bwd_ring(ring_bwd, attn, attn_bwd, contiguous, zigzag, striped=None):
    """The ring's block gradients, each taken with the rows' final (out,
    lse), add up to the single-pass gradient (the pages ask that gradients
    with context parallelism match a single card)."""
    q, k, v = (x.double().numpy() for x in make_qkv_page())
    dout = rand(q.shape, 121)
    out, lse = attn(q, k, v, causal=True)
    want = attn_bwd(q, k, v, dout, out, lse, causal=True)
    layouts = (contiguous, zigzag) + ((striped,) if striped is not None else ())
    for layout in layouts:
        got = ring_bwd(q, k, v, dout, 4, layout, True)
        for g, w in zip(got, want):
            np.testing.assert_allclose(g, w, atol=1e-12)
    # a length no split divides (padding): 30 rows over 4 ranks
    q, k, v, dout = q[:30], k[:30], v[:30], dout[:30]
    for causal in (True, False):
        out, lse = attn(q, k, v, causal=causal)
        want = attn_bwd(q, k, v, dout, out, lse, causal=causal)
        for layout in layouts:
            got = ring_bwd(q, k, v, dout, 4, layout, causal)
            for g, w in zip(got, want):
                np.testing.assert_allclose(g, w, atol=1e-12)


# ------------------------------------------------------------ USP hybrid
def pin_usp(usp, ring_fns, ulysses, layout_ids, attn):
    """USP (Ulysses inside groups, ring across them): every rank's rows equal
    the single pass for every layout, including the handbook's GQA exercise
    (32 query heads on 8 KV heads, 16 ranks = 8-way Ulysses x 2-way ring,
    one KV head per rank, where Ulysses alone stops at 8); every position is
    owned once; P_u = 1 is the plain ring and P_r = 1 plain Ulysses."""
    cases = [(64, 8, 4, 2, 2), (64, 8, 4, 4, 2), (64, 8, 2, 2, 4), (32, 32, 8, 8, 2)]
    for n, (S, Hq, Hkv, P_u, P_r) in enumerate(cases):
        D = 4 if Hq > 8 else 8
        q, k, v = rand((S, Hq, D), 600 + n), rand((S, Hkv, D), 610 + n), rand((S, Hkv, D), 620 + n)
        for causal in (True, False):
            ro, rl = attn(q, k, v, causal=causal)
            for layout in layout_ids:
                outs, lses, pos = usp(q, k, v, P_u, P_r, layout, causal=causal)
                assert len(outs) == P_u * P_r
                assert sorted(np.concatenate(pos).tolist()) == list(range(S))
                for o, l, p in zip(outs, lses, pos):
                    assert o.shape == (S // (P_u * P_r), Hq, D)
                    np.testing.assert_allclose(o, ro[p], rtol=0, atol=1e-12)
                    np.testing.assert_allclose(l, rl[:, p], rtol=0, atol=1e-12)
    # reductions
    q, k, v = rand((32, 4, 8), 630), rand((32, 2, 8), 631), rand((32, 2, 8), 632)
    for layout, ring in zip(layout_ids, ring_fns):
        outs, lses, _ = usp(q, k, v, 1, 4, layout)
        r_outs, r_lses = ring(q, k, v, 4)[:2]
        for a, b in zip(outs, r_outs):
            np.testing.assert_allclose(a, b, atol=1e-14)
        for a, b in zip(lses, r_lses):
            np.testing.assert_allclose(a, b, atol=1e-14)
    outs, _, pos = usp(q, k, v, 2, 1, layout_ids[0])
    u_outs, _ = ulysses(q, k, v, 2)
    for a, b in zip(outs, u_outs):
        np.testing.assert_allclose(a, b, atol=1e-14)
    # the GQA limit: more Ulysses ranks than KV heads is refused
    try:
        usp(q, k, v, 4, 1, layout_ids[0])
    except ValueError:
        pass
    else:
        raise AssertionError("P_u > Hkv accepted")


# ---------------------------------------------------------------- padding
def pin_padding(ring_padded, padded_length, layout_index, ring_plan, layouts, zigzag, attn,
                rings):
    """Padding (pad to a multiple of the split, compute, discard): the real
    rows equal the single pass for every layout, causal or not, when the
    split does not divide S -- including ranks made only of padding -- and
    every real position is owned once; with no padding it is the plain ring;
    the padded lengths round up to P (2P for zigzag); the plan's real row
    counts add up to the real positions of each rank."""
    assert padded_length(30, 4, layouts[0]) == 32 and padded_length(30, 4, zigzag) == 32
    assert padded_length(37, 8, zigzag) == 48 and padded_length(37, 8, layouts[0]) == 40
    assert padded_length(32, 4, zigzag) == 32 and padded_length(0, 4, zigzag) == 0
    for n, (S, P) in enumerate([(30, 4), (37, 8), (5, 8), (13, 3)]):
        q, k, v = rand((S, 4, 8), 700 + n), rand((S, 2, 8), 710 + n), rand((S, 2, 8), 720 + n)
        for causal in (True, False):
            ro, rl = attn(q, k, v, causal=causal)
            for layout in layouts:
                outs, lses, pos = ring_padded(q, k, v, P, layout, causal)
                assert sorted(np.concatenate(pos).tolist()) == list(range(S))
                for r, (o, l, p) in enumerate(zip(outs, lses, pos)):
                    idx = layout_index(layout, S, P, r)
                    assert idx.size == padded_length(S, P, layout) // P
                    assert np.array_equal(p, idx[idx < S])
                    np.testing.assert_allclose(o, ro[p], rtol=0, atol=1e-12)
                    np.testing.assert_allclose(l, rl[:, p], rtol=0, atol=1e-12)
                plan = ring_plan(S, P, layout, -1, causal)
                for r in range(P):
                    idx = layout_index(layout, S, P, r)
                    lens = {}
                    for (rr, _t, qc, _kc, _qo, _ko, lq, _lk, _kind) in plan:
                        if rr == r:
                            lens[qc] = lq
                    assert sum(lens.values()) == int(np.sum(idx < S))
    q, k, v = rand((32, 4, 8), 730), rand((32, 2, 8), 731), rand((32, 2, 8), 732)
    for layout, ring in zip(layouts, rings):
        outs, lses, _ = ring_padded(q, k, v, 4, layout, True)
        r_outs, r_lses = ring(q, k, v, 4)[:2]
        for a, b in zip(outs, r_outs):
            np.testing.assert_allclose(a, b, atol=1e-13)


def pin_usp_bwd(usp_bwd, attn, attn_bwd, layouts):
    """The USP backward equals the single-pass gradient for every layout,
    GQA included (8 query heads on 4 KV heads over 2 x 2 and 4 x 2 ranks)."""
    for n, (S, Hq, Hkv, P_u, P_r) in enumerate([(32, 8, 4, 2, 2), (32, 8, 4, 4, 2),
                                                (48, 4, 2, 2, 3)]):
        q, k, v = rand((S, Hq, 8), 800 + n), rand((S, Hkv, 8), 810 + n), rand((S, Hkv, 8), 820 + n)
        dout = rand((S, Hq, 8), 830 + n)
        for causal in (True, False):
            out, lse = attn(q, k, v, causal=causal)
            want = attn_bwd(q, k, v, dout, out, lse, causal=causal)
            for layout in layouts:
                got = usp_bwd(q, k, v, dout, P_u, P_r, layout, causal)
                for g, w in zip(got, want):
                    np.testing.assert_allclose(g, w, atol=1e-12)


def pin_usp_padded(usp_padded, usp, attn, layouts):
    """USP over a padded ring: the real rows equal the single pass for every
    layout (GQA, causal or not); with no padding it gives usp_attention's
    rows."""
    for n, (S, P_u, P_r) in enumerate([(30, 2, 2), (37, 2, 4), (13, 4, 3)]):
        q, k, v = rand((S, 8, 4), 900 + n), rand((S, 4, 4), 910 + n), rand((S, 4, 4), 920 + n)
        for causal in (True, False):
            ro, rl = attn(q, k, v, causal=causal)
            for layout in layouts:
                outs, lses, pos = usp_padded(q, k, v, P_u, P_r, layout, causal)
                assert sorted(np.concatenate(pos).tolist()) == list(range(S))
                for o, l, p in zip(outs, lses, pos):
                    np.testing.assert_allclose(o, ro[p], rtol=0, atol=1e-12)
                    np.testing.assert_allclose(l, rl[:, p], rtol=0, atol=1e-12)
    q, k, v = rand((32, 8, 4), 930), rand((32, 4, 4), 931), rand((32, 4, 4), 932)
    for layout in layouts:
        outs, _, pos = usp_padded(q, k, v, 2, 2, layout)
        u_outs, _, u_pos = usp(q, k, v, 2, 2, layout)
        for r in range(2):
            np.testing.assert_allclose(outs[r], np.concatenate(u_outs[2 * r:2 * r + 2]), atol=1e-13)
