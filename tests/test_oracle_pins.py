"""The oracle against its pins (CPU only).

Each test ties a function of ``oracle/`` to something other than itself:
brute force, closed forms, a library special case, the merge identity,
the global-max route, and the values fixed by the handbook page
"上下文并行：Ring Attention 与 Ulysses" (tests/golden).
"""
import math

import numpy as np
import pytest
import torch

import pins
from oracle import attention as A
from oracle import native
from oracle import schedules as R
from seeded_inputs import make_qkv


def c_attn(q, k, v, causal=True, q_offset=0, k_offset=0):
    """The C oracle with the numpy oracle's call shape (float32 inputs)."""
    t = [torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32) for x in (q, k, v)]
    return native.attention_rows(*t, causal=causal, q_offset=q_offset, k_offset=k_offset,
                                 n_threads=2)


@pytest.fixture
def f32_inputs():
    """Round the pins' random inputs to float32 (the C oracle reads float32)."""
    pins.ROUND_INPUTS = np.float32
    yield
    pins.ROUND_INPUTS = None


IMPLS = {"numpy": A.attention, "c": c_attn}


@pytest.mark.parametrize("impl", list(IMPLS))
def test_brute_force(impl, f32_inputs):
    pins.pin_brute_force(IMPLS[impl])


@pytest.mark.parametrize("impl", list(IMPLS))
def test_closed_forms(impl, f32_inputs):
    pins.pin_zero_query(IMPLS[impl])
    pins.pin_ones_value(IMPLS[impl])
    pins.pin_single_key(IMPLS[impl])


@pytest.mark.parametrize("impl", list(IMPLS))
def test_sdpa_special_case(impl, f32_inputs):
    pins.pin_sdpa(IMPLS[impl])


def test_merge_identity():
    pins.pin_merge_identity(A.attention, A.lse_merge)


def test_global_max_route():
    pins.pin_global_max_route(A.attention, A.attention_global_max)


def test_c_oracle_matches_numpy_on_rows_and_bf16():
    """Rows subsets, offsets, GQA and bf16 widening of the C oracle."""
    q, k, v = make_qkv(S=67, H=4, D=8, seed=5, dtype=torch.bfloat16, Hkv=2)
    ref_o, ref_l = A.attention(q, k, v, causal=True, q_offset=30, k_offset=3)
    rows = [0, 5, 17, 66]
    o, l = native.attention_rows(q, k, v, rows=rows, causal=True, q_offset=30, k_offset=3,
                                 n_threads=3)
    np.testing.assert_allclose(o, ref_o[rows], atol=1e-12)
    np.testing.assert_allclose(l, ref_l[:, rows], atol=1e-12)
    o_all, l_all = native.attention_rows(q, k, v, causal=True, q_offset=30, k_offset=3)
    np.testing.assert_allclose(o_all, ref_o, atol=1e-12)


def test_c_oracle_rejects_bad_arguments():
    q, k, v = make_qkv(S=8, H=3, D=4, Hkv=2)
    with pytest.raises(ValueError):
        native.attention_rows(q, k, v)           # 3 query heads over 2 KV heads
    q, k, v = make_qkv(S=8, H=2, D=4)
    with pytest.raises(ValueError):
        native.attention_rows(q, k, v, rows=[8])


# ------------------------------------------------------------- schedules
def test_work_model_golden():
    pins.pin_work(R.rank_chunks, R.causal_units, R.CONTIGUOUS, R.ZIGZAG)
    for P in (2, 4, 8, 16):
        assert all(R.causal_units(R.rank_chunks(R.ZIGZAG, P, r), 2 * P) == 2 * P
                   for r in range(P))


def test_page_make_qkv_is_the_seeded_generator():
    a = pins.make_qkv_page()
    b = make_qkv()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_ring_contiguous_equals_single_pass():
    q, k, v = make_qkv()
    ref_o, ref_l = A.attention(q, k, v)
    outs, lses, computed = R.ring_contiguous(q, k, v, P=4)
    assert computed == pins.load_golden("ring_counts_p4.txt")["counts"]
    C = 8
    for r in range(4):
        np.testing.assert_allclose(outs[r], ref_o[r * C:(r + 1) * C], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lses[r], ref_l[:, r * C:(r + 1) * C], rtol=0, atol=1e-12)


@pytest.mark.parametrize("P,S", [(4, 32), (8, 64), (2, 12)])
def test_ring_zigzag_equals_single_pass_and_balances(P, S):
    q, k, v = make_qkv(S=S, H=4, D=8, seed=P)
    ref_o, ref_l = A.attention(q, k, v)
    outs, lses, units = R.ring_zigzag(q, k, v, P=P)
    for r in range(P):
        idx = R.layout_index(R.ZIGZAG, S, P, r)
        np.testing.assert_allclose(outs[r], ref_o[idx], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lses[r], ref_l[:, idx], rtol=0, atol=1e-12)
        # the page: with the zigzag split every rank does the same work at every step
        assert units[r] == [2.0] * P
        assert sum(units[r]) == R.causal_units(R.rank_chunks(R.ZIGZAG, P, r), 2 * P)


def test_ring_noncausal_equals_single_pass():
    q, k, v = make_qkv(S=24, H=2, D=4, seed=9)
    ref_o, ref_l = A.attention(q, k, v, causal=False)
    outs, lses, computed = R.ring_contiguous(q, k, v, P=3, causal=False)
    assert computed == [3, 3, 3]
    for r in range(3):
        np.testing.assert_allclose(outs[r], ref_o[r * 8:(r + 1) * 8], atol=1e-12)
    outs, lses, _ = R.ring_zigzag(q, k, v, P=3, causal=False)
    for r in range(3):
        np.testing.assert_allclose(outs[r], ref_o[R.layout_index(R.ZIGZAG, 24, 3, r)], atol=1e-12)


def test_layout_index_matches_page_slices():
    S, P = 32, 4
    for r in range(P):
        assert R.layout_index(R.CONTIGUOUS, S, P, r).tolist() == list(range(r * 8, r * 8 + 8))
        zz = R.layout_index(R.ZIGZAG, S, P, r).tolist()
        assert zz == list(range(4 * r, 4 * r + 4)) + list(range(4 * (7 - r), 4 * (7 - r) + 4))
    # every position owned exactly once
    for layout in (R.CONTIGUOUS, R.ZIGZAG):
        allpos = np.concatenate([R.layout_index(layout, 64, 8, r) for r in range(8)])
        assert sorted(allpos.tolist()) == list(range(64))


@pytest.mark.parametrize("P", [4, 8])
def test_ring_plan_counts_and_coverage(P):
    S = 16 * P
    zz = R.ring_plan(S, P, R.ZIGZAG, -1)
    assert len(zz) == P * P * 4
    for r in range(P):
        mine = [p for p in zz if p[0] == r]
        n_comp = sum(1 for p in mine if p[8] != R.SKIP)
        assert n_comp == 2 * P + 1          # P=4: 9, P=8: 17 launches per rank
        units = sum(1.0 if p[8] == R.FULL else 0.5 for p in mine if p[8] != R.SKIP)
        assert units == R.causal_units(R.rank_chunks(R.ZIGZAG, P, r), 2 * P)
        # each (q chunk, k chunk <= q chunk) pair appears exactly once
        comp = sorted((p[2], p[3]) for p in mine if p[8] != R.SKIP)
        want = sorted((qc, kc) for qc in R.rank_chunks(R.ZIGZAG, P, r) for kc in range(qc + 1))
        assert comp == want
    cont = R.ring_plan(S, P, R.CONTIGUOUS, -1)
    counts = [sum(1 for p in cont if p[0] == r and p[8] != R.SKIP) for r in range(P)]
    assert counts == list(range(1, P + 1))


def test_ulysses_shapes_and_result():
    g = pins.load_golden("ulysses_shapes_p4.txt")
    q, k, v = make_qkv()
    outs, shapes = R.ulysses_attention(q, k, v, P=4)
    assert list(q[:8].shape) == g["input"]
    assert all(list(s) == g["attention"] for s in shapes)
    ref_o, _ = A.attention(q, k, v)
    for r in range(4):
        np.testing.assert_allclose(outs[r], ref_o[r * 8:(r + 1) * 8], rtol=0, atol=1e-12)


def test_ulysses_round_trip_and_head_slice_identity():
    S, H, D, P = 24, 8, 3, 4
    x = np.arange(S * H * D, dtype=np.float64).reshape(S, H, D)
    locals_ = [x[r * S // P:(r + 1) * S // P] for r in range(P)]
    heads = R.seq_to_head(locals_, P)
    for p in range(P):
        assert np.array_equal(heads[p], x[:, p * H // P:(p + 1) * H // P, :])
    back = R.head_to_seq(heads, P)
    assert np.array_equal(np.concatenate(back), x)


def test_ulysses_gqa_pins_head_mapping():
    """Ulysses with Hq=8, Hkv=2, P=2: rank p receives query heads 4p..4p+3
    and KV head p; its local attention must equal the single-pass GQA
    result, which fixes query head h -> KV head h // 4."""
    q, k, v = make_qkv(S=16, H=8, D=4, seed=3, Hkv=2)
    outs, _ = R.ulysses_attention(q, k, v, P=2)
    ref_o, _ = A.attention(q, k, v)
    for r in range(2):
        np.testing.assert_allclose(outs[r], ref_o[r * 8:(r + 1) * 8], atol=1e-12)
    lim = pins.load_golden("ulysses_gqa_limit.txt")
    assert lim["max_degree"][0] == lim["Hkv"][0]


def test_ulysses_kv_replication_exercise():
    """The exercise's answer for 16-way Ulysses on 32 query heads and 8 KV
    heads: copy every KV head to two ranks before the all-to-all.  Rank p
    then holds query heads 2p, 2p+1 and KV head p // 2, and the result is
    the single pass."""
    q, k, v = make_qkv(S=32, H=32, D=4, seed=5, Hkv=8)
    outs, shapes = R.ulysses_attention(q, k, v, P=16)
    ref_o, _ = A.attention(q, k, v)
    for r in range(16):
        np.testing.assert_allclose(outs[r], ref_o[2 * r:2 * (r + 1)], atol=1e-12)
    assert all(s_ == (32, 2, 4) for s_ in shapes)
    kr = R.replicate_kv(k.double().numpy(), 16)
    for p in range(16):
        assert np.array_equal(kr[:, p], k.double().numpy()[:, p // 2])
    with pytest.raises(ValueError):
        R.replicate_kv(np.zeros((4, 3, 2)), 8)


# ------------------------------------------------------------- backward
def test_bwd_finite_differences():
    pins.pin_bwd_finite_differences(A.attention, A.attention_bwd)


def test_bwd_autograd_special_case():
    pins.pin_bwd_autograd(A.attention, A.attention_bwd)


def test_bwd_closed_forms():
    pins.pin_bwd_closed_forms(A.attention, A.attention_bwd)


def test_ring_bwd_equals_single_pass():
    pins.pin_bwd_ring(R.ring_bwd, A.attention, A.attention_bwd, R.CONTIGUOUS, R.ZIGZAG, R.STRIPED)


def test_bwd_at_finite_differences():
    pins.pin_bwd_at_finite_differences(A.attention_at, A.attention_bwd_at)


# ------------------------------------------------------------- striped
def test_attention_at_brute_force_and_offsets():
    pins.pin_attention_at(A.attention_at, A.attention)


def test_striped_ring_equals_single_pass_and_balances():
    pins.pin_striped(R.ring_striped, R.layout_index, R.STRIPED, A.attention)


def test_striped_plan_local_offsets():
    pins.pin_striped_plan(R.ring_plan, R.layout_index, R.STRIPED, R.DIAG, R.FULL, A.attention,
                          A.attention_at)


def test_c_oracle_bwd_matches_numpy():
    """The C backward rows equal the (pinned) numpy backward: float32 and
    bfloat16 inputs, GQA, offsets with rows that see no key, causal or not."""
    for dtype in (torch.float32, torch.bfloat16):
        for (Sq, Sk, Hq, Hkv, D, causal, qo, ko) in [(9, 11, 4, 2, 8, True, 3, 5),
                                                      (7, 6, 2, 2, 4, False, 0, 0)]:
            g = torch.Generator().manual_seed(7)
            q, k, v, do = (torch.randn(s, generator=g).to(dtype)
                           for s in ((Sq, Hq, D), (Sk, Hkv, D), (Sk, Hkv, D), (Sq, Hq, D)))
            out, lse = A.attention(q, k, v, causal=causal, q_offset=qo, k_offset=ko)
            want = A.attention_bwd(q, k, v, do, out, lse, causal=causal, q_offset=qo, k_offset=ko)
            qr, kr = [Sq - 1, 0, 4], [Sk - 1, 2, 0]
            dq, dk, dv = native.attention_bwd_rows(q, k, v, do, qr, kr, causal=causal,
                                                   q_offset=qo, k_offset=ko, n_threads=2)
            np.testing.assert_allclose(dq, want[0][qr], atol=1e-10)
            np.testing.assert_allclose(dk, want[1][kr], atol=1e-10)
            np.testing.assert_allclose(dv, want[2][kr], atol=1e-10)


# ------------------------------------------------------------- USP hybrid
def test_usp_equals_single_pass_and_reduces():
    pins.pin_usp(R.usp_attention, (R.ring_contiguous, R.ring_zigzag, R.ring_striped),
                 R.ulysses_attention, (R.CONTIGUOUS, R.ZIGZAG, R.STRIPED), A.attention)


def test_usp_rank_numbering():
    """Ranks of one ring group are consecutive: rank = r * P_u + u."""
    assert [R.usp_rank(x, 8) for x in (0, 7, 8, 15)] == [(0, 0), (7, 0), (0, 1), (7, 1)]


# ---------------------------------------------------------------- padding
def test_padding_equals_single_pass():
    pins.pin_padding(R.ring_padded, R.padded_length, R.layout_index, R.ring_plan,
                     (R.CONTIGUOUS, R.ZIGZAG, R.STRIPED), R.ZIGZAG, A.attention,
                     (R.ring_contiguous, R.ring_zigzag, R.ring_striped))


def test_usp_bwd_equals_single_pass():
    pins.pin_usp_bwd(R.usp_bwd, A.attention, A.attention_bwd, (R.CONTIGUOUS, R.ZIGZAG, R.STRIPED))


def test_usp_padded_equals_single_pass():
    pins.pin_usp_padded(R.usp_padded, R.usp_attention, A.attention,
                        (R.CONTIGUOUS, R.ZIGZAG, R.STRIPED))
