"""Planted mistakes: every plausible slip in the oracle must fail a pin.

Each case rewrites one spot of the oracle's own source (a dropped term, a
wrong sign or index, a swapped operand, a shifted mask), loads the mutated
copy on the CPU and runs the pins against it.  The test passes when at
least one pin rejects the mutant; a mutant that every pin accepts would
mean the pins cannot tell that mistake from the real definition.
"""
import os
import sys
import types

import numpy as np
import pytest
import torch

import pins
from oracle import native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _load_mutant(relpath, old, new, modname):
    src = open(os.path.join(ROOT, relpath), encoding="utf-8").read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new, 1)
    pkg = types.ModuleType("oracle_mutant")
    pkg.__path__ = []
    sys.modules["oracle_mutant"] = pkg
    # the schedules module imports the attention module relatively
    att_src = open(os.path.join(ROOT, "oracle/attention.py"), encoding="utf-8").read()
    if relpath == "oracle/attention.py":
        att_src = src
    att = types.ModuleType("oracle_mutant.attention")
    exec(compile(att_src, "mutant_attention", "exec"), att.__dict__)
    sys.modules["oracle_mutant.attention"] = att
    if relpath == "oracle/attention.py":
        return att
    mod = types.ModuleType("oracle_mutant." + modname)
    mod.__package__ = "oracle_mutant"
    exec(compile(src, "mutant_" + modname, "exec"), mod.__dict__)
    return mod


def _attention_pins_fail(att):
    checks = [
        lambda: pins.pin_brute_force(att.attention),
        lambda: pins.pin_zero_query(att.attention),
        lambda: pins.pin_ones_value(att.attention),
        lambda: pins.pin_single_key(att.attention),
        lambda: pins.pin_sdpa(att.attention),
        lambda: pins.pin_merge_identity(att.attention, att.lse_merge),
        lambda: pins.pin_global_max_route(att.attention, att.attention_global_max),
    ]
    failed = 0
    for c in checks:
        try:
            c()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed += 1
    return failed


ATTENTION_MUTANTS = [
    ("diagonal masked", "kpos <= qpos", "kpos < qpos"),
    ("query offset dropped", "np.arange(Sq)[:, None] + q_offset", "np.arange(Sq)[:, None]"),
    ("key offset sign", "np.arange(Sk)[None, :] + k_offset", "np.arange(Sk)[None, :] - k_offset"),
    ("scale 1/D", "k[:, g, :].T) / np.sqrt(D)", "k[:, g, :].T) / D"),
    ("max term dropped from lse", "lse[h, i] = m + np.log", "lse[h, i] = np.log"),
    ("sum replaced by max", "np.exp(row - m).sum()", "np.exp(row - m).max()"),
    ("GQA head index", "        g = h // group\n        scores", "        g = h % Hkv\n        scores"),
    ("value operand swapped for key", "out[:, h, :] = w @ v[:, g, :]", "out[:, h, :] = w @ k[:, g, :]"),
    ("merge weight sign", "w1 = np.where(finite, np.exp(lse1 - safe)", "w1 = np.where(finite, np.exp(safe - lse1)"),
    ("merge uses one weight twice", "return o1 * w1 + o2 * w2", "return o1 * w1 + o2 * w1"),
    ("merge lse as max", "lse = np.logaddexp(lse1, lse2)", "lse = np.maximum(lse1, lse2)"),
]


def _bwd_pins_fail(att):
    checks = [
        lambda: pins.pin_bwd_finite_differences(att.attention, att.attention_bwd),
        lambda: pins.pin_bwd_autograd(att.attention, att.attention_bwd),
        lambda: pins.pin_bwd_closed_forms(att.attention, att.attention_bwd),
    ]
    failed = 0
    for c in checks:
        try:
            c()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed += 1
    return failed


BWD_MUTANTS = [
    ("softmax-gradient row term dropped", "ds = p * (dp - dvec[:, None])", "ds = p * dp"),
    ("row term sign", "ds = p * (dp - dvec[:, None])", "ds = p * (dp + dvec[:, None])"),
    ("row term from out only", "np.sum(dout[:, h, :] * out[:, h, :], axis=1)",
     "np.sum(out[:, h, :] * out[:, h, :], axis=1)"),
    ("dq scale missing", "dq[:, h, :] = ds @ k[:, g, :] * scale", "dq[:, h, :] = ds @ k[:, g, :]"),
    ("dk from dout", "dk[:, g, :] += ds.T @ q[:, h, :] * scale",
     "dk[:, g, :] += ds.T @ dout[:, h, :] * scale"),
    ("dv overwritten across the group", "dv[:, g, :] += p.T @ dout[:, h, :]",
     "dv[:, g, :] = p.T @ dout[:, h, :]"),
    ("P without the lse shift", "np.exp(s - np.where(finite, lse[h], 0.0)[:, None])",
     "np.exp(s)"),
    ("backward mask ignores offsets", "kpos = np.arange(Sk)[None, :] + k_offset\n    visible = (kpos <= qpos) if causal else np.ones((Sq, Sk), dtype=bool)\n    return _bwd_masked",
     "kpos = np.arange(Sk)[None, :]\n    visible = (kpos <= qpos) if causal else np.ones((Sq, Sk), dtype=bool)\n    return _bwd_masked"),
]


@pytest.mark.parametrize("name,old,new", BWD_MUTANTS, ids=[m[0] for m in BWD_MUTANTS])
def test_bwd_mutant_is_caught(name, old, new):
    att = _load_mutant("oracle/attention.py", old.replace("\\n", "\n"), new.replace("\\n", "\n"),
                       "attention")
    with np.errstate(all="ignore"):
        assert _bwd_pins_fail(att) >= 1, f"no pin catches: {name}"


def test_ring_bwd_mutants_are_caught():
    """Ring backward slips: block-local (out, lse) instead of the rows'
    final ones, and a KV block credited to the wrong rows."""
    for old, new in [
        ("dout[qo:qo + lq], out[qo:qo + lq], lse[:, qo:qo + lq],",
         "dout[qo:qo + lq], *attention(q[qo:qo + lq], k[ko:ko + lk], v[ko:ko + lk], causal=(kind == DIAG), q_offset=qo, k_offset=ko),"),
        ("dk[ko:ko + lk] += gk", "dk[qo:qo + lq] += gk"),
    ]:
        sch = _load_mutant("oracle/schedules.py", old, new, "schedules")
        with pytest.raises(AssertionError):
            pins.pin_bwd_ring(sch.ring_bwd, sch.attention, sch.attention_bwd, sch.CONTIGUOUS,
                              sch.ZIGZAG)


@pytest.mark.parametrize("name,old,new", ATTENTION_MUTANTS, ids=[m[0] for m in ATTENTION_MUTANTS])
def test_attention_mutant_is_caught(name, old, new):
    att = _load_mutant("oracle/attention.py", old, new, "attention")
    with np.errstate(all="ignore"):
        assert _attention_pins_fail(att) >= 1, f"no pin catches: {name}"


def _schedule_pins_fail(sch, att):
    import oracle.schedules as real
    failed = 0
    checks = []
    checks.append(lambda: pins.pin_work(sch.rank_chunks, sch.causal_units, sch.CONTIGUOUS,
                                        sch.ZIGZAG))

    def ring_checks():
        from oracle.attention import attention
        q, k, v = pins.make_qkv_page()
        ref, _ = attention(q, k, v)
        outs, _, computed = sch.ring_contiguous(q, k, v, P=4)
        assert computed == pins.load_golden("ring_counts_p4.txt")["counts"]
        for r in range(4):
            np.testing.assert_allclose(outs[r], ref[r * 8:(r + 1) * 8], atol=1e-12)
        outs, _, units = sch.ring_zigzag(q, k, v, P=4)
        for r in range(4):
            np.testing.assert_allclose(outs[r], ref[sch.layout_index(sch.ZIGZAG, 32, 4, r)],
                                       atol=1e-12)
            assert units[r] == [2.0] * 4
    checks.append(ring_checks)

    def plan_checks():
        for P in (4, 8):
            S = 16 * P
            mine = sch.ring_plan(S, P, sch.ZIGZAG, -1)
            ref = real.ring_plan(S, P, real.ZIGZAG, -1)
            # counts and coverage facts (not the reference plan itself)
            for r in range(P):
                comp = sorted((p[2], p[3]) for p in mine if p[0] == r and p[8] != sch.SKIP)
                want = sorted((qc, kc) for qc in pins_split_zigzag(P)[r] for kc in range(qc + 1))
                assert comp == want
            assert len(mine) == len(ref)
    checks.append(plan_checks)

    def ulysses_checks():
        S, H, D, P = 24, 8, 3, 4
        x = np.arange(S * H * D, dtype=np.float64).reshape(S, H, D)
        heads = sch.seq_to_head([x[r * 6:(r + 1) * 6] for r in range(P)], P)
        for p in range(P):
            assert np.array_equal(heads[p], x[:, 2 * p:2 * p + 2, :])
        assert np.array_equal(np.concatenate(sch.head_to_seq(heads, P)), x)
        g = pins.load_golden("ulysses_shapes_p4.txt")
        q, k, v = pins.make_qkv_page()
        outs, shapes = sch.ulysses_attention(q, k, v, P=4)
        assert all(list(s) == g["attention"] for s in shapes)
    checks.append(ulysses_checks)

    for c in checks:
        try:
            c()
        except (AssertionError, ValueError, IndexError, KeyError, TypeError):
            failed += 1
    return failed


def pins_split_zigzag(P):
    """The zigzag split as the page's prose states it: rank r takes the r-th
    chunk and the (r+1)-th chunk from the end (counting from the front, chunk
    2P - r - 1)."""
    out = {}
    for r in range(P):
        nth_from_end = r + 1
        out[r] = [r, 2 * P - nth_from_end]
    return out


SCHEDULE_MUTANTS = [
    ("zigzag mirror owner", "owner = [min(c, n - 1 - c) for c in range(n)]",
     "owner = [min(c, n - 2 - c) % P for c in range(n)]"),
    ("contiguous owner", "owner = [c // 2 for c in range(n)]", "owner = [c % P for c in range(n)]"),
    ("work counts diagonal fully", "+ 0.5 * np.eye(n_chunks)", "+ 1.0 * np.eye(n_chunks)"),
    ("work grid upper triangle", "np.tril(np.ones((n_chunks, n_chunks)), k=-1)",
     "np.triu(np.ones((n_chunks, n_chunks)), k=1)"),
    ("ring skip rule", "if not causal or s <= r]", "if not causal or s < r]"),
    ("ring key offset", "q_offset=r * C, k_offset=s * C)", "q_offset=r * C, k_offset=r * C)"),
    ("ring one step short", "held = np.array([[(r - t) % P for t in range(P)]",
     "held = np.array([[(r - t) % P for t in range(P - 1)]"),
    ("zigzag skip rule", "if causal and kc > qc:", "if causal and kc >= qc:"),
    ("plan classification", "elif kc == qc:\n                        kind = DIAG",
     "elif kc == qc + 1:\n                        kind = DIAG"),
    ("seq_to_head transpose dropped", "x.reshape(Sl, P, H // P, D).transpose(1, 0, 2, 3)",
     "x.reshape(P, Sl, H // P, D)"),
    ("all_to_all block index", "np.stack([sendbufs[r][p] for r in range(P)])",
     "np.stack([sendbufs[p][r] for r in range(P)])"),
]


@pytest.mark.parametrize("name,old,new", SCHEDULE_MUTANTS, ids=[m[0] for m in SCHEDULE_MUTANTS])
def test_schedule_mutant_is_caught(name, old, new):
    sch = _load_mutant("oracle/schedules.py", old, new, "schedules")
    assert _schedule_pins_fail(sch, None) >= 1, f"no pin catches: {name}"


C_MUTANTS = [
    ("diagonal masked", "k_offset + j > pos_q", "k_offset + j >= pos_q"),
    ("scale 1/D", "1.0 / sqrt((double)D)", "1.0 / (double)D"),
    ("max term dropped", "const double l = m + log(sum);", "const double l = log(sum);"),
    ("GQA head index", "const int g = h / group;", "const int g = h % Hkv;"),
    ("weights not normalised", "const double w = exp(s[j] - l);", "const double w = exp(s[j] - m);"),
    ("bf16 widening shift", "<< 16;", "<< 15;"),
]


@pytest.mark.parametrize("name,old,new", C_MUTANTS, ids=[m[0] for m in C_MUTANTS])
def test_c_oracle_mutant_is_caught(name, old, new, tmp_path):
    src = open(os.path.join(ROOT, "oracle/cp_oracle.c"), encoding="utf-8").read()
    assert old in src
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new, 1))
    lib = native.bind(native.build(src=str(mpath), out=str(tmp_path / "libmutant.so")))

    def attn(q, k, v, causal=True, q_offset=0, k_offset=0):
        t = [torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32) for x in (q, k, v)]
        return native.attention_rows(*t, causal=causal, q_offset=q_offset,
                                     k_offset=k_offset, n_threads=1, lib=lib)

    def bf16_check():
        from oracle.attention import attention
        from seeded_inputs import make_qkv
        q, k, v = make_qkv(S=9, H=2, D=4, dtype=torch.bfloat16)
        o, l = native.attention_rows(q, k, v, n_threads=1, lib=lib)
        ro, rl = attention(q, k, v)
        np.testing.assert_allclose(o, ro, atol=1e-12)

    pins.ROUND_INPUTS = np.float32
    failed = 0
    try:
        for c in (lambda: pins.pin_brute_force(attn), lambda: pins.pin_zero_query(attn),
                  lambda: pins.pin_single_key(attn), lambda: pins.pin_sdpa(attn), bf16_check):
            try:
                with np.errstate(all="ignore"):
                    c()
            except (AssertionError, ValueError):
                failed += 1
    finally:
        pins.ROUND_INPUTS = None
    assert failed >= 1, f"no pin catches: {name}"


C_BWD_MUTANTS = [
    ("row term dropped", "const double ds = p * (dp - dvi);", "const double ds = p * dp;"),
    ("dk row term dropped", "const double ds = p * (dp - dvec[(int64_t)h * n_stat + i]);",
     "const double ds = p * dp;"),
    ("dv without P", "ov[d] += p * di;", "ov[d] += di;"),
    ("dk scale missing", "ok[d] += ds * widen(q, dtype, (i * Hq + h) * (int64_t)D + d) * inv_sqrt_d;",
     "ok[d] += ds * widen(q, dtype, (i * Hq + h) * (int64_t)D + d);"),
]


@pytest.mark.parametrize("name,old,new", C_BWD_MUTANTS, ids=[m[0] for m in C_BWD_MUTANTS])
def test_c_oracle_bwd_mutant_is_caught(name, old, new, tmp_path):
    src = open(os.path.join(ROOT, "oracle/cp_oracle.c"), encoding="utf-8").read()
    assert old in src
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new, 1))
    lib = native.bind(native.build(src=str(mpath), out=str(tmp_path / "libmutant.so")))
    from oracle.attention import attention, attention_bwd
    g = torch.Generator().manual_seed(3)
    Sq, Sk, Hq, Hkv, D, qo, ko = 7, 9, 4, 2, 8, 4, 2
    q, k, v, do = (torch.randn(s, generator=g) for s in ((Sq, Hq, D), (Sk, Hkv, D),
                                                        (Sk, Hkv, D), (Sq, Hq, D)))
    out, lse = attention(q, k, v, q_offset=qo, k_offset=ko)
    want = attention_bwd(q, k, v, do, out, lse, q_offset=qo, k_offset=ko)
    rows = list(range(Sq)), list(range(Sk))
    dq, dk, dv = native.attention_bwd_rows(q, k, v, do, *rows, q_offset=qo, k_offset=ko,
                                           n_threads=1, lib=lib)
    with pytest.raises(AssertionError):
        for got, w in zip((dq, dk, dv), want):
            np.testing.assert_allclose(got, w, atol=1e-10)


def _schedules_over(att):
    """The real schedules module bound to a (possibly mutated) attention module."""
    sys.modules["oracle_mutant.attention"] = att
    src = open(os.path.join(ROOT, "oracle/schedules.py"), encoding="utf-8").read()
    mod = types.ModuleType("oracle_mutant.schedules")
    mod.__package__ = "oracle_mutant"
    exec(compile(src, "schedules_over_mutant", "exec"), mod.__dict__)
    return mod


def _striped_pins_fail(att, sch):
    checks = [
        lambda: pins.pin_attention_at(att.attention_at, att.attention),
        lambda: pins.pin_bwd_at_finite_differences(att.attention_at, att.attention_bwd_at),
        lambda: pins.pin_striped(sch.ring_striped, sch.layout_index, sch.STRIPED, att.attention),
        lambda: pins.pin_bwd_ring(sch.ring_bwd, att.attention, att.attention_bwd, sch.CONTIGUOUS,
                                  sch.ZIGZAG, sch.STRIPED),
        lambda: pins.pin_striped_plan(sch.ring_plan, sch.layout_index, sch.STRIPED, sch.DIAG,
                                      sch.FULL, att.attention, att.attention_at),
    ]
    failed = 0
    for c in checks:
        try:
            c()
        except (AssertionError, ValueError, IndexError):
            failed += 1
    return failed


STRIPED_MUTANTS = [
    ("explicit-position mask strict", "oracle/attention.py",
     "visible = (kp <= qp) if causal else np.ones((Sq, Sk), dtype=bool)",
     "visible = (kp < qp) if causal else np.ones((Sq, Sk), dtype=bool)"),
    ("explicit-position mask reversed", "oracle/attention.py",
     "visible = (kp <= qp) if causal else np.ones((Sq, Sk), dtype=bool)",
     "visible = (qp <= kp) if causal else np.ones((Sq, Sk), dtype=bool)"),
    ("explicit-position backward mask strict", "oracle/attention.py",
     "visible = (kp <= qp) if causal else np.ones((qp.shape[0]",
     "visible = (kp < qp) if causal else np.ones((qp.shape[0]"),
    ("striped split is contiguous", "oracle/schedules.py",
     "return np.arange(rank, S, P, dtype=np.int64)",
     "return np.arange(rank * (S // P), (rank + 1) * (S // P), dtype=np.int64)"),
    ("striped ring masks keys with the query positions", "oracle/schedules.py",
     "attention_at(q[qpos], k[kpos], v[kpos], qpos, kpos,",
     "attention_at(q[qpos], k[kpos], v[kpos], qpos, qpos,"),
    ("striped ring keys never leave their rank", "oracle/schedules.py",
     "kpos = layout_index(STRIPED, S, P, src)",
     "kpos = layout_index(STRIPED, S, P, rank)"),
    ("striped work counts the diagonal out", "oracle/schedules.py",
     "n += int(np.sum(kpos[None, :] <= qpos[:, None]))",
     "n += int(np.sum(kpos[None, :] < qpos[:, None]))"),
    ("striped ring backward dq to key rows", "oracle/schedules.py",
     "dq[qi] += gq\n            dk[ki]", "dq[ki] += gq\n            dk[ki]"),
    ("striped plan key offset dropped", "oracle/schedules.py",
     "pairs.append((r, t, r, src, 0, int(src > r), C, C,",
     "pairs.append((r, t, r, src, 0, 0, C, C,"),
    ("striped plan key offset reversed", "oracle/schedules.py",
     "pairs.append((r, t, r, src, 0, int(src > r), C, C,",
     "pairs.append((r, t, r, src, 0, int(src < r), C, C,"),
    ("striped ring backward dk to query rows", "oracle/schedules.py",
     "dk[ki] += gk", "dk[qi] += gk"),
]


@pytest.mark.parametrize("name,relpath,old,new", STRIPED_MUTANTS, ids=[m[0] for m in STRIPED_MUTANTS])
def test_striped_mutant_is_caught(name, relpath, old, new):
    if relpath == "oracle/attention.py":
        att = _load_mutant(relpath, old, new, "attention")
        sch = _schedules_over(att)
    else:
        sch = _load_mutant(relpath, old, new, "schedules")
        att = sys.modules["oracle_mutant.attention"]
    with np.errstate(all="ignore"):
        assert _striped_pins_fail(att, sch) >= 1, f"no pin catches: {name}"


USP_MUTANTS = [
    ("USP shard of the wrong Ulysses rank", "shards = [x[group_rows[r][u * Sl:(u + 1) * Sl]] for u in range(P_u)]",
     "shards = [x[group_rows[r][(P_u - 1 - u) * Sl:(P_u - u) * Sl]] for u in range(P_u)]"),
    ("USP head shares scattered to natural rows", "full[u][group_rows[r]] = y",
     "full[u][r * Sg:(r + 1) * Sg] = y"),
    ("USP positions of the wrong shard", "positions[r * P_u + u] = group_rows[r][u * Sl:(u + 1) * Sl]",
     "positions[r * P_u + u] = group_rows[r][:Sl]"),
    ("USP lse not transposed back", "lses[r * P_u + u] = l[u][:, :, 0].T",
     "lses[r * P_u + u] = l[u][:, :, 0].T[::-1]"),
    ("USP rank numbering ring-major", "return rank % P_u, rank // P_u", "return rank // P_u, rank % P_u"),
]


@pytest.mark.parametrize("name,old,new", USP_MUTANTS, ids=[m[0] for m in USP_MUTANTS])
def test_usp_mutant_is_caught(name, old, new):
    sch = _load_mutant("oracle/schedules.py", old, new, "schedules")
    failed = 0
    for check in (
        lambda: pins.pin_usp(sch.usp_attention, (sch.ring_contiguous, sch.ring_zigzag,
                                                 sch.ring_striped),
                             sch.ulysses_attention, (sch.CONTIGUOUS, sch.ZIGZAG, sch.STRIPED),
                             sch.attention),
        lambda: [sch.usp_rank(x, 8) for x in (0, 7, 8, 15)] == [(0, 0), (7, 0), (0, 1), (7, 1)]
        or (_ for _ in ()).throw(AssertionError("rank numbering")),
    ):
        try:
            with np.errstate(all="ignore"):
                check()
        except (AssertionError, ValueError, IndexError, ZeroDivisionError):
            failed += 1
    assert failed >= 1, f"no pin catches: {name}"


PAD_MUTANTS = [
    ("padding keys visible", "oracle/attention.py",
     "visible = visible & np.asarray(kvalid, dtype=bool)[None, :]", "visible = visible"),
    ("zigzag padded to a multiple of P", "oracle/schedules.py",
     "m = 2 * P if layout == ZIGZAG else P", "m = P"),
    ("padded rows kept", "oracle/schedules.py", "real = qpos < S", "real = qpos <= S"),
    ("plan clips one row short", "oracle/schedules.py",
     "lq, lk = min(max(S_real - qo, 0), lq), min(max(S_real - ko, 0), lk)",
     "lq, lk = min(max(S_real - qo - 1, 0), lq), min(max(S_real - ko - 1, 0), lk)"),
    ("striped real rows off by one", "oracle/schedules.py",
     "return int(np.sum(rank + P * np.arange(C) < S))",
     "return int(np.sum(rank + P * np.arange(C) <= S))"),
    ("striped backward keeps padded rows", "oracle/schedules.py",
     "qi, ki = qi[qi < S], ki[ki < S]", "qi, ki = qi[qi < S], ki"),
]


@pytest.mark.parametrize("name,relpath,old,new", PAD_MUTANTS, ids=[m[0] for m in PAD_MUTANTS])
def test_padding_mutant_is_caught(name, relpath, old, new):
    if relpath == "oracle/attention.py":
        att = _load_mutant(relpath, old, new, "attention")
        sch = _schedules_over(att)
    else:
        sch = _load_mutant(relpath, old, new, "schedules")
        att = sys.modules["oracle_mutant.attention"]
    failed = 0
    for check in (
        lambda: pins.pin_padding(sch.ring_padded, sch.padded_length, sch.layout_index,
                                 sch.ring_plan, (sch.CONTIGUOUS, sch.ZIGZAG, sch.STRIPED),
                                 sch.ZIGZAG, att.attention,
                                 (sch.ring_contiguous, sch.ring_zigzag, sch.ring_striped)),
        lambda: pins.pin_bwd_ring(sch.ring_bwd, att.attention, att.attention_bwd,
                                  sch.CONTIGUOUS, sch.ZIGZAG, sch.STRIPED),
        lambda: pins.pin_attention_at(att.attention_at, att.attention),
    ):
        try:
            with np.errstate(all="ignore"):
                check()
        except (AssertionError, ValueError, IndexError):
            failed += 1
    assert failed >= 1, f"no pin catches: {name}"


@pytest.mark.parametrize("old,new", [
    ("dq[:, hs], dk[:, ks], dv[:, ks] = gq, gk, gv", "dq[:, hs], dk[:, ks], dv[:, ks] = gq, gv, gk"),
    ("hs, ks = slice(u * Hp, (u + 1) * Hp), slice(u * Hkp, (u + 1) * Hkp)",
     "hs, ks = slice(u * Hp, (u + 1) * Hp), slice(0, Hkp)"),
])
def test_usp_bwd_mutant_is_caught(old, new):
    sch = _load_mutant("oracle/schedules.py", old, new, "schedules")
    with pytest.raises(AssertionError):
        pins.pin_usp_bwd(sch.usp_bwd, sch.attention, sch.attention_bwd,
                         (sch.CONTIGUOUS, sch.ZIGZAG, sch.STRIPED))


@pytest.mark.parametrize("old,new", [
    ("return np.repeat(x, P // H, axis=1)", "return np.tile(x, (1, P // H, 1))"),
    ("k, v = replicate_kv(k, P), replicate_kv(v, P)", "k, v = replicate_kv(k, P), replicate_kv(k, P)"),
])
def test_kv_replication_mutant_is_caught(old, new):
    import test_oracle_pins as T
    sch = _load_mutant("oracle/schedules.py", old, new, "schedules")
    real = T.R
    T.R = sch
    try:
        with pytest.raises(AssertionError):
            T.test_ulysses_kv_replication_exercise()
    finally:
        T.R = real


@pytest.mark.parametrize("old,new", [
    ("outs = [np.concatenate([shares[u][0][r] for u in range(P_u)], axis=1) for r in range(P_r)]",
     "outs = [np.concatenate([shares[u][0][r] for u in range(P_u)][::-1], axis=1) for r in range(P_r)]"),
    ("v[:, u * Hkp:(u + 1) * Hkp], P_r, layout, causal) for u in range(P_u)]",
     "v[:, 0:Hkp], P_r, layout, causal) for u in range(P_u)]"),
])
def test_usp_padded_mutant_is_caught(old, new):
    sch = _load_mutant("oracle/schedules.py", old, new, "schedules")
    with pytest.raises(AssertionError):
        pins.pin_usp_padded(sch.usp_padded, sch.usp_attention, sch.attention,
                            (sch.CONTIGUOUS, sch.ZIGZAG, sch.STRIPED))
