"""Sequence splits, the causal work model, the ring loops and the Ulysses
all-to-all, restated on P virtual ranks in one process (numpy, float64).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources, all on the handbook page "上下文并行：Ring Attention 与 Ulysses"
(Context parallelism: Ring Attention and Ulysses):

* section "Ring Attention：KV 沿环传一圈": rank r owns rows
  [r*C, (r+1)*C) with C = S/P; at step t it holds the KV block of rank
  src = (r - t) mod P, computes only when src <= r, merges with the
  log-sum-exp rule and passes the block to rank r+1;
* section "之字形切分" (zigzag split): the sequence is cut into 2P chunks;
  the zigzag split gives each rank one chunk from the front and its mirror
  from the back, the contiguous split gives consecutive chunks; causal work
  counts the key chunks a query chunk sees, the diagonal one as half;
* section "Ulysses：在序列和头之间转置": seq_to_head and head_to_seq are
  a reshape/transpose followed by ``all_to_all_single``.

Readings where the page is silent (the page has no zigzag ring code):

* zigzag ring -- rank r's local rows are [chunk r, chunk 2P-1-r] in that
  order, its KV block is the same two chunks, src = (r - t) mod P as in
  the contiguous ring, and every (query chunk, key chunk) pair is
  skipped when the key chunk comes after the query chunk, computed with
  the causal mask when they are the same chunk, and computed in full
  when the key chunk comes first.
* plan order -- for each rank, each step, each query chunk in local
  order, each key chunk in local order.
* striped split (from the "Sequence Parallel vs Context Parallel" blog,
  section 3.3, prose only) -- stripes of one token dealt round-robin:
  position t lives on rank t mod P.  Every (rank, source) pair of the ring
  is computed (the positions interleave, so no block is wholly masked),
  under the causal mask taken on the true positions.
"""
from __future__ import annotations

import functools

import numpy as np

from .attention import attention, attention_at, attention_bwd, attention_bwd_at, lse_merge

CONTIGUOUS, ZIGZAG, STRIPED = 0, 1, 2
SKIP, FULL, DIAG = 0, 1, 2


# ----------------------------------------------------------------- splits
def rank_chunks(layout: int, P: int, rank: int) -> list[int]:
    """The chunks of the 2P-way split that ``rank`` holds, in its local
    order (the zigzag section's two splits, stated as ownership rules):

    * contiguous: chunks are handed out two at a time in sequence order, so
      chunk c belongs to rank c // 2;
    * zigzag: chunk c and its mirror chunk 2P-1-c belong to one rank, the
      one numbered by the nearer end, min(c, 2P-1-c).
    """
    n = 2 * P
    if layout == CONTIGUOUS:
        owner = [c // 2 for c in range(n)]
    elif layout == ZIGZAG:
        owner = [min(c, n - 1 - c) for c in range(n)]
    else:
        raise ValueError("rank_chunks covers the contiguous and zigzag splits")
    return [c for c in range(n) if owner[c] == rank]


def causal_units(query_chunks, n_chunks: int) -> float:
    """Causal work of the given query chunks, in units of one full
    chunk-by-chunk block (the zigzag section's work model): in the
    n_chunks x n_chunks grid of blocks, query chunk i needs the blocks of
    key chunks before it in full and the one on the diagonal, whose visible
    pairs are half of it."""
    grid = np.tril(np.ones((n_chunks, n_chunks)), k=-1) + 0.5 * np.eye(n_chunks)
    return float(grid[list(query_chunks)].sum())


def padded_length(S: int, P: int, layout: int) -> int:
    """The practitioner blog's padding (section 7.1): when the split does
    not divide S, the sequence is padded up to the next multiple of P (2P
    for zigzag, whose chunks are 2P)."""
    m = 2 * P if layout == ZIGZAG else P
    return -(-S // m) * m


def layout_index(layout: int, S: int, P: int, rank: int) -> np.ndarray:
    """Natural sequence position of each local row of ``rank``.

    Contiguous: the ring section's ``slice(rank*C, (rank+1)*C)``.
    Zigzag: the 2P-chunk split, chunks concatenated in the order listed.
    Striped: positions rank, rank + P, rank + 2P, ... (stripes of one token
    dealt round-robin, the reading stated in ``ring_striped``).
    When the split does not divide S the layout is that of the padded
    length (``padded_length``): positions >= S are padding rows.
    """
    S = padded_length(S, P, layout)
    if layout == CONTIGUOUS:
        C = S // P
        return np.arange(rank * C, (rank + 1) * C, dtype=np.int64)
    if layout == STRIPED:
        return np.arange(rank, S, P, dtype=np.int64)
    C = S // (2 * P)
    return np.concatenate([np.arange(c * C, (c + 1) * C, dtype=np.int64)
                           for c in rank_chunks(ZIGZAG, P, rank)])


def _chunks(layout: int, S: int, P: int, rank: int):
    """(chunk ids, chunk length) of ``rank`` for the ring schedule."""
    if layout == CONTIGUOUS:
        return [rank], S // P
    return rank_chunks(ZIGZAG, P, rank), S // (2 * P)


def ring_plan(S: int, P: int, layout: int, rank: int, causal: bool = True):
    """Every (rank, step, q_chunk, k_chunk) pair of the ring, classified.

    Returns a list of tuples (rank, step, q_chunk, k_chunk, q_offset,
    k_offset, len_q, len_k, kind) with kind SKIP / FULL / DIAG.  rank=-1
    lists all ranks.
    """
    ranks = range(P) if rank < 0 else [rank]
    pairs = []
    S_real, S = S, padded_length(S, P, layout)
    if S != S_real:
        # padded sequence: each chunk keeps its real rows only; a pair with
        # no real query or key row is skipped
        out = []
        for p in ring_plan(S, P, layout, rank, causal):
            (r, t, qc, kc, qo, ko, lq, lk, kind) = p
            if layout == STRIPED:
                lq, lk = _real_rows(S_real, P, qc, lq), _real_rows(S_real, P, kc, lk)
            else:
                lq, lk = min(max(S_real - qo, 0), lq), min(max(S_real - ko, 0), lk)
            out.append((r, t, qc, kc, qo, ko, lq, lk, SKIP if lq == 0 or lk == 0 else kind))
        return out
    if layout == STRIPED:
        # every rank's positions interleave with every other's: each pair is
        # computed, under the causal mask when causal; chunk id = rank id.
        # Local row i of rank r is position r + i*P and local key j of rank
        # src is src + j*P, so j is visible to i iff j <= i - (src > r): the
        # offsets given are these local ones, q 0 and k (src > r).
        C = S // P
        for r in ranks:
            for t in range(P):
                src = (r - t) % P
                pairs.append((r, t, r, src, 0, int(src > r), C, C, DIAG if causal else FULL))
        return pairs
    for r in ranks:
        q_chunks, C = _chunks(layout, S, P, r)
        for t in range(P):
            src = (r - t) % P
            k_chunks, _ = _chunks(layout, S, P, src)
            for qc in q_chunks:
                for kc in k_chunks:
                    if not causal or kc < qc:
                        kind = FULL
                    elif kc == qc:
                        kind = DIAG
                    else:
                        kind = SKIP
                    pairs.append((r, t, qc, kc, qc * C, kc * C, C, C, kind))
    return pairs


def _real_rows(S: int, P: int, rank: int, C: int) -> int:
    """Striped: how many of rank's C rows (positions rank + jP) lie below S."""
    return int(np.sum(rank + P * np.arange(C) < S))


# ---------------------------------------------------------------- the ring
def ring_contiguous(q, k, v, P: int, causal: bool = True):
    """The ring section's schedule on P virtual ranks: rank r owns rows
    [r*C, (r+1)*C); at step t it holds the KV block of rank (r - t) mod P
    (blocks move one rank to the right per step).  Under the causal mask a
    block of a later rank lies wholly after the rank's queries and is not
    computed; the blocks computed are folded into one result with the
    log-sum-exp merge, in the order the steps bring them.

    Returns (outs, lses, computed): per rank its local out [C, Hq, D],
    lse [Hq, C] and the number of KV blocks it computed.
    """
    S = q.shape[0]
    C = S // P
    owned = [slice(r * C, (r + 1) * C) for r in range(P)]
    # source rank of the block each rank holds at each step
    held = np.array([[(r - t) % P for t in range(P)] for r in range(P)])
    outs, lses, computed = [], [], []
    for r in range(P):
        sources = [int(s) for s in held[r] if not causal or s <= r]
        parts = [attention(q[owned[r]], k[owned[s]], v[owned[s]], causal=causal,
                           q_offset=r * C, k_offset=s * C) for s in sources]
        o, l = functools.reduce(lambda acc, part: lse_merge(*acc, *part), parts)
        outs.append(o)
        lses.append(l)
        computed.append(len(parts))
    return outs, lses, computed


def ring_zigzag(q, k, v, P: int, causal: bool = True):
    """Zigzag ring (reading stated in the module docstring).

    Returns (outs, lses, units): per rank its local out [2C, Hq, D] in the
    order [chunk r, chunk 2P-1-r], lse [Hq, 2C], and the work units it
    computed at each step (full pair = 1, diagonal pair = 1/2).
    """
    S, Hq, D = q.shape
    C = S // (2 * P)
    split = [rank_chunks(ZIGZAG, P, r) for r in range(P)]
    outs, lses, units = [], [], []
    for rank in range(P):
        state = {}
        per_step = []
        for step in range(P):
            src = (rank - step) % P
            u = 0.0
            for qc in split[rank]:
                for kc in split[src]:
                    if causal and kc > qc:
                        continue
                    o, l = attention(q[qc * C:(qc + 1) * C], k[kc * C:(kc + 1) * C],
                                     v[kc * C:(kc + 1) * C], causal=causal,
                                     q_offset=qc * C, k_offset=kc * C)
                    state[qc] = (o, l) if qc not in state else lse_merge(*state[qc], o, l)
                    u += 0.5 if (causal and kc == qc) else 1.0
            per_step.append(u)
        outs.append(np.concatenate([state[c][0] for c in split[rank]], axis=0))
        lses.append(np.concatenate([state[c][1] for c in split[rank]], axis=1))
        units.append(per_step)
    return outs, lses, units


def ring_striped(q, k, v, P: int, causal: bool = True):
    """Striped ring.  The "Sequence Parallel vs Context Parallel" blog,
    section 3.3, gives Striped Attention in prose only: KV is dealt to the
    devices in interleaved stripes so that each holds early and late
    positions and every ring step carries about the same causal work (the
    handbook's zigzag section mentions a similar striped split).

    Reading: stripes of one token, position t on rank t mod P, so rank r's
    local row j is position r + j*P; the ring is the handbook's loop
    (src = (r - t) mod P, merge every block with the log-sum-exp rule), each
    block attended with the true positions of its rows.

    Returns (outs, lses, pairs): per rank its local out [S/P, Hq, D], lse
    [Hq, S/P], and the number of visible (query, key) pairs it computed per
    head.
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    S = q.shape[0]
    outs, lses, work_pairs = [], [], []
    for rank in range(P):
        qpos = layout_index(STRIPED, S, P, rank)
        state = None
        n = 0
        for step in range(P):
            src = (rank - step) % P
            kpos = layout_index(STRIPED, S, P, src)
            o, l = attention_at(q[qpos], k[kpos], v[kpos], qpos, kpos, causal=causal)
            state = (o, l) if state is None else lse_merge(*state, o, l)
            n += int(np.sum(kpos[None, :] <= qpos[:, None])) if causal else qpos.size * kpos.size
        outs.append(state[0])
        lses.append(state[1])
        work_pairs.append(n)
    return outs, lses, work_pairs


def ring_padded(q, k, v, P: int, layout: int, causal: bool = True):
    """Ring attention when the split does not divide S (the practitioner
    blog, section 7.1: pad up to a multiple of the CP degree, compute,
    discard what the padding produced).

    Reading: zero rows are appended at positions S .. S_pad-1
    (``padded_length``); the padded sequence is split with ``layout``;
    every rank runs the handbook's ring loop over all P steps (a block with
    no visible key contributes (0, -inf), the merge's identity), attending
    with true positions and with the padding keys removed from every row's
    visible set; the rows at positions >= S are then discarded.

    Returns (outs, lses, positions): per rank the out [n_r, Hq, D] and lse
    [Hq, n_r] of its real rows, in local order, and their positions.
    """
    q, k, v = (np.asarray(x, dtype=np.float64) if not hasattr(x, "detach")
               else x.detach().double().numpy() for x in (q, k, v))
    S = q.shape[0]
    S_pad = padded_length(S, P, layout)

    def pad(x):
        return np.concatenate([x, np.zeros((S_pad - S,) + x.shape[1:])])

    qp, kp, vp = pad(q), pad(k), pad(v)
    outs, lses, positions = [], [], []
    for rank in range(P):
        qpos = layout_index(layout, S_pad, P, rank)
        state = None
        for step in range(P):
            src = (rank - step) % P
            kpos = layout_index(layout, S_pad, P, src)
            o, l = attention_at(qp[qpos], kp[kpos], vp[kpos], qpos, kpos, causal=causal,
                                kvalid=kpos < S)
            state = (o, l) if state is None else lse_merge(*state, o, l)
        real = qpos < S
        outs.append(state[0][real])
        lses.append(state[1][:, real])
        positions.append(qpos[real])
    return outs, lses, positions


def ring_bwd(q, k, v, dout, P: int, layout: int, causal: bool = True):
    """Backward pass through the ring (no algorithm on the pages; the
    plainest reading of running the forward ring backwards).

    Every pair that the forward plan computes (``ring_plan``, all ranks)
    contributes ``attention_bwd`` of its query chunk against its key chunk,
    taken with the query rows' final (out, lse) -- the forward result of
    the whole ring, which equals the single-pass result.  dq accumulates on
    the query rows' rank; dk and dv accumulate on the KV block's rows (on a
    real ring these accumulators travel with the block and return to its
    owner after P steps).  Returns dq, dk, dv in natural order, float64.
    """
    q, k, v, dout = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    S = q.shape[0]
    out, lse = attention(q, k, v, causal=causal)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for (r, _t, _qc, src, qo, ko, lq, lk, kind) in ring_plan(S, P, layout, -1, causal):
        if kind == SKIP:
            continue
        if layout == STRIPED:
            qi, ki = layout_index(STRIPED, S, P, r), layout_index(STRIPED, S, P, src)
            qi, ki = qi[qi < S], ki[ki < S]
            gq, gk, gv = attention_bwd_at(q[qi], k[ki], v[ki], dout[qi], out[qi], lse[:, qi],
                                          qi, ki, causal=causal)
            dq[qi] += gq
            dk[ki] += gk
            dv[ki] += gv
            continue
        gq, gk, gv = attention_bwd(q[qo:qo + lq], k[ko:ko + lk], v[ko:ko + lk],
                                   dout[qo:qo + lq], out[qo:qo + lq], lse[:, qo:qo + lq],
                                   causal=(kind == DIAG), q_offset=qo, k_offset=ko)
        dq[qo:qo + lq] += gq
        dk[ko:ko + lk] += gk
        dv[ko:ko + lk] += gv
    return dq, dk, dv


# ---------------------------------------------------------------- Ulysses
def all_to_all(sendbufs):
    """``all_to_all_single`` over P virtual ranks: block p of rank r's send
    buffer becomes block r of rank p's receive buffer."""
    P = len(sendbufs)
    return [np.stack([sendbufs[r][p] for r in range(P)]) for p in range(P)]


def seq_to_head(local_x, P: int):
    """Ulysses section: every rank's [S/P, H, D] -> every rank's [S, H/P, D]."""
    Sl, H, D = local_x[0].shape
    sends = [x.reshape(Sl, P, H // P, D).transpose(1, 0, 2, 3) for x in local_x]
    return [r.reshape(P * Sl, H // P, D) for r in all_to_all(sends)]


def head_to_seq(head_x, P: int):
    """Ulysses section: every rank's [S, H/P, D] -> every rank's [S/P, H, D]."""
    S, Hp, D = head_x[0].shape
    sends = [y.reshape(P, S // P, Hp, D) for y in head_x]
    return [r.transpose(1, 0, 2, 3).reshape(S // P, P * Hp, D) for r in all_to_all(sends)]


def replicate_kv(x, P: int):
    """The exercise's way past the KV-head limit: when P exceeds the KV head
    count, every KV head is copied P/Hkv times (consecutive copies) before
    the all-to-all, so rank p receives KV head p // (P/Hkv)."""
    H = x.shape[1]
    if H >= P:
        return x
    if P % H:
        raise ValueError("KV replication needs Hkv | P")
    return np.repeat(x, P // H, axis=1)


def ulysses_attention(q, k, v, P: int, causal: bool = True):
    """Ulysses on P virtual ranks: split rows, seq_to_head q, k, v, local
    full-sequence attention on each rank's head share, head_to_seq.  With
    fewer KV heads than ranks the KV heads are replicated first
    (``replicate_kv``).
    Returns (per-rank local outputs, per-rank attention-time q shapes)."""
    q, k, v = (np.asarray(x, dtype=np.float64) if not hasattr(x, "detach")
               else x.detach().double().numpy() for x in (q, k, v))
    k, v = replicate_kv(k, P), replicate_kv(v, P)
    S = q.shape[0]
    C = S // P
    rows = [slice(r * C, (r + 1) * C) for r in range(P)]
    ql = seq_to_head([q[s] for s in rows], P)
    kl = seq_to_head([k[s] for s in rows], P)
    vl = seq_to_head([v[s] for s in rows], P)
    out_heads = [attention(ql[p], kl[p], vl[p], causal=causal)[0] for p in range(P)]
    return head_to_seq(out_heads, P), [x.shape for x in ql]


# ------------------------------------------------------------ USP hybrid
def usp_rank(rank: int, P_u: int) -> tuple[int, int]:
    """(Ulysses index u, ring group r) of a rank: the P_u ranks of one ring
    group are consecutive (Ulysses inside a node, Ring across nodes)."""
    return rank % P_u, rank // P_u


def usp_attention(q, k, v, P_u: int, P_r: int, layout: int = ZIGZAG, causal: bool = True):
    """The hybrid the handbook names in its comparison table and its GQA
    exercise (Ulysses inside a node, Ring Attention across nodes; 32 query
    heads on 8 KV heads over 16 ranks = 8-way Ulysses x 2-way ring).

    Reading: P = P_u * P_r ranks, rank = r * P_u + u.  The sequence is split
    over the P_r ring groups with ``layout``; inside group r its rows (in the
    group's local order) are cut into P_u consecutive shards, shard u on rank
    (u, r).  Then, as the pages' steps:
      1. seq_to_head inside every group (P_u-way all-to-all): rank (u, r)
         holds all of group r's rows for query heads u*Hq/P_u ... and KV
         heads u*Hkv/P_u ...;
      2. for every head share u, the ring over the P_r groups (the ring loop
         of ``layout``) on those heads;
      3. head_to_seq inside every group.
    Returns (outs, lses, positions): per rank its out [S/P, Hq, D], lse
    [Hq, S/P] and the natural positions of its rows.
    """
    q, k, v = (np.asarray(x, dtype=np.float64) if not hasattr(x, "detach")
               else x.detach().double().numpy() for x in (q, k, v))
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    if Hkv % P_u or Hq % Hkv or S % (P_u * P_r * (2 if layout == ZIGZAG else 1)):
        # the exercise: every Ulysses rank needs at least one whole KV head
        raise ValueError("USP needs P_u | Hkv, Hkv | Hq and the split to divide S")
    Sg = S // P_r
    Sl = Sg // P_u
    ring = {CONTIGUOUS: ring_contiguous, ZIGZAG: ring_zigzag, STRIPED: ring_striped}[layout]
    group_rows = [layout_index(layout, S, P_r, r) for r in range(P_r)]
    # 1. all-to-all inside each group, then the head shares reassembled over
    #    the whole sequence (what the P_r ranks with index u hold together)
    heads = {}
    for name, x in (("q", q), ("k", k), ("v", v)):
        full = [np.zeros((S, x.shape[1] // P_u, D)) for _ in range(P_u)]
        for r in range(P_r):
            shards = [x[group_rows[r][u * Sl:(u + 1) * Sl]] for u in range(P_u)]
            for u, y in enumerate(seq_to_head(shards, P_u)):
                full[u][group_rows[r]] = y
        heads[name] = full
    # 2. ring over the groups on each head share
    ring_out = [ring(heads["q"][u], heads["k"][u], heads["v"][u], P_r, causal=causal)[:2]
                for u in range(P_u)]
    # 3. all-to-all back inside each group; lse [Hp, Sg] follows the same
    #    route as a [Sg, Hp, 1] tensor
    outs, lses, positions = [None] * (P_u * P_r), [None] * (P_u * P_r), [None] * (P_u * P_r)
    for r in range(P_r):
        o = head_to_seq([ring_out[u][0][r] for u in range(P_u)], P_u)
        l = head_to_seq([ring_out[u][1][r].T[:, :, None] for u in range(P_u)], P_u)
        for u in range(P_u):
            outs[r * P_u + u] = o[u]
            lses[r * P_u + u] = l[u][:, :, 0].T
            positions[r * P_u + u] = group_rows[r][u * Sl:(u + 1) * Sl]
    return outs, lses, positions


def usp_bwd(q, k, v, dout, P_u: int, P_r: int, layout: int = ZIGZAG, causal: bool = True):
    """Backward of ``usp_attention`` (the pages give no algorithm; the
    plainest reading): per head share u the ring backward over the P_r
    groups (``ring_bwd``) on that share's query heads and KV heads -- the
    all-to-alls only move rows between ranks and leave every gradient where
    the forward's rows came from.  Returns dq, dk, dv in natural order."""
    q, k, v, dout = (np.asarray(x, dtype=np.float64) if not hasattr(x, "detach")
                     else x.detach().double().numpy() for x in (q, k, v, dout))
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    if Hkv % P_u or Hq % Hkv:
        raise ValueError("USP needs P_u | Hkv and Hkv | Hq")
    Hp, Hkp = Hq // P_u, Hkv // P_u
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for u in range(P_u):
        hs, ks = slice(u * Hp, (u + 1) * Hp), slice(u * Hkp, (u + 1) * Hkp)
        gq, gk, gv = ring_bwd(q[:, hs], k[:, ks], v[:, ks], dout[:, hs], P_r, layout, causal)
        dq[:, hs], dk[:, ks], dv[:, ks] = gq, gk, gv
    return dq, dk, dv


def usp_padded(q, k, v, P_u: int, P_r: int, layout: int = ZIGZAG, causal: bool = True):
    """USP when the ring split does not divide S (the practitioner blog's
    padding, section 7.1, applied to the ring groups): per head share u the
    padded ring over the P_r groups (``ring_padded``) on that share's heads;
    the all-to-all back then gives each group its real rows with every head.
    (The Ulysses shards of a group's rows are then of unequal length; the
    rows and their results are those of the padded ring.)

    Returns (outs, lses, positions) per ring group: out [n_r, Hq, D], lse
    [Hq, n_r] of the group's real rows in its local order, and their
    positions."""
    q, k, v = (np.asarray(x, dtype=np.float64) if not hasattr(x, "detach")
               else x.detach().double().numpy() for x in (q, k, v))
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    if Hkv % P_u or Hq % Hkv:
        raise ValueError("USP needs P_u | Hkv and Hkv | Hq")
    Hp, Hkp = Hq // P_u, Hkv // P_u
    shares = [ring_padded(q[:, u * Hp:(u + 1) * Hp], k[:, u * Hkp:(u + 1) * Hkp],
                          v[:, u * Hkp:(u + 1) * Hkp], P_r, layout, causal) for u in range(P_u)]
    outs = [np.concatenate([shares[u][0][r] for u in range(P_u)], axis=1) for r in range(P_r)]
    lses = [np.concatenate([shares[u][1][r] for u in range(P_u)], axis=0) for r in range(P_r)]
    return outs, lses, shares[0][2]
