"""Plain float64 definition of blockwise attention with per-row log-sum-exp.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Everything here follows the handbook page "上下文并行：Ring Attention 与
Ulysses" (Context parallelism: Ring Attention and Ulysses), section
"哪些运算可以直接切" (which operations split directly), whose ``attention``
function defines the operation, and its section "Ring Attention：KV 沿环传
一圈" for the merge.  Readings where the page is silent:

* a query row that sees no key gets ``lse = -inf`` and ``out = 0`` (the
  page's code would produce NaN there; the ring on that page never asks
  for such a row);
* grouped-query attention: query head ``h`` reads KV head
  ``h // (Hq // Hkv)`` (contiguous head groups, as the Ulysses section
  hands rank p the p-th contiguous share of heads).
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def _as_f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor (any dtype) -> exact float64
        import torch
        x = x.detach().to(torch.float64).cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def attention(q, k, v, causal: bool = True, q_offset: int = 0, k_offset: int = 0):
    """Single-pass attention of a query chunk against a key/value block.

    q: [Sq, Hq, D]; k, v: [Sk, Hkv, D]; offsets are the absolute sequence
    positions of row 0 of q and of k.  Returns ``out [Sq, Hq, D]`` and
    ``lse [Hq, Sq]`` (natural log), both float64.

    Steps, as in the handbook's ``attention``: scores = q.k / sqrt(D) with
    D the last dimension of q; keys whose absolute position exceeds the
    query's absolute position are masked (the diagonal stays visible);
    lse = logsumexp over the visible keys; out = sum_j exp(s_j - lse) v_j.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    Sq, Hq, D = q.shape
    Sk, Hkv, Dk = k.shape
    assert Dk == D and v.shape == k.shape and Hq % Hkv == 0
    group = Hq // Hkv
    out = np.zeros((Sq, Hq, D), dtype=np.float64)
    lse = np.full((Hq, Sq), NEG_INF, dtype=np.float64)
    qpos = np.arange(Sq)[:, None] + q_offset          # [Sq, 1]
    kpos = np.arange(Sk)[None, :] + k_offset          # [1, Sk]
    visible = (kpos <= qpos) if causal else np.ones((Sq, Sk), dtype=bool)
    for h in range(Hq):
        g = h // group
        scores = (q[:, h, :] @ k[:, g, :].T) / np.sqrt(D)     # [Sq, Sk]
        scores = np.where(visible, scores, NEG_INF)
        for i in range(Sq):
            row = scores[i][visible[i]]
            if row.size == 0:
                continue                                      # (0, -inf)
            m = row.max()
            lse[h, i] = m + np.log(np.exp(row - m).sum())
        has_key = np.isfinite(lse[h])
        w = np.where(visible & has_key[:, None],
                     np.exp(scores - np.where(has_key, lse[h], 0.0)[:, None]), 0.0)
        out[:, h, :] = w @ v[:, g, :]
    return out, lse


def lse_merge(o1, lse1, o2, lse2):
    """Fold two partial results over disjoint key sets into one.

    lse = log(e^lse1 + e^lse2); o = o1 e^(lse1 - lse) + o2 e^(lse2 - lse)
    (handbook, Ring Attention section).  o*: [Sq, H, D]; lse*: [H, Sq].
    A side with lse = -inf contributes nothing; two such sides give
    (0, -inf).
    """
    o1, lse1, o2, lse2 = map(_as_f64, (o1, lse1, o2, lse2))
    lse = np.logaddexp(lse1, lse2)
    finite = np.isfinite(lse)
    safe = np.where(finite, lse, 0.0)
    w1 = np.where(finite, np.exp(lse1 - safe), 0.0).T[..., None]   # [Sq, H, 1]
    w2 = np.where(finite, np.exp(lse2 - safe), 0.0).T[..., None]
    return o1 * w1 + o2 * w2, lse


def attention_global_max(q, k, v, key_parts, causal=True, q_offset=0, k_offset=0):
    """The distributed-softmax route of the "Sequence Parallel vs Context
    Parallel" blog, section 3.2: each part of the keys yields its local
    row max; the global max is the max of those; every part rescales its
    exp-scores by the global max; the normaliser is the sum over parts;
    out = (sum over parts of p.v) / normaliser.

    ``key_parts`` is a list of index arrays partitioning range(Sk).  Used
    only to cross-check the merge: it reaches the same numbers by another
    route.  Returns (out, lse) like ``attention``.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    Sq, Hq, D = q.shape
    Sk, Hkv, _ = k.shape
    group = Hq // Hkv
    qpos = np.arange(Sq)[:, None] + q_offset
    out = np.zeros((Sq, Hq, D))
    lse = np.full((Hq, Sq), NEG_INF)
    for h in range(Hq):
        g = h // group
        local = []
        for idx in key_parts:
            idx = np.asarray(idx, dtype=np.int64)
            s = (q[:, h, :] @ k[idx, g, :].T) / np.sqrt(D)
            if causal:
                s = np.where((idx[None, :] + k_offset) <= qpos, s, NEG_INF)
            local.append((idx, s, s.max(axis=1) if idx.size else np.full(Sq, NEG_INF)))
        m_global = np.max(np.stack([m for _, _, m in local]), axis=0)     # [Sq]
        m_safe = np.where(np.isfinite(m_global), m_global, 0.0)
        l_global = np.zeros(Sq)
        acc = np.zeros((Sq, D))
        for idx, s, _ in local:
            p = np.exp(s - m_safe[:, None])
            l_global += p.sum(axis=1)
            acc += p @ v[idx, g, :]
        nz = l_global > 0
        out[nz, h, :] = acc[nz] / l_global[nz, None]
        lse[h, nz] = m_safe[nz] + np.log(l_global[nz])
    return out, lse


def attention_bwd(q, k, v, dout, out, lse, causal: bool = True, q_offset: int = 0,
                  k_offset: int = 0):
    """Gradients (dq, dk, dv) of one query chunk against one KV block.

    The loss is ``sum(dout * out)`` where ``out`` / ``lse`` are the *final*
    results of the query rows over every key they see (this block alone, or
    all the blocks of a ring).  The block's share of each row's softmax is
    then ``P_ij = exp(s_ij - lse_i)``, so the gradients of several blocks
    add up to the gradient of the whole row.  With this block's own
    ``(out, lse)`` from ``attention`` it is the ordinary gradient of that
    function.

    Chain rule through out_i = sum_j P_ij v_j, P_ij = exp(s_ij - lse_i),
    lse_i = log sum_j exp(s_ij), s = q k^T / sqrt(D) (definitions of the
    handbook's ``attention``):

      dv_j  = sum_i P_ij dout_i
      dP_ij = dout_i . v_j
      Dv_i  = dout_i . out_i      (= sum over the row's keys of P_ij dP_ij)
      ds_ij = P_ij (dP_ij - Dv_i)
      dq_i  = sum_j ds_ij k_j / sqrt(D),   dk_j = sum_i ds_ij q_i / sqrt(D)

    Grouped-query attention: KV head g receives the sum over its query
    heads.  Rows with lse = -inf (no visible key) contribute nothing.
    Shapes as in ``attention``; dout and out [Sq, Hq, D], lse [Hq, Sq].
    Returns float64 dq [Sq, Hq, D], dk and dv [Sk, Hkv, D].
    """
    Sq, Sk = q.shape[0], k.shape[0]
    qpos = np.arange(Sq)[:, None] + q_offset
    kpos = np.arange(Sk)[None, :] + k_offset
    visible = (kpos <= qpos) if causal else np.ones((Sq, Sk), dtype=bool)
    return _bwd_masked(q, k, v, dout, out, lse, visible)


def attention_bwd_at(q, k, v, dout, out, lse, qpos, kpos, causal: bool = True):
    """``attention_bwd`` with explicit absolute positions (as ``attention_at``)."""
    qp = np.asarray(qpos, dtype=np.int64)[:, None]
    kp = np.asarray(kpos, dtype=np.int64)[None, :]
    visible = (kp <= qp) if causal else np.ones((qp.shape[0], kp.shape[1]), dtype=bool)
    return _bwd_masked(q, k, v, dout, out, lse, visible)


def _bwd_masked(q, k, v, dout, out, lse, visible):
    """The chain rule of ``attention_bwd`` for a given visibility matrix."""
    q, k, v, dout, out, lse = map(_as_f64, (q, k, v, dout, out, lse))
    Sq, Hq, D = q.shape
    Sk, Hkv, _ = k.shape
    group = Hq // Hkv
    dq = np.zeros((Sq, Hq, D))
    dk = np.zeros((Sk, Hkv, D))
    dv = np.zeros((Sk, Hkv, D))
    scale = 1.0 / np.sqrt(D)
    for h in range(Hq):
        g = h // group
        finite = np.isfinite(lse[h])
        s = (q[:, h, :] @ k[:, g, :].T) * scale
        p = np.where(visible & finite[:, None],
                     np.exp(s - np.where(finite, lse[h], 0.0)[:, None]), 0.0)   # [Sq, Sk]
        dv[:, g, :] += p.T @ dout[:, h, :]
        dp = dout[:, h, :] @ v[:, g, :].T
        dvec = np.sum(dout[:, h, :] * out[:, h, :], axis=1)                      # [Sq]
        ds = p * (dp - dvec[:, None])
        dq[:, h, :] = ds @ k[:, g, :] * scale
        dk[:, g, :] += ds.T @ q[:, h, :] * scale
    return dq, dk, dv


def attention_at(q, k, v, qpos, kpos, causal: bool = True, kvalid=None):
    """``attention`` with explicit absolute positions: key j is visible to
    query i iff kpos[j] <= qpos[i] (the handbook's mask, whose positions are
    q_offset + i and k_offset + j, for any position arrays -- needed when a
    rank's rows are not one contiguous run, as in the striped split).
    ``kvalid`` (bool per key, optional) removes the keys marked False from
    every row's visible set (padding keys).
    Returns (out [Sq, Hq, D], lse [Hq, Sq]) like ``attention``.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    Sq, Hq, D = q.shape
    Sk, Hkv, _ = k.shape
    group = Hq // Hkv
    qp = np.asarray(qpos, dtype=np.int64)[:, None]
    kp = np.asarray(kpos, dtype=np.int64)[None, :]
    visible = (kp <= qp) if causal else np.ones((Sq, Sk), dtype=bool)
    if kvalid is not None:
        visible = visible & np.asarray(kvalid, dtype=bool)[None, :]
    out = np.zeros((Sq, Hq, D))
    lse = np.full((Hq, Sq), NEG_INF)
    for h in range(Hq):
        g = h // group
        s = np.where(visible, (q[:, h, :] @ k[:, g, :].T) / np.sqrt(D), NEG_INF)
        has = visible.any(axis=1)
        m = np.where(has, s.max(axis=1, initial=NEG_INF), 0.0)
        e = np.where(visible, np.exp(s - m[:, None]), 0.0)
        tot = e.sum(axis=1)
        lse[h, has] = m[has] + np.log(tot[has])
        out[has, h, :] = (e[has] / tot[has, None]) @ v[:, g, :]
    return out, lse
