"""SVG-EAR: centroid compensation of skipped blocks and error-aware routing
(oracle; TEST INFRASTRUCTURE, float64).

Source: the Sparse-VideoGen write-up, section "Three generations of the same
idea": SVG-EAR recovers the attention blocks the sparse pattern skips with a
parameter-free centroid compensation, and routes the blocks with a high error
to exact computation while compensating the others.  (A related-work list on
the USV page names it "parameter-free linear compensation ... via error-aware
routing".)  The pages give no formulas, so the steps below are this
library's reading, stated in full:

Per head, in the executing layout, kv-block b = keys 64 b .. 64 b + 63 that
exist (j < N), n_b of them:
  centroid key   kbar_b = mean of the block's K rows,
  mean value     vbar_b = mean of its V rows,
  key radius     r_b    = max_j || k_j - kbar_b ||_2.

Compensated attention.  A query i of q-block Q attends exactly the keys of
the blocks in its exact set X_Q; every other block b contributes as n_b
copies of (kbar_b, vbar_b):
  O_i = (sum_{j in X_Q} e^{s_ij} v_j + sum_{b not in X_Q} n_b e^{t_ib} vbar_b)
        / (sum_{j in X_Q} e^{s_ij} + sum_{b not in X_Q} n_b e^{t_ib}),
  s_ij = tau q_i . k_j,  t_ib = tau q_i . kbar_b,  tau = 1/sqrt(d).
This is the softmax over the exact keys plus one centroid key per skipped
block with log-weight ln n_b: parameter-free, and exact when a skipped
block's keys are all equal (then e^{s_ij} = e^{t_ib} for each of them).

Error-aware routing.  For the block b's keys |s_ij - t_ib| <= tau ||q_i||
r_b, so the centroid's stand-in for the block's attention mass errs by at
most n_b e^{t_ib} (e^{tau ||q_i|| r_b} - 1).  Evaluated at the q-block's
mean query qbar_Q this gives the block's error score
  E_Qb = n_b exp(tau qbar_Q . kbar_b) (exp(tau ||qbar_Q|| r_b) - 1),
compared in the log domain (ln n_b + tau qbar . kbar_b + ln(expm1(tau
||qbar|| r_b)); -inf when r_b = 0, whose compensation is exact).  X_Q is the
block mask's kept set, plus the ragged last block (fewer than 64 keys: it is
always exact, so every compensated block has n_b = 64), plus the route_k
skipped blocks of largest E_Qb (ties to the lower block index), or all
skipped blocks if there are fewer.
"""

import numpy as np

from .attention import default_scale


def block_stats(k, v, bk: int = 64):
    """n, kbar, vbar, radius per kv-block of one head (k, v: [N][d])."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, d = k.shape
    nkb = -(-N // bk)
    n = np.zeros(nkb, dtype=np.int64)
    kbar = np.zeros((nkb, d))
    vbar = np.zeros((nkb, d))
    rad = np.zeros(nkb)
    for b in range(nkb):
        kb, vb = k[b * bk:(b + 1) * bk], v[b * bk:(b + 1) * bk]
        n[b] = kb.shape[0]
        kbar[b] = kb.mean(axis=0)
        vbar[b] = vb.mean(axis=0)
        rad[b] = np.sqrt(((kb - kbar[b]) ** 2).sum(axis=1)).max()
    return n, kbar, vbar, rad


def route_scores(q, n, kbar, rad, bq: int, scale=None):
    """log E_Qb for every (q-block, kv-block) of one head: [nQB][nKB]."""
    q = np.asarray(q, dtype=np.float64)
    N, d = q.shape
    tau = default_scale(d) if scale is None else scale
    nqb = -(-N // bq)
    out = np.empty((nqb, kbar.shape[0]))
    with np.errstate(divide="ignore"):
        for Q in range(nqb):
            qbar = q[Q * bq:(Q + 1) * bq].mean(axis=0)
            out[Q] = np.log(n) + tau * (kbar @ qbar) + np.log(np.expm1(tau * np.linalg.norm(qbar) * rad))
    return out


def exact_sets(bitmap, scores, N: int, bk: int, route_k: int):
    """The exact sets X_Q as a bitmap [nQB][nKB]: the kept tiles, the ragged
    last block, and the route_k skipped blocks of largest score (ties to the
    lower index)."""
    x = (np.asarray(bitmap) != 0).astype(np.uint8).copy()
    nkb = x.shape[1]
    if N % bk:
        x[:, nkb - 1] = 1
    for Q in range(x.shape[0]):
        skipped = np.flatnonzero(x[Q] == 0)
        if skipped.size == 0:
            continue
        # descending score, ascending index on ties (a stable sort of -score)
        order = skipped[np.argsort(-scores[Q, skipped], kind="stable")]
        x[Q, order[:route_k]] = 1
    return x


def ear_attention(q, k, v, exact, bq: int, bk: int = 64, scale=None, qblocks=None):
    """Compensated attention of one head (q, k, v: [N][d] float64, executing
    layout; exact: [nQB][nKB] bitmap of the exact sets).  {qb: O rows}."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, d = q.shape
    tau = default_scale(d) if scale is None else scale
    n, kbar, vbar, _ = block_stats(k, v, bk)
    nqb = exact.shape[0]
    out = {}
    for Q in (range(nqb) if qblocks is None else qblocks):
        qq = q[Q * bq:min(N, (Q + 1) * bq)]
        xs = np.flatnonzero(exact[Q])
        comp = np.flatnonzero(exact[Q] == 0)
        cols = np.concatenate([np.arange(b * bk, min(N, (b + 1) * bk)) for b in xs]) if xs.size else \
            np.zeros(0, dtype=np.int64)
        logits = np.concatenate([tau * (qq @ k[cols].T), tau * (qq @ kbar[comp].T) + np.log(n[comp])], axis=1)
        vals = np.concatenate([v[cols], vbar[comp]], axis=0)
        if logits.shape[1] == 0:
            out[Q] = np.zeros((qq.shape[0], d))
            continue
        m = logits.max(axis=1, keepdims=True)
        p = np.exp(logits - m)
        out[Q] = (p @ vals) / p.sum(axis=1, keepdims=True)
    return out
