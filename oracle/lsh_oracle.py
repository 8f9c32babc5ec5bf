"""CPU oracle for the Reformer's shared-QK LSH self-attention forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares
no code with the HIP library (no kernels, headers, helpers or tables) and does
not import it; the only thing both sides share is the seeded input generator,
which holds none of the method's arithmetic.

Everything is float64 numpy, written to be read against the pages, not to be
fast.  Sources (page titles as they appear on the pages):

* "Reformer: The Efficient Transformer" (research summary page), *Summary*:
  queries and keys share one projection, are hashed with random rotations,
  sorted by bucket, and attention runs inside small fixed-size chunks; several
  hash rounds are used.
* same page, *Key points*, "LSH attention" bullet: ``h(x) = argmax([xR; -xR])``
  with a random matrix R; the sorted positions are cut into chunks of m, and
  the queries of a chunk see the keys of that chunk and of the preceding one.
* same page, *Key points*, "Shared-QK Transformer" bullet: a position's own
  key is excluded, except when nothing else is left for it to attend to.
* same page, *Key points*, "Number of hash rounds" bullet: more rounds come
  closer to full attention.

Where the pages are silent the oracle takes these readings (each is listed,
with its reason, in the repository's design notes):

* R has shape ``[n_rounds, d, n_buckets/2]``, one independent matrix per round,
  shared by every batch row and head.
* ``[xR; -xR]`` is a concatenation along the bucket axis: bucket ``k < b/2``
  is ``+(xR)_k`` and bucket ``b/2 + k`` is ``-(xR)_k``.
* argmax ties go to the lowest index (numpy's convention).
* ``n_buckets == 1`` puts every position in bucket 0 and never reads R; any
  other odd bucket count is rejected.
* sort key is (bucket, original position), ascending; rounds are independent.
* chunk length is ``m' = min(chunk_len, L)``; L must be a multiple of m' .
  The first chunk of a round has no predecessor (no wrap-around).
* every key in the window (own chunk + previous chunk) is eligible; there is
  no same-bucket mask.
* score ``s_ij = x_i . x_j / sqrt(d)`` with the raw shared vector as both
  query and key.
* optional causal mask by original positions: key j is allowed for query i
  only if ``j < i`` (``j == i`` is the self case, handled below).
* whether anything else is left is decided over all rounds together: a round with
  no non-self target contributes nothing (log-normaliser ``-inf``); if no
  round has any, the output is the token's own value vector.
* rounds are combined with logsumexp weights: ``out_i = sum_r
  exp(z_r(i) - Z_i) o_r(i)`` with ``Z_i = logsumexp_r z_r(i)``; a key seen in
  k rounds therefore counts k times.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "lsh_hash",
    "lsh_sort",
    "chunk_attention_round",
    "combine_rounds",
    "lsh_attention_head",
    "lsh_attention",
    "attend_positions",
    "exact_projection_margin",
]


def _check_buckets(n_buckets: int) -> None:
    if n_buckets < 1 or (n_buckets != 1 and n_buckets % 2 != 0):
        raise ValueError(f"n_buckets must be 1 or even, got {n_buckets}")


def lsh_hash(x, rotations, n_buckets: int):
    """Bucket ids of one head's vectors for every hash round.

    Follows "Reformer: The Efficient Transformer", *Key points*, LSH attention
    bullet: ``h(x) = argmax([xR; -xR])``.

    x: ``[L, d]`` (upcast to float64).  rotations: ``[r, d, n_buckets/2]``
    (ignored, may be None, when ``n_buckets == 1``; then ``n_rounds`` is taken
    from ``rotations.shape[0]`` if given, else 1).

    Returns ``(buckets int64 [r, L], margin float64 [r, L])`` where ``margin``
    is the gap between the largest and second largest entry of ``[xR; -xR]``
    (``+inf`` when there is one bucket).  The margin is what decides whether a
    float32 implementation may legitimately pick a different bucket.
    """
    _check_buckets(n_buckets)
    x = np.asarray(x, dtype=np.float64)
    L = x.shape[0]
    if n_buckets == 1:
        r = 1 if rotations is None else int(np.asarray(rotations).shape[0])
        return np.zeros((r, L), np.int64), np.full((r, L), np.inf)
    R = np.asarray(rotations, dtype=np.float64)
    r, d, half = R.shape
    if d != x.shape[1] or half != n_buckets // 2:
        raise ValueError("rotations must be [n_rounds, d, n_buckets/2]")
    buckets = np.empty((r, L), np.int64)
    margin = np.empty((r, L), np.float64)
    rows = max(1, (1 << 23) // n_buckets)   # bound the [rows, b] temporaries (64 MiB)
    for rho in range(r):
        for a in range(0, L, rows):
            e = min(L, a + rows)
            p = x[a:e] @ R[rho]                   # projections, [rows, b/2]
            y = np.concatenate([p, -p], axis=1)   # [xR; -xR] along the bucket axis
            buckets[rho, a:e] = np.argmax(y, axis=1)   # first index of the maximum
            top2 = np.partition(y, n_buckets - 2, axis=1)[:, -2:]
            margin[rho, a:e] = top2[:, 1] - top2[:, 0]
    return buckets, margin


def exact_projection_margin(x_row, rotation, n_buckets: int):
    """Exact argmax and margin for a single vector with rational arithmetic.

    Used by tests on tiny inputs: every float64 value is converted exactly to a
    ``fractions.Fraction`` so the projection has no rounding at all.
    """
    from fractions import Fraction

    xs = [Fraction(float(t)) for t in np.asarray(x_row, np.float64)]
    R = np.asarray(rotation, np.float64)
    half = n_buckets // 2
    p = []
    for k in range(half):
        p.append(sum((xs[j] * Fraction(float(R[j, k])) for j in range(len(xs))), Fraction(0)))
    y = p + [-t for t in p]
    best = 0
    for k in range(1, len(y)):
        if y[k] > y[best]:
            best = k
    ordered = sorted(y, reverse=True)
    return best, ordered[0] - ordered[1]


def lsh_sort(buckets):
    """Stable sort of every round by (bucket, position).

    "Reformer: The Efficient Transformer", *Summary* (sorted by bucket) and
    *Key points*, LSH attention bullet ("after sorting").

    buckets: ``[r, L]`` integers.  Returns ``(perm, inv)`` int64 ``[r, L]``:
    ``perm[rho, s]`` is the original position at sorted slot ``s`` and
    ``inv[rho, perm[rho, s]] = s``.
    """
    buckets = np.asarray(buckets)
    r, L = buckets.shape
    pos = np.arange(L)
    perm = np.empty((r, L), np.int64)
    inv = np.empty((r, L), np.int64)
    for rho in range(r):
        perm[rho] = np.lexsort((pos, buckets[rho]))  # primary key: bucket
        inv[rho, perm[rho]] = pos
    return perm, inv


def _chunk_len(chunk_len: int, L: int) -> int:
    m = min(int(chunk_len), L)
    if m < 1 or L % m != 0:
        raise ValueError(f"seq_len {L} must be a multiple of chunk_len {chunk_len} (or chunk_len >= seq_len)")
    return m


def chunk_attention_round(x, v, perm, chunk_len: int, causal: bool):
    """One hash round of chunked attention, returned in sequence order.

    "Reformer: The Efficient Transformer", *Key points*: the sorted positions
    form chunks of m whose queries see the keys of their own chunk and of the
    preceding one (LSH attention bullet); queries and keys are the same
    vectors and a position's own key is excluded (Shared-QK bullet).

    x, v: ``[L, d]``; perm: ``[L]`` (original position at each sorted slot).
    Returns ``(o [L, d], z [L])`` indexed by original position:
    ``z_i = log sum_{j in T(i)} exp(s_ij)`` and ``o_i = sum_j exp(s_ij - z_i) v_j``
    over the valid non-self targets ``T(i)`` of the round; a position with no
    such target gets ``o_i = 0`` and ``z_i = -inf``.
    """
    x = np.asarray(x, np.float64)
    v = np.asarray(v, np.float64)
    perm = np.asarray(perm)
    L, d = x.shape
    m = _chunk_len(chunk_len, L)
    scale = 1.0 / math.sqrt(d)
    xs, vs = x[perm], v[perm]
    o_sorted = np.zeros((L, v.shape[1]), np.float64)
    z_sorted = np.full(L, -np.inf)
    for c in range(L // m):
        q = slice(c * m, (c + 1) * m)                  # the chunk's own slots
        k = slice(max(0, (c - 1) * m), (c + 1) * m)    # previous chunk + own chunk
        pq, pk = perm[q], perm[k]
        s = (xs[q] @ xs[k].T) * scale
        valid = pk[None, :] != pq[:, None]             # no attention to self
        if causal:
            valid &= pk[None, :] < pq[:, None]         # no attention to later positions
        s = np.where(valid, s, -np.inf)
        row_max = s.max(axis=1)
        has = np.isfinite(row_max)
        shift = np.where(has, row_max, 0.0)
        e = np.where(valid, np.exp(s - shift[:, None]), 0.0)
        total = e.sum(axis=1)
        with np.errstate(divide="ignore", invalid="ignore"):
            z_sorted[q] = np.where(has, shift + np.log(total), -np.inf)
            o_sorted[q] = np.where(has[:, None], (e @ vs[k]) / total[:, None], 0.0)
    o = np.empty_like(o_sorted)
    z = np.empty_like(z_sorted)
    o[perm] = o_sorted     # un-sort: slot s belongs to position perm[s]
    z[perm] = z_sorted
    return o, z


def combine_rounds(o, z, v):
    """Combine the per-round results with logsumexp weights.

    o: ``[r, L, d]``, z: ``[r, L]``, v: ``[L, d]``.  ``out_i = sum_r
    exp(z_r(i) - Z_i) o_r(i)`` with ``Z_i = logsumexp_r z_r(i)``.  When every
    round has ``z = -inf`` (no valid non-self target anywhere) the token falls
    back to attending to itself, whose only target is itself: ``out_i = v_i``
    ("Reformer: The Efficient Transformer", *Key points*, Shared-QK bullet).
    """
    o = np.asarray(o, np.float64)
    z = np.asarray(z, np.float64)
    v = np.asarray(v, np.float64)
    z_max = z.max(axis=0)
    fallback = ~np.isfinite(z_max)
    shift = np.where(fallback, 0.0, z_max)
    w = np.exp(z - shift[None, :])                    # exp(-inf) = 0 for empty rounds
    total = w.sum(axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        w = np.where(fallback[None, :], 0.0, w / total[None, :])
    out = np.einsum("rl,rld->ld", w, o)
    out[fallback] = v[fallback]
    return out


def lsh_attention_head(x, v, rotations, n_buckets, chunk_len, causal, buckets=None, perm=None):
    """Full forward pass for one (batch, head) slice.

    Hash -> sort -> chunked attention per round -> logsumexp combine with the
    self fallback -> output in sequence order.  ``buckets`` may be supplied
    (e.g. to consume another implementation's bucket ids, so that a near-tie
    flip does not reshuffle a whole bucket range); ``perm`` may be supplied to
    bypass hashing and sorting altogether.

    Returns a dict with ``out [L, d]`` and the intermediates ``buckets``,
    ``margin``, ``perm``, ``inv``, ``o [r, L, d]`` and ``z [r, L]``.
    """
    x = np.asarray(x, np.float64)
    v = np.asarray(v, np.float64)
    margin = None
    if perm is None:
        if buckets is None:
            buckets, margin = lsh_hash(x, rotations, n_buckets)
        perm, inv = lsh_sort(buckets)
    else:
        perm = np.asarray(perm)
        inv = np.empty_like(perm)
        for rho in range(perm.shape[0]):
            inv[rho, perm[rho]] = np.arange(perm.shape[1])
    r = perm.shape[0]
    o = np.empty((r,) + v.shape, np.float64)
    z = np.empty((r, x.shape[0]), np.float64)
    for rho in range(r):
        o[rho], z[rho] = chunk_attention_round(x, v, perm[rho], chunk_len, causal)
    out = combine_rounds(o, z, v)
    return {"out": out, "buckets": buckets, "margin": margin, "perm": perm, "inv": inv, "o": o, "z": z}


def lsh_attention(qk, v, rotations, n_buckets, chunk_len, causal, buckets=None):
    """Forward pass over ``[B, H, L, d]`` inputs, one (batch, head) at a time.

    ``buckets``, if given, is ``[B, H, r, L]``.  Returns ``out [B, H, L, d]``
    (float64) and ``buckets`` / ``margin`` ``[B, H, r, L]``.
    """
    qk = np.asarray(qk, np.float64)
    v = np.asarray(v, np.float64)
    B, H, L, d = qk.shape
    out = np.empty(v.shape, np.float64)
    all_b, all_m = [], []
    for b in range(B):
        row_b, row_m = [], []
        for h in range(H):
            res = lsh_attention_head(qk[b, h], v[b, h], rotations, n_buckets, chunk_len, causal,
                                     buckets=None if buckets is None else buckets[b, h])
            out[b, h] = res["out"]
            row_b.append(res["buckets"])
            row_m.append(res["margin"])
        all_b.append(row_b)
        all_m.append(row_m)
    bk = np.asarray(all_b)
    mg = None if all_m[0][0] is None else np.asarray(all_m)
    return {"out": out, "buckets": bk, "margin": mg}


def attend_positions(x, v, perm, inv, positions, chunk_len: int, causal: bool):
    """Output rows for selected positions only, computed one position at a time.

    The same definition as ``chunk_attention_round`` + ``combine_rounds``, but
    written per query so that sampled rows of very long sequences can be
    checked without the whole attention: for each round the query's chunk is
    ``slot // m`` and its window is the previous chunk plus its own.

    perm, inv: ``[r, L]``.  Returns ``(out [n, d], o [r, n, d], z [r, n])``.
    """
    x = np.asarray(x, np.float64)
    v = np.asarray(v, np.float64)
    L, d = x.shape
    m = _chunk_len(chunk_len, L)
    r = perm.shape[0]
    positions = np.asarray(positions, np.int64)
    n = positions.shape[0]
    o = np.zeros((r, n, v.shape[1]), np.float64)
    z = np.full((r, n), -np.inf)
    scale = 1.0 / math.sqrt(d)
    for t, i in enumerate(positions):
        for rho in range(r):
            c = int(inv[rho, i]) // m
            keys = perm[rho, max(0, (c - 1) * m):(c + 1) * m]
            keys = keys[keys != i]
            if causal:
                keys = keys[keys < i]
            if keys.size == 0:
                continue
            s = (x[keys] @ x[i]) * scale
            top = s.max()
            e = np.exp(s - top)
            z[rho, t] = top + math.log(e.sum())
            o[rho, t] = (e / e.sum()) @ v[keys]
    out = np.empty((n, v.shape[1]), np.float64)
    for t, i in enumerate(positions):
        zt = z[:, t]
        if not np.isfinite(zt).any():
            out[t] = v[i]
            continue
        top = zt.max()
        w = np.exp(zt - top)
        out[t] = (w / w.sum()) @ o[:, t, :]
    return out, o, z
