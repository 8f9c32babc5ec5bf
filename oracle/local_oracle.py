"""CPU oracle for local (sliding-chunk) self-attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares
no code with the HIP library and does not import it.

Source: "The Reformer - Pushing the limits of language modeling" (summary
page), *Approach / What changed* and *Takeaways*: local self-attention cuts the
input into chunks of length l_c and lets each chunk attend to itself plus an
overlap from the preceding and following chunks, so positions keep access to
their immediate neighbours.

Readings where the page is silent (listed in the repository's design notes):

* queries, keys and values are separate inputs (q may equal k);
* chunk length ``m' = min(l_c, L)`` with L a multiple of m'; chunk of
  position i is ``c = i // m'``;
* the window of i is every position of chunks ``c - n_before .. c + n_after``
  that exist (no wrap-around); causal keeps only positions ``j <= i``;
* no self-mask: i is always in its own window;
* score ``q_i . k_j / sqrt(d)``, one softmax over the window, float64.
"""
from __future__ import annotations

import math

import numpy as np


def local_window(i: int, L: int, chunk_len: int, n_before: int, n_after: int, causal: bool) -> range:
    """Key positions visible to query i."""
    m = min(int(chunk_len), L)
    if m < 1 or L % m != 0:
        raise ValueError(f"seq_len {L} must be a multiple of chunk_len {chunk_len} (or chunk_len >= seq_len)")
    if n_before < 0 or n_after < 0:
        raise ValueError("n_before and n_after must be >= 0")
    c = i // m
    lo = max(0, (c - n_before) * m)
    hi = min(L, (c + 1 + n_after) * m)
    if causal:
        hi = min(hi, i + 1)
    return range(lo, hi)


def local_attention_head(q, k, v, chunk_len: int, n_before: int, n_after: int, causal: bool):
    """Local attention for one (batch, head) slice: ``q, k, v [L, d]`` -> ``out [L, d]``."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    L, d = q.shape
    scale = 1.0 / math.sqrt(d)
    out = np.empty((L, v.shape[1]), np.float64)
    for i in range(L):
        w = local_window(i, L, chunk_len, n_before, n_after, causal)
        s = (k[w.start:w.stop] @ q[i]) * scale
        e = np.exp(s - s.max())
        out[i] = (e / e.sum()) @ v[w.start:w.stop]
    return out


def local_attention(q, k, v, chunk_len: int, n_before: int, n_after: int, causal: bool):
    """``q, k, v [B, H, L, d]`` -> ``out [B, H, L, d]`` (float64)."""
    q = np.asarray(q)
    B, H = q.shape[:2]
    out = np.empty(q.shape[:3] + (np.asarray(v).shape[3],), np.float64)
    for b in range(B):
        for h in range(H):
            out[b, h] = local_attention_head(q[b, h], k[b, h], v[b, h], chunk_len, n_before, n_after, causal)
    return out
