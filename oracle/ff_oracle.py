"""CPU oracle for the position-wise feed-forward layer, whole or in chunks.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares
no code with the HIP library and does not import it.

Source: "Reformer: The Efficient Transformer" (research summary), *Summary*
(feed-forward layers are processed in chunks) and *Key points*, reversible
layers bullet (run a chunk of positions at a time, the feed-forward layers
no longer hold a d_ff-wide activation for the whole sequence, and the results
do not change).  The layer acts on each
position independently, so cutting the positions into chunks changes nothing
but the size of the d_ff-wide intermediate held at one time.

Readings (listed in the design notes): ``y = relu(x W1^T + b1) W2^T + b2`` with
weights in the output-feature-major layout of a linear layer (``W1 [d_ff, d]``,
``W2 [d, d_ff]``); the pages name no activation, ReLU is the plainest choice.
"""
from __future__ import annotations

import numpy as np


def feed_forward(x, w1, b1, w2, b2):
    """``x [n, d]`` -> ``[n, d]`` in float64, one position at a time.

    Each row goes through the same matrix-vector products, so the result of a
    row does not depend on how many rows are processed together (a batched
    matrix product may change its summation order with the batch size).
    """
    x = np.asarray(x, np.float64)
    w1 = np.asarray(w1, np.float64)
    b1 = np.asarray(b1, np.float64)
    w2 = np.asarray(w2, np.float64)
    b2 = np.asarray(b2, np.float64)
    out = np.empty((x.shape[0], w2.shape[0]), np.float64)
    for i in range(x.shape[0]):
        h = np.maximum(w1 @ x[i] + b1, 0.0)
        out[i] = w2 @ h + b2
    return out


def chunked_feed_forward(x, w1, b1, w2, b2, chunk: int):
    """The same layer applied to ``chunk`` positions at a time."""
    x = np.asarray(x, np.float64)
    if chunk < 1:
        raise ValueError("chunk must be >= 1")
    parts = [feed_forward(x[i:i + chunk], w1, b1, w2, b2) for i in range(0, x.shape[0], chunk)]
    return np.concatenate(parts, axis=0) if parts else np.zeros((0, np.asarray(w2).shape[0]))
