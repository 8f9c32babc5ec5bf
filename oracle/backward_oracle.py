"""Gradients of the shared-QK LSH attention forward (test infrastructure).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares
no code with the HIP library and does not import it.

Reading (the pages give no backward): the bucket ids, hence the sorted order,
are piecewise constant in the inputs, so they are held fixed and gradients
flow through the attention scores and the values only.  With that, the
forward of "Reformer: The Efficient Transformer" (research summary), Key
points (LSH attention, Shared-QK and Number of hash rounds bullets) combined
with logsumexp weights is one softmax per query over the multiset of
(round, key) pairs it sees:

    out_i = sum_j M_ij exp(s_ij) v_j / sum_j M_ij exp(s_ij),  s_ij = x_i . x_j / sqrt(d)

where ``M_ij`` counts the rounds in which key j is a valid (non-self, and if
causal earlier) target of i.  Rows with no target at all return ``v_i`` (the
self fallback).  This module writes that dense form in float64 torch and
differentiates it with ``torch.autograd``; the tests check the dense form
against the round-by-round oracle and the gradients against finite
differences.
"""
from __future__ import annotations

import math

import numpy as np
import torch


def target_counts(perm, chunk_len: int, causal: bool) -> np.ndarray:
    """``M [L, L]``: in how many rounds key j is a valid target of query i.

    perm: ``[r, L]`` sorted order of each round.  A query in chunk c of a
    round sees the slots of chunks c-1 (if any) and c, except itself and, if
    causal, positions not before its own.
    """
    perm = np.asarray(perm)
    r, L = perm.shape
    m = min(int(chunk_len), L)
    if m < 1 or L % m != 0:
        raise ValueError(f"seq_len {L} must be a multiple of chunk_len {chunk_len} (or chunk_len >= seq_len)")
    M = np.zeros((L, L), np.int64)
    for rho in range(r):
        for s in range(L):
            c = s // m
            i = perm[rho, s]
            for w in range(max(0, (c - 1) * m), (c + 1) * m):
                j = perm[rho, w]
                if j == i or (causal and j >= i):
                    continue
                M[i, j] += 1
    return M


def dense_forward(x: torch.Tensor, v: torch.Tensor, M: np.ndarray) -> torch.Tensor:
    """The combined forward in the dense multiset form (float64 torch)."""
    L, d = x.shape
    Mt = torch.from_numpy(M).to(torch.float64)
    s = (x @ x.T) / math.sqrt(d)
    has = Mt.sum(dim=1) > 0
    logits = torch.where(Mt > 0, s + torch.log(torch.where(Mt > 0, Mt, torch.ones_like(Mt))),
                         torch.full_like(s, -math.inf))
    out = v.clone()
    idx = torch.nonzero(has).flatten()
    if idx.numel():
        p = torch.softmax(logits[idx], dim=1)
        out = out.index_put((idx,), p @ v)
    return out


def lsh_attention_head_grad(x, v, perm, chunk_len: int, causal: bool, dout):
    """``(out, dx, dv)`` for one (batch, head) slice, float64 numpy arrays.

    dout is the gradient of the loss with respect to ``out``; the returned
    ``dx`` collects both roles of the shared vector (query and key).
    """
    M = target_counts(perm, chunk_len, causal)
    xt = torch.tensor(np.asarray(x, np.float64), requires_grad=True)
    vt = torch.tensor(np.asarray(v, np.float64), requires_grad=True)
    out = dense_forward(xt, vt, M)
    out.backward(torch.from_numpy(np.asarray(dout, np.float64)))
    return out.detach().numpy(), xt.grad.numpy(), vt.grad.numpy()


def _targets(perm, inv, i: int, m: int, causal: bool):
    """Targets of query i over all rounds with their multiplicities M_ij
    (the sparse row i of ``target_counts``)."""
    r, L = perm.shape
    keys = []
    for rho in range(r):
        c = inv[rho, i] // m
        w = perm[rho, max(0, (c - 1) * m):(c + 1) * m]
        w = w[w != i]
        if causal:
            w = w[w < i]
        keys.append(w)
    return np.unique(np.concatenate(keys), return_counts=True)


def _observers(perm, inv, k: int, m: int, causal: bool):
    """Queries that have key k among their targets in some round: those in
    k's own chunk and the chunk after it."""
    r, L = perm.shape
    obs = []
    for rho in range(r):
        c = inv[rho, k] // m
        w = perm[rho, c * m:min(L, (c + 2) * m)]
        w = w[w != k]
        if causal:
            w = w[w > k]
        obs.append(w)
    return np.unique(np.concatenate(obs))


def grad_positions(x, v, perm, positions, chunk_len: int, causal: bool, dout):
    """``(dx, dv)`` of the dense multiset form at the given positions only,
    float64, written out with the softmax derivative instead of autograd, so
    that it scales to long sequences (each position touches a few chunks).

    With P_i = softmax_j(s_ij + log M_ij), out_i = sum_j P_ij v_j and
    dS_ij = P_ij (dout_i . v_j - dout_i . out_i):
        dv_k = sum_i P_ik dout_i                       (+ dout_k if k has no target)
        dx_k = (sum_j dS_kj x_j + sum_i dS_ik x_i) / sqrt(d)
    where the first sum is k's own row (k as query) and the second runs over
    the queries that see k (k as key).
    """
    x = np.asarray(x, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(dout, np.float64)
    perm = np.asarray(perm)
    r, L = perm.shape
    d = x.shape[1]
    m = min(int(chunk_len), L)
    if m < 1 or L % m != 0:
        raise ValueError(f"seq_len {L} must be a multiple of chunk_len {chunk_len} (or chunk_len >= seq_len)")
    inv = np.empty_like(perm)
    for rho in range(r):
        inv[rho, perm[rho]] = np.arange(L)
    scale = 1.0 / math.sqrt(d)
    rows = {}

    def row(i):
        if i not in rows:
            j, cnt = _targets(perm, inv, i, m, causal)
            if j.size == 0:
                rows[i] = None
            else:
                logit = (x[j] @ x[i]) * scale + np.log(cnt)
                p = np.exp(logit - logit.max())
                p /= p.sum()
                out = p @ v[j]
                ds = p * (v[j] @ g[i] - g[i] @ out)
                rows[i] = (j, p, ds)
        return rows[i]

    pos = np.asarray(positions, np.int64)
    dx = np.zeros((pos.size, d))
    dv = np.zeros((pos.size, d))
    for n, k in enumerate(pos):
        own = row(int(k))
        if own is None:
            dv[n] += g[k]
        else:
            j, _, ds = own
            dx[n] += ds @ x[j]
        for i in _observers(perm, inv, int(k), m, causal):
            j, p, ds = row(int(i))
            t = np.searchsorted(j, k)
            dv[n] += p[t] * g[i]
            dx[n] += ds[t] * x[i]
        dx[n] *= scale
    return dx, dv
