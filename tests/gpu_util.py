"""Helpers shared by the GPU parity tests (device upload, oracle comparisons)."""
import os

import numpy as np

import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2}    # max-abs tolerance on attention outputs
NEAR_TIE = 1e-5                      # bucket flips allowed only below this exact top-two gap


def ensure_library():
    from efficient_long_sequence_lsh_amd import _native

    if not os.path.exists(_native.LIB_PATH):
        from efficient_long_sequence_lsh_amd import build

        build.build()
    return _native


def to_device(inp):
    """Upload a workloads.Inputs to cuda:0 with the exact same bytes the oracle sees."""
    import torch

    if inp.qk_bits is not None:
        qk = torch.from_numpy(inp.qk_bits.view(np.int16)).view(torch.bfloat16).cuda()
        v = torch.from_numpy(inp.v_bits.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        qk = torch.from_numpy(np.ascontiguousarray(inp.qk)).cuda()
        v = torch.from_numpy(np.ascontiguousarray(inp.v)).cuda()
    rot = torch.from_numpy(np.ascontiguousarray(inp.rotations)).cuda()
    return qk, v, rot


def host(t):
    import torch

    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def compare_buckets(gpu, x, rotations, n_buckets, rows=None):
    """gpu: [B, H, r, L] ints.  Returns (n_flips, n_compared); asserts every flip is a near-tie."""
    B, H, r, L = gpu.shape
    flips, total = 0, 0
    for b in range(B):
        for h in range(H):
            sel = np.arange(L) if rows is None else np.asarray(rows)
            ob, om = oracle.lsh_hash(x[b, h][sel], rotations, n_buckets)
            g = gpu[b, h][:, sel]
            mism = g != ob
            bad = mism & (om >= NEAR_TIE)
            assert not bad.any(), (
                f"bucket mismatch at (b={b}, h={h}) rows {sel[np.nonzero(bad)[1]][:8]} "
                f"gpu {g[bad][:8]} oracle {ob[bad][:8]} margins {om[bad][:8]}")
            assert np.all((g >= 0) & (g < n_buckets))
            flips += int(mism.sum())
            total += mism.size
    return flips, total


def oracle_hash_all(x, rotations, n_buckets, rows_per_task=16384, threads=None):
    """oracle.lsh_hash on every row of x [B, H, L, d] (float64), in a thread pool.

    The hash is row-independent, so the rows are cut into slices and each
    slice is one call of the oracle; numpy releases the interpreter lock in
    the matrix product, the concatenation, argmax and partition, so threads
    scale.  BLAS itself is held to one thread per call.  Returns buckets and
    margins, both [B, H, r, L].
    """
    from concurrent.futures import ThreadPoolExecutor

    import threadpoolctl

    B, H, L, _ = x.shape
    r = 1 if n_buckets == 1 else rotations.shape[0]
    buckets = np.empty((B, H, r, L), np.int64)
    margin = np.empty((B, H, r, L), np.float64)
    tasks = [(b, h, a) for b in range(B) for h in range(H) for a in range(0, L, rows_per_task)]

    def run(t):
        b, h, a = t
        e = min(L, a + rows_per_task)
        ob, om = oracle.lsh_hash(x[b, h, a:e], rotations, n_buckets)
        buckets[b, h, :, a:e] = ob
        margin[b, h, :, a:e] = om

    n = threads or min(16, len(os.sched_getaffinity(0)))
    with threadpoolctl.threadpool_limits(1):
        with ThreadPoolExecutor(n) as ex:
            list(ex.map(run, tasks))
    return buckets, margin


def bucket_parity(gpu, want, margin):
    """Every id compared: returns (flips, near_ties, bad) where flips counts
    differing ids, near_ties the (position, round) pairs whose exact top-two
    gap is below NEAR_TIE, and bad the flips outside near-ties (must be 0)."""
    mism = gpu != want
    bad = mism & (margin >= NEAR_TIE)
    return int(mism.sum()), int((margin < NEAR_TIE).sum()), int(bad.sum())


def oracle_perm(buckets):
    """Stable sort of every (b, h, round) of the given bucket ids with the oracle."""
    B, H, r, L = buckets.shape
    perm = np.empty((B, H, r, L), np.int64)
    inv = np.empty((B, H, r, L), np.int64)
    for b in range(B):
        for h in range(H):
            perm[b, h], inv[b, h] = oracle.lsh_sort(buckets[b, h])
    return perm, inv
