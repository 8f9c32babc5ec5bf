"""Chunked feed-forward on the GPU: against the float64 oracle, and bit-equal
results for every chunk size (chunking must not change any result)."""
import numpy as np
import pytest

import oracle
from efficient_long_sequence_lsh_amd import workloads as W
from gpu_util import ensure_library, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nat():
    return ensure_library()


def _bf16(a):
    import torch

    bits = W.f32_to_bf16_bits(a.astype(np.float32))
    return W.bf16_bits_to_f32(bits), torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def _params(n, d, f, seed):
    import torch

    g = np.random.default_rng(seed)
    x, xd = _bf16(g.standard_normal((n, d)))
    w1, w1d = _bf16(g.standard_normal((f, d)) / np.sqrt(d))
    w2, w2d = _bf16(g.standard_normal((d, f)) / np.sqrt(f))
    b1 = (0.1 * g.standard_normal(f)).astype(np.float32)
    b2 = (0.1 * g.standard_normal(d)).astype(np.float32)
    return (x, w1, b1, w2, b2), (xd, w1d, torch.from_numpy(b1).cuda(), w2d, torch.from_numpy(b2).cuda())


@pytest.mark.parametrize("n,d,f,chunk", [(300, 128, 256, 0), (1024, 256, 512, 128), (1000, 128, 384, 333),
                                         (600, 512, 1024, 0)])   # several 256-wide tiles, ragged rows
def test_feed_forward_matches_oracle(nat, n, d, f, chunk):
    h, dev = _params(n, d, f, n + d + f)
    out = host(nat.feed_forward(*dev, chunk_tokens=chunk))
    want = oracle.feed_forward(*h)
    scale = max(1.0, float(np.abs(want).max()))
    err = float(np.abs(out - want).max())
    print(f"[ff] n{n} d{d} f{f} chunk{chunk}: max abs err {err:.3e} (scale {scale:.2f})", flush=True)
    assert err <= 1e-2 * scale


def test_chunking_changes_no_bit(nat):
    import torch

    _, dev = _params(1000, 256, 512, 5)
    whole = nat.feed_forward(*dev, chunk_tokens=0)
    for chunk in (1, 7, 64, 129, 999, 1000, 5000):
        assert torch.equal(nat.feed_forward(*dev, chunk_tokens=chunk).view(torch.int16), whole.view(torch.int16)), chunk



def test_feed_forward_full_size(nat):
    """The layer as `bench.py --ff` times it (65536 positions, d_model 1024,
    d_ff 4096, chunks of 8192): the oracle works one position at a time, so
    sampled rows (including the first and last of a chunk) are checked."""
    n, d, f = 65536, 1024, 4096
    h, dev = _params(n, d, f, 2020)
    out = nat.feed_forward(*dev, chunk_tokens=8192)
    rows = np.unique(np.concatenate([[0, 8191, 8192, n - 1], np.random.default_rng(1).integers(0, n, 60)]))
    x, w1, b1, w2, b2 = h
    want = oracle.feed_forward(x[rows], w1, b1, w2, b2)
    got = host(out)[rows]
    scale = max(1.0, float(np.abs(want).max()))
    err = float(np.abs(got - want).max())
    print(f"[ff-full] n{n} d{d} f{f}: max abs err on {rows.size} rows {err:.3e} (scale {scale:.2f})", flush=True)
    assert err <= 1e-2 * scale
