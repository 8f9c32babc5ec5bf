"""Pins for the local-attention oracle against facts that do not come from
the oracle itself: window hand examples, a library routine (scaled
dot-product attention) where the window covers everything or is one chunk,
the closed form for windows of one position, a pure-Python brute force, and
locality / causality invariants."""
import math

import numpy as np
import pytest
import torch

import oracle


def _data(L, d, seed):
    g = np.random.default_rng(seed)
    return (g.standard_normal((L, d)), g.standard_normal((L, d)), g.standard_normal((L, d)))


def test_window_hand_examples():
    # L = 16, chunks of 4: position 5 is in chunk 1 (positions 4..7).
    assert list(oracle.local_window(5, 16, 4, 0, 0, False)) == [4, 5, 6, 7]
    assert list(oracle.local_window(5, 16, 4, 1, 0, False)) == list(range(0, 8))
    assert list(oracle.local_window(5, 16, 4, 1, 1, False)) == list(range(0, 12))
    assert list(oracle.local_window(5, 16, 4, 1, 1, True)) == list(range(0, 6))
    assert list(oracle.local_window(0, 16, 4, 3, 0, False)) == [0, 1, 2, 3]          # no wrap-around
    assert list(oracle.local_window(15, 16, 4, 0, 5, False)) == [12, 13, 14, 15]
    assert list(oracle.local_window(3, 16, 100, 0, 0, False)) == list(range(16))      # chunk >= L: one chunk
    with pytest.raises(ValueError):
        oracle.local_window(0, 10, 4, 0, 0, False)


@pytest.mark.parametrize("causal", [False, True])
def test_window_covering_everything_is_full_attention(causal):
    q, k, v = _data(48, 16, 1)
    out = oracle.local_attention_head(q, k, v, 8, 10, 10, causal)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None], is_causal=causal)[0].numpy()
    np.testing.assert_allclose(out, want, rtol=0, atol=1e-12)


def test_zero_overlap_is_attention_inside_each_chunk():
    q, k, v = _data(40, 8, 2)
    out = oracle.local_attention_head(q, k, v, 10, 0, 0, False)
    for c in range(4):
        sl = slice(10 * c, 10 * c + 10)
        want = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[sl])[None], torch.from_numpy(k[sl])[None], torch.from_numpy(v[sl])[None])[0].numpy()
        np.testing.assert_allclose(out[sl], want, rtol=0, atol=1e-12)


def test_windows_of_one_position_return_v():
    q, k, v = _data(12, 8, 3)
    np.testing.assert_array_equal(oracle.local_attention_head(q, k, v, 1, 0, 0, False), v)
    # causal with no look-back leaves position 0 of each chunk alone with itself
    out = oracle.local_attention_head(q, k, v, 4, 0, 2, True)
    np.testing.assert_allclose(out[[0, 4, 8]], v[[0, 4, 8]], rtol=0, atol=0)


@pytest.mark.parametrize("L,m,nb,na,causal", [(12, 4, 1, 0, True), (12, 3, 1, 1, False), (10, 5, 0, 1, True),
                                             (8, 2, 2, 1, False)])
def test_pure_python_brute_force(L, m, nb, na, causal):
    q, k, v = _data(L, 4, 10 + L + m)
    out = oracle.local_attention_head(q, k, v, m, nb, na, causal)
    for i in range(L):
        c = i // m
        keys = [j for j in range(L) if c - nb <= j // m <= c + na and (not causal or j <= i)]
        s = [sum(q[i][t] * k[j][t] for t in range(4)) / 2.0 for j in keys]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        tot = math.fsum(w)
        for t in range(4):
            assert abs(out[i][t] - math.fsum(w[a] * v[j][t] for a, j in enumerate(keys)) / tot) < 1e-12


def test_outside_the_window_does_not_matter():
    q, k, v = _data(32, 8, 4)
    base = oracle.local_attention_head(q, k, v, 8, 1, 0, False)
    k2, v2 = k.copy(), v.copy()
    k2[24:] += 5.0           # chunk 3 is outside the windows of chunks 0 and 1
    v2[24:] -= 7.0
    out = oracle.local_attention_head(q, k2, v2, 8, 1, 0, False)
    np.testing.assert_array_equal(out[:16], base[:16])
    assert np.abs(out[24:] - base[24:]).max() > 1e-3


def test_causal_outputs_ignore_later_positions():
    q, k, v = _data(30, 8, 5)
    base = oracle.local_attention_head(q, k, v, 6, 2, 2, True)
    k2, v2 = k.copy(), v.copy()
    k2[17:] = 0.0
    v2[17:] = 3.0
    out = oracle.local_attention_head(q, k2, v2, 6, 2, 2, True)
    np.testing.assert_array_equal(out[:17], base[:17])
