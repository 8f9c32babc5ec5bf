"""Pins for the gradient oracle: its dense multiset forward equals the
round-by-round oracle, and its autograd gradients equal central finite
differences of the round-by-round forward (buckets held fixed)."""
import numpy as np
import pytest
import torch

import oracle


def _case(L, d, r, nb, seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal((L, d))
    v = g.standard_normal((L, d))
    rot = g.standard_normal((r, d, nb // 2)).astype(np.float32)
    buckets, _ = oracle.lsh_hash(x, rot, nb)
    perm, _ = oracle.lsh_sort(buckets)
    return x, v, perm


@pytest.mark.parametrize("L,d,r,nb,m,causal", [(32, 8, 2, 4, 8, False), (32, 8, 3, 4, 4, True),
                                               (24, 4, 1, 2, 24, True), (16, 4, 2, 8, 1, False)])
def test_dense_multiset_form_equals_round_by_round(L, d, r, nb, m, causal):
    x, v, perm = _case(L, d, r, nb, L + r + m)
    want = oracle.lsh_attention_head(x, v, None, nb, m, causal, perm=perm)["out"]
    M = oracle.target_counts(perm, m, causal)
    got = oracle.dense_forward(torch.from_numpy(x), torch.from_numpy(v), M).numpy()
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_target_counts_hand_example():
    # L = 4, one round, identity order, chunks of 2, causal: query 1 sees 0;
    # query 2 (chunk 1) sees chunk 0 and 1 before it: 0, 1; query 3 sees 0, 1, 2.
    M = oracle.target_counts(np.array([[0, 1, 2, 3]]), 2, True)
    want = np.array([[0, 0, 0, 0], [1, 0, 0, 0], [1, 1, 0, 0], [1, 1, 1, 0]])
    np.testing.assert_array_equal(M, want)
    # two identical rounds double every count
    np.testing.assert_array_equal(oracle.target_counts(np.array([[0, 1, 2, 3]] * 2), 2, True), 2 * want)


@pytest.mark.parametrize("L,d,r,nb,m,causal", [(16, 4, 2, 4, 4, True), (12, 3, 2, 2, 6, False)])
def test_gradients_equal_finite_differences(L, d, r, nb, m, causal):
    x, v, perm = _case(L, d, r, nb, 7 * L + d)
    g = np.random.default_rng(3)
    dout = g.standard_normal((L, d))
    _, dx, dv = oracle.lsh_attention_head_grad(x, v, perm, m, causal, dout)

    def loss(xx, vv):
        return float((oracle.lsh_attention_head(xx, vv, None, nb, m, causal, perm=perm)["out"] * dout).sum())

    h = 1e-6
    for (i, k) in [(0, 0), (3, 1), (L - 1, d - 1), (L // 2, 2)]:
        xp, xm = x.copy(), x.copy()
        xp[i, k] += h
        xm[i, k] -= h
        assert abs((loss(xp, v) - loss(xm, v)) / (2 * h) - dx[i, k]) < 1e-6
        vp, vm = v.copy(), v.copy()
        vp[i, k] += h
        vm[i, k] -= h
        assert abs((loss(x, vp) - loss(x, vm)) / (2 * h) - dv[i, k]) < 1e-6


def test_self_fallback_rows_pass_the_gradient_to_v():
    # causal, one round, identity order: position 0 has no target, so out_0 = v_0
    x = np.random.default_rng(1).standard_normal((8, 4))
    v = np.random.default_rng(2).standard_normal((8, 4))
    dout = np.zeros((8, 4))
    dout[0] = [1.0, 2.0, 3.0, 4.0]
    _, dx, dv = oracle.lsh_attention_head_grad(x, v, np.arange(8)[None], 4, True, dout)
    np.testing.assert_array_equal(dv[0], dout[0])
    np.testing.assert_array_equal(dv[1:], 0.0)
    np.testing.assert_array_equal(dx, 0.0)


@pytest.mark.parametrize("L,d,r,nb,m,causal", [(32, 8, 2, 4, 8, False), (32, 8, 3, 4, 4, True),
                                               (24, 4, 1, 2, 24, True), (16, 4, 2, 8, 1, False),
                                               (64, 6, 4, 8, 8, True)])
def test_sampled_gradients_equal_autograd(L, d, r, nb, m, causal):
    """The per-position gradient (softmax derivative written out, observers
    found from the chunk structure) equals autograd of the dense form at every
    position, including self-fallback rows and keys seen in several rounds."""
    x, v, perm = _case(L, d, r, nb, 5 * L + r)
    dout = np.random.default_rng(L).standard_normal((L, d))
    _, wx, wv = oracle.lsh_attention_head_grad(x, v, perm, m, causal, dout)
    pos = np.random.default_rng(r).permutation(L)
    gx, gv = oracle.grad_positions(x, v, perm, pos, m, causal, dout)
    np.testing.assert_allclose(gx, wx[pos], rtol=0, atol=1e-12)
    np.testing.assert_allclose(gv, wv[pos], rtol=0, atol=1e-12)


def test_sampled_gradients_equal_finite_differences():
    L, d, r, nb, m, causal = 16, 4, 2, 4, 4, True
    x, v, perm = _case(L, d, r, nb, 99)
    dout = np.random.default_rng(4).standard_normal((L, d))

    def loss(xx, vv):
        return float((oracle.lsh_attention_head(xx, vv, None, nb, m, causal, perm=perm)["out"] * dout).sum())

    pos = [0, 5, L - 1]
    gx, gv = oracle.grad_positions(x, v, perm, pos, m, causal, dout)
    h = 1e-6
    for n, i in enumerate(pos):
        for k in range(d):
            xp, xm = x.copy(), x.copy()
            xp[i, k] += h
            xm[i, k] -= h
            assert abs((loss(xp, v) - loss(xm, v)) / (2 * h) - gx[n, k]) < 1e-6
            vp, vm = v.copy(), v.copy()
            vp[i, k] += h
            vm[i, k] -= h
            assert abs((loss(x, vp) - loss(x, vm)) / (2 * h) - gv[n, k]) < 1e-6
