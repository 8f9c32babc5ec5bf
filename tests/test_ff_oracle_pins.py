"""Pins for the feed-forward oracle: chunking is exact, the layer against a
written-out two-layer perceptron on a tiny input, and closed forms."""
import numpy as np
import pytest

import oracle


def _params(d, f, seed):
    g = np.random.default_rng(seed)
    return g.standard_normal((f, d)), g.standard_normal(f), g.standard_normal((d, f)), g.standard_normal(d)


@pytest.mark.parametrize("chunk", [1, 3, 16, 100])
def test_chunked_equals_whole_exactly(chunk):
    w1, b1, w2, b2 = _params(8, 24, 1)
    x = np.random.default_rng(2).standard_normal((37, 8))
    np.testing.assert_array_equal(oracle.chunked_feed_forward(x, w1, b1, w2, b2, chunk),
                                  oracle.feed_forward(x, w1, b1, w2, b2))


def test_tiny_case_written_out():
    x = np.array([[1.0, -2.0]])
    w1 = np.array([[1.0, 1.0], [2.0, 0.0], [0.0, -1.0]])   # h_pre = [-1, 2, 2] + b1
    b1 = np.array([0.5, -1.0, 0.0])                         # h = relu([-0.5, 1, 2]) = [0, 1, 2]
    w2 = np.array([[1.0, 2.0, 3.0], [-1.0, 0.0, 1.0]])      # y = [0+2+6, 0+0+2] + b2
    b2 = np.array([0.25, -0.25])
    np.testing.assert_array_equal(oracle.feed_forward(x, w1, b1, w2, b2), [[8.25, 1.75]])


def test_closed_forms():
    w1, b1, w2, b2 = _params(6, 10, 3)
    x = np.random.default_rng(4).standard_normal((5, 6))
    # zero second layer: output is the second bias on every row
    np.testing.assert_array_equal(oracle.feed_forward(x, w1, b1, np.zeros_like(w2), b2), np.tile(b2, (5, 1)))
    # hidden units that are never positive contribute nothing
    out = oracle.feed_forward(x, np.zeros_like(w1), -np.ones(10), w2, b2)
    np.testing.assert_array_equal(out, np.tile(b2, (5, 1)))
    # identity first layer with d_ff = d and non-negative input: y = (x + b1) W2^T + b2 where x + b1 >= 0
    xp = np.abs(x)
    eye = np.eye(6)
    np.testing.assert_allclose(oracle.feed_forward(xp, eye, np.zeros(6), w2[:, :6], b2), xp @ w2[:, :6].T + b2,
                               rtol=0, atol=1e-12)
