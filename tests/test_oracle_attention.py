"""Pins of the oracle's attention over the selected tokens (textbook softmax attention
with grouped-query heads)."""

import math

import numpy as np

from oracle.attention import sparse_attention


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_single_token_returns_its_value():
    rng = np.random.default_rng(0)
    q, k, v = _rand(rng, 8, 16), _rand(rng, 1, 2, 16), _rand(rng, 1, 2, 16)
    out = sparse_attention(q, k, v, 0.25)
    for h in range(8):
        assert np.array_equal(out[h], v[0, h // 4])


def test_identical_keys_average_the_values():
    rng = np.random.default_rng(1)
    key = _rand(rng, 1, 2, 16)
    k = np.repeat(key, 7, axis=0)
    v = _rand(rng, 7, 2, 16)
    out = sparse_attention(_rand(rng, 4, 16), k, v, 1.0)
    for h in range(4):
        assert np.allclose(out[h], v[:, h // 2].mean(axis=0), rtol=0, atol=1e-14)


def test_two_tokens_closed_form():
    rng = np.random.default_rng(2)
    q, k, v = _rand(rng, 2, 8), _rand(rng, 2, 1, 8), _rand(rng, 2, 1, 8)
    scale = 1.0 / math.sqrt(8)
    out = sparse_attention(q, k, v, scale)
    for h in range(2):
        d = scale * float(q[h] @ (k[0, 0] - k[1, 0]))
        w0 = 1.0 / (1.0 + math.exp(-d))  # logistic of the score difference
        assert np.allclose(out[h], w0 * v[0, 0] + (1.0 - w0) * v[1, 0], rtol=0, atol=1e-14)


def test_permutation_invariance_and_dominance():
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 4, 32), _rand(rng, 50, 4, 32), _rand(rng, 50, 4, 32)
    perm = rng.permutation(50)
    a = sparse_attention(q, k, v, 0.2)
    b = sparse_attention(q, k[perm], v[perm], 0.2)
    assert np.allclose(a, b, rtol=0, atol=1e-13)
    # a key parallel to the query with a score 60 above the others takes all the weight
    k2 = k.copy()
    k2[17, 0] = q[0] * (60.0 / (0.2 * float(q[0] @ q[0]))) + 0.0
    s = 0.2 * (k2[:, 0] @ q[0])
    assert s[17] - np.delete(s, 17).max() > 40
    out = sparse_attention(q[:1], k2[:, :1], v[:, :1], 0.2)
    assert np.allclose(out[0], v[17, 0], rtol=0, atol=1e-12)


def test_grouped_heads_read_their_own_kv_head():
    rng = np.random.default_rng(4)
    q, k, v = _rand(rng, 8, 16), _rand(rng, 20, 4, 16), _rand(rng, 20, 4, 16)
    base = sparse_attention(q, k, v, 0.3)
    v2 = v.copy()
    v2[:, 1] += 5.0
    moved = sparse_attention(q, k, v2, 0.3)
    changed = np.any(base != moved, axis=1)
    assert changed.tolist() == [False, False, True, True, False, False, False, False]
    # with as many query heads as KV heads each head is plain attention over its own head
    one = sparse_attention(q[:4], k, v, 0.3)
    for h in range(4):
        alone = sparse_attention(q[h:h + 1], k[:, h:h + 1], v[:, h:h + 1], 0.3)
        assert np.array_equal(one[h], alone[0])


def test_empty_selection_gives_zeros():
    out = sparse_attention(np.ones((4, 8)), np.zeros((0, 2, 8)), np.zeros((0, 2, 8)), 1.0)
    assert out.shape == (4, 8) and not out.any()
