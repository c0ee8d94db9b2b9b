"""Pins of the oracle's attention refresh and sparse delta step.

Fixed outside the oracle: torch's scaled_dot_product_attention (the textbook
softmax(Q K^T) V the Chipmunk post writes), the delta reformulation's special
cases (all keys = dense step on the new inputs; no keys = the cached output),
softmax shift invariance (the frozen row max cancels), and closed forms (a
constant V row is reproduced exactly; key-mass scores of a block sum to its row
count)."""
import numpy as np
import torch

from oracle import attn_dense, attn_rest, attn_sparse, from_bf16_bits, identify_topk, rel_frobenius
from synthetic import heads_activations

SCALE = 1.0 / np.sqrt(128.0)


def _qkv(step, n=300, seed=0):
    return [from_bf16_bits(heads_activations(seed, t, step, 1, n))[0] for t in "QKV"]


def _sdpa(q, k, v):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None],
        torch.from_numpy(v)[None, None], scale=SCALE)[0, 0].numpy()


def test_dense_matches_sdpa_and_scores_sum_to_rows():
    q, k, v = _qkv(0)
    m, den, num, o, score = attn_dense(q, k, v, SCALE)
    np.testing.assert_allclose(o, _sdpa(q, k, v), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(m, (q @ k.T).max(axis=1) * SCALE, rtol=1e-14)
    assert score.shape == (3, 300)
    np.testing.assert_allclose(score.sum(axis=1), [128, 128, 44], rtol=1e-12)
    assert np.all(score >= 0)


def test_rest_plus_chosen_is_full_cache():
    q, k, v = _qkv(0)
    m, den, num, o, score = attn_dense(q, k, v, SCALE)
    idx = identify_topk(score.astype(np.float32), 50)
    num_rest, den_rest = attn_rest(q, k, v, m, idx, SCALE)
    for b, (r0, r1) in enumerate([(0, 128), (128, 256), (256, 300)]):
        s = idx[b]
        p = np.exp(SCALE * q[r0:r1] @ k[s].T - m[r0:r1, None])
        np.testing.assert_allclose(num_rest[r0:r1] + p @ v[s], num[r0:r1], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(den_rest[r0:r1] + p.sum(1), den[r0:r1], rtol=1e-13)


def test_sparse_all_keys_is_dense_on_new_inputs_and_max_cancels():
    q0, k0, v0 = _qkv(0)
    q1, k1, v1 = _qkv(1)
    m, den, num, o, score = attn_dense(q0, k0, v0, SCALE)
    every = np.tile(np.arange(300, dtype=np.int32), (3, 1))
    num_rest, den_rest = attn_rest(q0, k0, v0, m, every, SCALE)
    assert np.all(num_rest == 0) and np.all(den_rest == 0)
    o1 = attn_sparse(q1, k1, v1, m, num_rest, den_rest, every, SCALE)
    np.testing.assert_allclose(o1, _sdpa(q1, k1, v1), rtol=1e-11, atol=1e-12)
    o1b = attn_sparse(q1, k1, v1, m + 1.0, num_rest, den_rest, every, SCALE)
    np.testing.assert_allclose(o1b, o1, rtol=1e-12, atol=1e-13)


def test_sparse_no_keys_returns_refresh_output():
    q0, k0, v0 = _qkv(0)
    q1, k1, v1 = _qkv(1)
    m, den, num, o, _ = attn_dense(q0, k0, v0, SCALE)
    none = np.zeros((3, 0), np.int32)
    num_rest, den_rest = attn_rest(q0, k0, v0, m, none, SCALE)
    o1 = attn_sparse(q1, k1, v1, m, num_rest, den_rest, none, SCALE)
    np.testing.assert_allclose(o1, o, rtol=1e-13, atol=1e-14)


def test_constant_values_and_linearity_in_v():
    q0, k0, v0 = _qkv(0)
    q1, k1, v1 = _qkv(1)
    c = np.linspace(-1, 1, 128)
    vc = np.tile(c, (300, 1))
    m, den, num, o, score = attn_dense(q0, k0, vc, SCALE)
    np.testing.assert_allclose(o, np.tile(c, (300, 1)), rtol=1e-13, atol=1e-14)
    idx = identify_topk(score.astype(np.float32), 60)
    nr, dr = attn_rest(q0, k0, vc, m, idx, SCALE)
    o1 = attn_sparse(q1, k1, vc, m, nr, dr, idx, SCALE)
    np.testing.assert_allclose(o1, np.tile(c, (300, 1)), rtol=1e-12, atol=1e-13)
    # the output is linear in V when the cached part scales with it
    nr1, dr1 = attn_rest(q0, k0, v0, m, idx, SCALE)
    oa = attn_sparse(q1, k1, v1, m, nr1, dr1, idx, SCALE)
    ob = attn_sparse(q1, k1, 2.0 * v1, m, 2.0 * nr1, dr1, idx, SCALE)
    np.testing.assert_array_equal(ob, 2.0 * oa)


def test_sparse_close_to_dense_informational():
    q0, k0, v0 = _qkv(0)
    q1, k1, v1 = _qkv(1)
    m, den, num, o, score = attn_dense(q0, k0, v0, SCALE)
    idx = identify_topk(score.astype(np.float32), 100)
    nr, dr = attn_rest(q0, k0, v0, m, idx, SCALE)
    o1 = attn_sparse(q1, k1, v1, m, nr, dr, idx, SCALE)
    assert rel_frobenius(o1, _sdpa(q1, k1, v1)) < 0.2
