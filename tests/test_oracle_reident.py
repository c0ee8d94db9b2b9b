"""Pins of the oracle's re-identifying attention step (reading R13: the cache
keeps totals; a step swaps the chosen keys' previous-step share for this step's
and rescores those keys).

Fixed outside the function itself:
  * with S held fixed it telescopes to the refresh-rest form (attn_rest +
    attn_sparse, pinned on their own against torch's attention);
  * with every key chosen at every step it is dense attention on each step's
    inputs: torch's scaled_dot_product_attention for o, and the refresh of that
    step shifted to the frozen row max for num and den;
  * on unchanged inputs it changes nothing, and the rescored keys get the
    refresh's scores back;
  * with no key chosen it returns the cached output;
  * swapping two disjoint halves of S in turn gives the same cache as swapping S
    at once (each key's share enters on its own);
  * with every key chosen, a block's new scores sum to sum_i den_new_i / den_old_i.
"""
import numpy as np
import torch

from oracle import attn_dense, attn_reident, attn_rest, attn_sparse, from_bf16_bits, identify_topk
from synthetic import heads_activations

SCALE = 1.0 / np.sqrt(128.0)
N = 300
BLOCKS = [(0, 128), (128, 256), (256, 300)]


def _qkv(step, n=N, seed=3):
    return [from_bf16_bits(heads_activations(seed, t, step, 1, n))[0] for t in "QKV"]


def _sdpa(q, k, v):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None],
        torch.from_numpy(v)[None, None], scale=SCALE)[0, 0].numpy()


def _refresh():
    q0, k0, v0 = _qkv(0)
    m, den, num, o, score = attn_dense(q0, k0, v0, SCALE)
    return (q0, k0, v0), m, den, num, o, score


def test_fixed_set_telescopes_to_rest_form():
    prev, m, den, num, o0, score = _refresh()
    idx = identify_topk(score.astype(np.float32), 70)
    nr, dr = attn_rest(*prev, m, idx, SCALE)
    for t in range(1, 4):
        cur = _qkv(t)
        o_rest = attn_sparse(*cur, m, nr, dr, idx, SCALE)
        o, num, den, score = attn_reident(*prev, *cur, m, num, den, score, idx, SCALE)
        np.testing.assert_allclose(o, o_rest, rtol=1e-10, atol=1e-12)
        prev = cur


def test_every_key_is_dense_attention_each_step():
    prev, m, den, num, o0, score = _refresh()
    every = np.tile(np.arange(N, dtype=np.int32), (3, 1))
    for t in range(1, 4):
        cur = _qkv(t)
        o, num, den, score = attn_reident(*prev, *cur, m, num, den, score, every, SCALE)
        np.testing.assert_allclose(o, _sdpa(*cur), rtol=1e-10, atol=1e-12)
        mt, dent, numt, _, _ = attn_dense(*cur, SCALE)
        shift = np.exp(mt - m)           # the same sums taken against the frozen max
        np.testing.assert_allclose(den, dent * shift, rtol=1e-10)
        np.testing.assert_allclose(num, numt * shift[:, None], rtol=1e-9, atol=1e-10)
        prev = cur


def test_unchanged_inputs_change_nothing():
    prev, m, den, num, o0, score = _refresh()
    idx = np.stack([np.sort(np.random.default_rng(b).choice(N, 90, replace=False)) for b in range(3)]).astype(np.int32)
    o, num1, den1, score1 = attn_reident(*prev, *prev, m, num, den, score, idx, SCALE)
    np.testing.assert_allclose(num1, num, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(den1, den, rtol=1e-13)
    np.testing.assert_allclose(o, o0, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(score1, score, rtol=1e-12, atol=1e-15)


def test_no_keys_returns_cached_output():
    prev, m, den, num, o0, score = _refresh()
    none = np.zeros((3, 0), np.int32)
    o, num1, den1, score1 = attn_reident(*prev, *_qkv(1), m, num, den, score, none, SCALE)
    np.testing.assert_array_equal(num1, num)
    np.testing.assert_array_equal(den1, den)
    np.testing.assert_array_equal(score1, score)
    np.testing.assert_allclose(o, o0, rtol=1e-14)


def test_disjoint_halves_in_turn_equal_the_whole_set():
    prev, m, den, num, o0, score = _refresh()
    cur = _qkv(1)
    g = np.random.default_rng(7)
    whole = np.stack([np.sort(g.choice(N, 100, replace=False)) for _ in range(3)]).astype(np.int32)
    a, b = whole[:, ::2], whole[:, 1::2]
    _, num_w, den_w, _ = attn_reident(*prev, *cur, m, num, den, score, whole, SCALE)
    _, num_a, den_a, score_a = attn_reident(*prev, *cur, m, num, den, score, a, SCALE)
    _, num_ab, den_ab, _ = attn_reident(*prev, *cur, m, num_a, den_a, score_a, b, SCALE)
    np.testing.assert_allclose(num_ab, num_w, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(den_ab, den_w, rtol=1e-12)


def test_every_key_scores_sum_to_denominator_ratio():
    prev, m, den, num, o0, score = _refresh()
    every = np.tile(np.arange(N, dtype=np.int32), (3, 1))
    cur = _qkv(1)
    _, _, den1, score1 = attn_reident(*prev, *cur, m, num, den, score, every, SCALE)
    for b, (r0, r1) in enumerate(BLOCKS):
        np.testing.assert_allclose(score1[b].sum(), (den1[r0:r1] / den[r0:r1]).sum(), rtol=1e-12)
    assert np.all(score1 >= 0)


def test_set_changes_when_mass_moves():
    # Rescored keys drop out when their mass falls below a kept key's score.
    prev, m, den, num, o0, score = _refresh()
    idx = identify_topk(score.astype(np.float32), 40)
    cur = _qkv(1)
    k1 = cur[1].copy()
    k1[idx[0][:10]] *= -1.0          # block 0's first ten chosen keys lose their mass
    _, _, _, score1 = attn_reident(*prev, cur[0], k1, cur[2], m, num, den, score, idx, SCALE)
    idx1 = identify_topk(score1.astype(np.float32), 40)
    assert not np.array_equal(idx1[0], idx[0])
    np.testing.assert_array_equal(np.delete(score1, idx[0], axis=1)[0], np.delete(score, idx[0], axis=1)[0])
