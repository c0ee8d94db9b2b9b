"""Pins of the oracle's step caching (reading R16: a cached step recomputes
nothing; its output is the latest computed output and every cache keeps its
value), against the already pinned dense and sparse steps:

  * a cached step returns exactly the previous output, any number in a row;
  * cached steps leave no trace: dense, cached..., sparse equals dense, sparse
    on the same inputs (MLP and attention);
  * for the MLP, a cached step is a sparse step with k = 0 (the S = empty set
    case, pinned separately as a bit identity);
  * the MLP invariant y = a W2 + b2 holds after every step of a mixed schedule;
  * a schedule must start with a dense step.
"""
import numpy as np
import pytest

import oracle
import synthetic as syn
from oracle import CACHED, DENSE, SPARSE


def _mlp(n=300, d=64, h=256, steps=5, seed=2):
    w1t, w2 = (oracle.from_bf16_bits(a) for a in syn.mlp_weights(seed, d, h))
    xs = [oracle.from_bf16_bits(syn.activations(seed, "X", t, n, d)) for t in range(steps)]
    g = np.random.default_rng(seed)
    b1, b2 = g.standard_normal(h) * 0.1, g.standard_normal(d) * 0.1
    return xs, w1t, b1, w2, b2


def test_mlp_cached_steps_return_the_previous_output():
    xs, w1t, b1, w2, b2 = _mlp()
    out = oracle.mlp_schedule(xs, w1t, b1, w2, b2, 64, [DENSE, SPARSE, CACHED, CACHED, SPARSE])
    assert np.array_equal(out[2], out[1]) and np.array_equal(out[3], out[1])
    assert not np.array_equal(out[4], out[3])


def test_mlp_cached_steps_leave_no_trace():
    xs, w1t, b1, w2, b2 = _mlp()
    a = oracle.mlp_schedule(xs, w1t, b1, w2, b2, 64, [DENSE, CACHED, CACHED, SPARSE])
    b = oracle.mlp_schedule([xs[0], xs[3]], w1t, b1, w2, b2, 64, [DENSE, SPARSE])
    assert np.array_equal(a[3], b[1])


def test_mlp_cached_step_is_the_empty_set_delta():
    xs, w1t, b1, w2, b2 = _mlp()
    h = w1t.shape[0]
    a0, y0, _ = oracle.mlp_dense(xs[0], w1t, b1, w2, b2, np.zeros((xs[0].shape[0], h)))
    nb = (xs[0].shape[0] + 127) // 128
    a1, y1 = oracle.mlp_sparse(xs[1], w1t, b1, w2, a0, y0, np.zeros((nb, 0), np.int32))
    out = oracle.mlp_schedule(xs, w1t, b1, w2, b2, 64, [DENSE, CACHED])
    assert np.array_equal(out[1], y1) and np.array_equal(a1, a0)


def test_mlp_invariant_holds_through_a_mixed_schedule():
    xs, w1t, b1, w2, b2 = _mlp(steps=6)
    sched = [DENSE, SPARSE, CACHED, SPARSE, DENSE, CACHED]
    out = oracle.mlp_schedule(xs, w1t, b1, w2, b2, 64, sched)
    # rebuild the activation cache by replaying the computed steps
    n, h = xs[0].shape[0], w1t.shape[0]
    a = np.zeros((n, h))
    score = None
    for t, kind in enumerate(sched):
        if kind == DENSE:
            a, _, score = oracle.mlp_dense(xs[t], w1t, b1, w2, b2, a)
        elif kind == SPARSE:
            idx = oracle.identify_topk(score.astype(np.float32), 64)
            a, _ = oracle.mlp_sparse(xs[t], w1t, b1, w2, a, out[t - 1] if t else None, idx)
        np.testing.assert_allclose(out[t], a @ w2 + b2, rtol=1e-10, atol=1e-10)


def _attn(n=300, heads=1, steps=4, seed=3):
    walks = [[oracle.from_bf16_bits(syn.heads_activations(seed, tag, t, heads, n)[0]) for t in range(steps)]
             for tag in "QKV"]
    return walks


def test_attention_cached_steps_return_the_previous_output_and_leave_no_trace():
    qs, ks, vs = _attn()
    sc = 1.0 / np.sqrt(128.0)
    a = oracle.attn_schedule(qs, ks, vs, sc, 50, [DENSE, SPARSE, CACHED, SPARSE])
    assert np.array_equal(a[2], a[1])
    b = oracle.attn_schedule([qs[0], qs[3]], [ks[0], ks[3]], [vs[0], vs[3]], sc, 50, [DENSE, SPARSE])
    assert np.array_equal(a[3], b[1])
    c = oracle.attn_schedule(qs, ks, vs, sc, 50, [DENSE, CACHED, CACHED, CACHED])
    assert all(np.array_equal(c[t], c[0]) for t in range(4))
    # a cached attention step is not a sparse step with no keys: that one
    # returns the rest state alone (num_rest / den_rest)
    m, _, _, o0, score = oracle.attn_dense(qs[0], ks[0], vs[0], sc)
    idx = oracle.identify_topk(score.astype(np.float32), 50)
    nr, dr = oracle.attn_rest(qs[0], ks[0], vs[0], m, idx, sc)
    assert not np.allclose(nr / dr[:, None], o0)


def test_schedule_needs_a_dense_step_first():
    xs, w1t, b1, w2, b2 = _mlp(steps=2)
    with pytest.raises(ValueError):
        oracle.mlp_schedule(xs, w1t, b1, w2, b2, 64, [CACHED, DENSE])
    qs, ks, vs = _attn(steps=2)
    with pytest.raises(ValueError):
        oracle.attn_schedule(qs, ks, vs, 0.1, 10, [SPARSE, DENSE])
