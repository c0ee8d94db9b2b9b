"""Pins of the oracle's MLP dense refresh and sparse delta step.

What fixes the answers here, independent of the oracle's own code:
* torch.nn.functional (linear + tanh GELU) for the dense forward pass;
* the delta reformulation in the Chipmunk post (Activation Deltas section): with
  S = all columns a sparse step IS the dense step on the new input, with S empty
  it changes nothing;
* the linear-combination view (same section): the output is always the cached
  coefficients times the rows of W2 plus a bias, which cancels from the delta;
* explicit loops on tiny inputs for the per-block L1 score.
"""
import numpy as np
import pytest
import torch

from oracle import bf16_round, from_bf16_bits, identify_topk, mlp_dense, mlp_sparse, rel_frobenius
from synthetic import activations, mlp_weights


def _setup(n=300, d=64, h=192, seed=0, bias=True):
    w1t_b, w2_b = mlp_weights(seed, d, h)
    w1t, w2 = from_bf16_bits(w1t_b), from_bf16_bits(w2_b)
    g = np.random.default_rng(seed)
    b1 = g.standard_normal(h).astype(np.float32).astype(np.float64) * 0.1 if bias else None
    b2 = g.standard_normal(d).astype(np.float32).astype(np.float64) * 0.1 if bias else None
    xs = [from_bf16_bits(activations(seed, "X", t, n, d)) for t in range(4)]
    return xs, w1t, b1, w2, b2


def test_dense_matches_torch_functional():
    xs, w1t, b1, w2, b2 = _setup()
    a_new, y, _ = mlp_dense(xs[0], w1t, b1, w2, b2, np.zeros((300, 192)))
    xt = torch.from_numpy(xs[0])
    z = torch.nn.functional.linear(xt, torch.from_numpy(w1t), torch.from_numpy(b1))
    a = torch.nn.functional.gelu(z, approximate="tanh").numpy()
    a = torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).to(torch.float64)
    # The bf16 rounding of fp32(gelu) and of fp64(gelu) can differ only on the
    # rare values whose fp64 sits within an fp32 ulp of a bf16 tie.
    mism = np.mean(a.numpy() != a_new)
    assert mism < 1e-3
    yt = torch.nn.functional.linear(torch.from_numpy(a_new), torch.from_numpy(w2).T.contiguous(),
                                    torch.from_numpy(b2)).numpy()
    np.testing.assert_allclose(y, yt, rtol=1e-12, atol=1e-12)


def test_score_brute_force_ragged_block():
    n, d, h = 130, 8, 5                          # blocks of 128 and 2 rows
    xs, w1t, b1, w2, b2 = _setup(n, d, h, seed=2)
    a_old = bf16_round(np.random.default_rng(1).standard_normal((n, h)))
    a_new, _, score = mlp_dense(xs[0], w1t, b1, w2, b2, a_old)
    assert score.shape == (2, h)
    for b, (r0, r1) in enumerate([(0, 128), (128, 130)]):
        for j in range(h):
            s = 0.0
            for i in range(r0, r1):
                s += abs(a_new[i, j] - a_old[i, j])
            assert abs(score[b, j] - s) <= 1e-12 * max(1.0, s)


def test_sparse_all_columns_equals_dense():
    xs, w1t, b1, w2, b2 = _setup()
    a0, y0, _ = mlp_dense(xs[0], w1t, b1, w2, b2, np.zeros((300, 192)))
    every = np.tile(np.arange(192, dtype=np.int32), (3, 1))
    a1, y1 = mlp_sparse(xs[1], w1t, b1, w2, a0, y0, every)
    a1d, y1d, _ = mlp_dense(xs[1], w1t, b1, w2, b2, a0)
    np.testing.assert_array_equal(a1, a1d)
    assert rel_frobenius(y1, y1d) < 1e-13


def test_sparse_empty_set_is_identity():
    xs, w1t, b1, w2, b2 = _setup()
    a0, y0, _ = mlp_dense(xs[0], w1t, b1, w2, b2, np.zeros((300, 192)))
    a1, y1 = mlp_sparse(xs[1], w1t, b1, w2, a0, y0, np.zeros((3, 0), np.int32))
    np.testing.assert_array_equal(a1, a0)
    np.testing.assert_array_equal(y1, y0)


def test_output_stays_coefficients_times_w2():
    # Y = A W2 + b2 after every step, whatever subsets were recomputed.
    xs, w1t, b1, w2, b2 = _setup()
    a, y, score = mlp_dense(xs[0], w1t, b1, w2, b2, np.zeros((300, 192)))
    for t in range(1, 4):
        k = [10, 77, 192][t - 1]
        idx = identify_topk(score.astype(np.float32), k)
        a, y = mlp_sparse(xs[t], w1t, b1, w2, a, y, idx)
        np.testing.assert_allclose(y, a @ w2 + b2[None, :], rtol=1e-11, atol=1e-11)


def test_only_chosen_columns_change():
    xs, w1t, b1, w2, b2 = _setup()
    a0, y0, score = mlp_dense(xs[0], w1t, b1, w2, b2, np.zeros((300, 192)))
    idx = identify_topk(score.astype(np.float32), 50)
    a1, _ = mlp_sparse(xs[1], w1t, b1, w2, a0, y0, idx)
    for b, (r0, r1) in enumerate([(0, 128), (128, 256), (256, 300)]):
        mask = np.ones(192, bool)
        mask[idx[b]] = False
        np.testing.assert_array_equal(a1[r0:r1][:, mask], a0[r0:r1][:, mask])
        fresh, _, _ = mlp_dense(xs[1][r0:r1], w1t, b1, w2, b2, a0[r0:r1])
        np.testing.assert_array_equal(a1[r0:r1][:, idx[b]], fresh[:, idx[b]])


def test_telescoping_fixed_set():
    # With S fixed, steps telescope: Y_T = Y_0 + (A_T - A_0)[:, S] W2[S].
    xs, w1t, b1, w2, b2 = _setup()
    a0, y0, score = mlp_dense(xs[0], w1t, b1, w2, b2, np.zeros((300, 192)))
    idx = identify_topk(score.astype(np.float32), 40)
    a, y = a0, y0
    for t in range(1, 4):
        a, y = mlp_sparse(xs[t], w1t, b1, w2, a, y, idx)
    for b, (r0, r1) in enumerate([(0, 128), (128, 256), (256, 300)]):
        s = idx[b]
        expect = y0[r0:r1] + (a[r0:r1][:, s] - a0[r0:r1][:, s]) @ w2[s]
        np.testing.assert_allclose(y[r0:r1], expect, rtol=1e-12, atol=1e-12)


def test_delta_linear_in_w2_and_bias_cancels():
    xs, w1t, b1, w2, b2 = _setup()
    a0, y0, score = mlp_dense(xs[0], w1t, b1, w2, b2, np.zeros((300, 192)))
    idx = identify_topk(score.astype(np.float32), 64)
    _, y1 = mlp_sparse(xs[1], w1t, b1, w2, a0, y0, idx)
    # the delta alone (zero output cache) scales exactly with a power-of-two W2
    zero = np.zeros_like(y0)
    _, dy = mlp_sparse(xs[1], w1t, b1, w2, a0, zero, idx)
    _, dy2 = mlp_sparse(xs[1], w1t, b1, 2.0 * w2, a0, zero, idx)
    np.testing.assert_array_equal(dy2, 2.0 * dy)
    np.testing.assert_allclose(y1 - y0, dy, rtol=1e-12, atol=1e-14)
    # the static bias b2 is one extra vector that every step shares: it cancels
    _, y_nb = mlp_sparse(xs[1], w1t, b1, w2, a0, y0 - b2[None, :], idx)
    np.testing.assert_allclose((y1 - y0), (y_nb - (y0 - b2[None, :])), rtol=1e-12, atol=1e-14)


def test_partial_last_block_only_touches_real_rows():
    xs, w1t, b1, w2, b2 = _setup(n=130, d=32, h=64)
    a0, y0, score = mlp_dense(xs[0], w1t, b1, w2, b2, np.zeros((130, 64)))
    assert score.shape == (2, 64)
    idx = identify_topk(score.astype(np.float32), 16)
    a1, y1 = mlp_sparse(xs[1], w1t, b1, w2, a0, y0, idx)
    assert a1.shape == (130, 64) and y1.shape == (130, 32)


@pytest.mark.parametrize("seed", [0, 1])
def test_drifting_input_sparse_close_to_dense(seed):
    # Informational quality check (not a parity pin): recomputing most columns
    # keeps the output near the dense forward pass.
    xs, w1t, b1, w2, b2 = _setup(seed=seed)
    a0, y0, score = mlp_dense(xs[0], w1t, b1, w2, b2, np.zeros((300, 192)))
    idx = identify_topk(score.astype(np.float32), 150)
    _, y1 = mlp_sparse(xs[1], w1t, b1, w2, a0, y0, idx)
    _, y1d, _ = mlp_dense(xs[1], w1t, b1, w2, b2, a0)
    assert rel_frobenius(y1, y1d) < 0.05


# --------------------------------------------- per-step rescoring (R12) ---
def test_rescore_equals_dense_score_on_recomputed_units():
    # The rescore of a recomputed unit is the dense step's score formula (R1)
    # for that step: mlp_dense(X1, a_old = A0) gives sum_i |A1 - A0| for every
    # unit; a sparse step from A0 must reproduce it exactly on S_b and keep the
    # previous scores elsewhere.  Random S per block (ragged tail block).
    xs, w1t, b1, w2, b2 = _setup(n=300, d=64, h=192)
    a0, y0, sc0 = mlp_dense(xs[0], w1t, b1, w2, b2, np.zeros((300, 192)))
    _, _, sc_dense1 = mlp_dense(xs[1], w1t, b1, w2, b2, a0)
    g = np.random.default_rng(3)
    idx = np.stack([np.sort(g.choice(192, size=50, replace=False)) for _ in range(3)]).astype(np.int32)
    a1, y1, sc1 = mlp_sparse(xs[1], w1t, b1, w2, a0, y0, idx, score=sc0)
    a1n, y1n = mlp_sparse(xs[1], w1t, b1, w2, a0, y0, idx)
    np.testing.assert_array_equal(a1, a1n)          # rescoring changes no other output
    np.testing.assert_array_equal(y1, y1n)
    for b in range(3):
        inside = np.zeros(192, bool)
        inside[idx[b]] = True
        np.testing.assert_allclose(sc1[b, inside], sc_dense1[b, inside], rtol=1e-12, atol=0)
        np.testing.assert_array_equal(sc1[b, ~inside], sc0[b, ~inside])


def test_rescore_brute_force_tiny():
    n, d, h = 130, 8, 6
    xs, w1t, b1, w2, b2 = _setup(n, d, h, seed=5)
    a0 = bf16_round(np.random.default_rng(2).standard_normal((n, h)))
    y0 = np.zeros((n, d))
    sc0 = np.full((2, h), 7.0)
    idx = np.array([[1, 4], [0, 5]], np.int32)
    _, _, sc = mlp_sparse(xs[1], w1t, b1, w2, a0, y0, idx, score=sc0)
    for b, (r0, r1) in enumerate([(0, 128), (128, 130)]):
        for j in range(h):
            if j in idx[b]:
                z = [sum(xs[1][i, c] * w1t[j, c] for c in range(d)) + b1[j] for i in range(r0, r1)]
                a_new = [bf16_round(np.array(0.5 * v * (1 + np.tanh(np.sqrt(2 / np.pi) * (v + 0.044715 * v ** 3)))))
                         for v in z]
                want = sum(abs(float(a_new[i - r0]) - a0[i, j]) for i in range(r0, r1))
                assert abs(sc[b, j] - want) <= 1e-9 * max(1.0, want)
            else:
                assert sc[b, j] == 7.0


def test_rescore_empty_set_keeps_scores():
    xs, w1t, b1, w2, b2 = _setup()
    a0, y0, sc0 = mlp_dense(xs[0], w1t, b1, w2, b2, np.zeros((300, 192)))
    _, _, sc = mlp_sparse(xs[1], w1t, b1, w2, a0, y0, np.zeros((3, 0), np.int32), score=sc0)
    np.testing.assert_array_equal(sc, sc0)
