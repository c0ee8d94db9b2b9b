"""Pins of the oracle's storage rounding and GELU against facts fixed outside it:
a library conversion, hand-derived values of the bf16 format, and closed-form
identities of the tanh-form GELU."""
import math

import numpy as np
import pytest
import torch

from oracle import bf16_bits, bf16_round, from_bf16_bits, gelu_tanh


def _torch_bf16(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()


def test_bf16_round_matches_torch_conversion():
    # torch's fp32 -> bf16 conversion is round-to-nearest-even: a library pin.
    g = np.random.default_rng(0)
    x = np.concatenate([
        g.standard_normal(100000).astype(np.float32),
        (g.standard_normal(20000) * 1e-38).astype(np.float32),      # bf16 subnormal range
        (g.standard_normal(20000) * 1e38).astype(np.float32),       # near overflow
        (g.integers(-2**20, 2**20, 20000) * 2.0**-12).astype(np.float32),
    ])
    # exact ties: 1 + odd multiples of 2^-8
    ties = (1.0 + (2 * np.arange(64) + 1) * 2.0**-8).astype(np.float32)
    x = np.concatenate([x, ties, -ties])
    np.testing.assert_array_equal(bf16_round(x.astype(np.float64)), _torch_bf16(x))


@pytest.mark.parametrize("x,expect", [
    (1.0 + 2.0**-8, 1.0),                      # tie -> even mantissa (0)
    (1.0 + 3 * 2.0**-8, 1.0 + 2.0**-6),        # tie -> even mantissa (2)
    (1.0 + 2.0**-8 + 2.0**-30, 1.0 + 2.0**-7), # just above the tie
    (-(1.0 + 2.0**-8), -1.0),
    ((2 - 2.0**-7) * 2.0**127, (2 - 2.0**-7) * 2.0**127),    # largest finite bf16
    ((2 - 2.0**-8) * 2.0**127, math.inf),      # halfway to 2^128 rounds to even -> overflow
    (2.0**-133, 2.0**-133),                    # smallest subnormal
    (2.0**-134, 0.0),                          # tie at half the smallest subnormal -> even (0)
    (3 * 2.0**-134, 2.0**-132),                # 1.5 subnormal quanta -> 2 (even)
    (0.0, 0.0),
])
def test_bf16_round_hand_values(x, expect):
    assert bf16_round(np.array([x]))[0] == expect


def test_bf16_bits_roundtrip_and_specials():
    b = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    v = from_bf16_bits(b)
    finite = np.isfinite(v)
    np.testing.assert_array_equal(bf16_bits(v[finite]), b[finite])
    assert np.isnan(bf16_round(np.array([np.nan]))[0])
    assert bf16_round(np.array([-np.inf]))[0] == -np.inf
    assert math.copysign(1.0, bf16_round(np.array([-0.0]))[0]) == -1.0
    assert from_bf16_bits(np.array([0x3F80], np.uint16))[0] == 1.0
    assert from_bf16_bits(np.array([0xC000], np.uint16))[0] == -2.0


def test_gelu_tanh_library_and_identities():
    z = np.linspace(-12, 12, 20001)
    ref = torch.nn.functional.gelu(torch.from_numpy(z), approximate="tanh").numpy()
    np.testing.assert_allclose(gelu_tanh(z), ref, rtol=1e-14, atol=1e-15)
    assert gelu_tanh(np.array([0.0]))[0] == 0.0
    # gelu(x) - gelu(-x) = x exactly in real arithmetic for the tanh form
    np.testing.assert_allclose(gelu_tanh(z) - gelu_tanh(-z), z, rtol=1e-14, atol=1e-14)
    # limits
    assert abs(gelu_tanh(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(gelu_tanh(np.array([-40.0]))[0]) < 1e-12
    # a value computed by hand: u = sqrt(2/pi) * (1 + 0.044715) at z = 1
    u = math.sqrt(2 / math.pi) * 1.044715
    assert abs(gelu_tanh(np.array([1.0]))[0] - 0.5 * (1 + math.tanh(u))) < 1e-15


def test_incremental_walk_matches_per_step_generation():
    import synthetic as syn
    w = syn.activation_walk(3, "X", 4, 300, 64)
    for t in range(4):
        np.testing.assert_array_equal(w[t], syn.activations(3, "X", t, 300, 64))
    hw = syn.heads_walk(3, "K", 3, 2, 200)
    for t in range(3):
        np.testing.assert_array_equal(hw[t], syn.heads_activations(3, "K", t, 2, 200))
    # bf16 packing of the generator agrees with torch's conversion
    x = syn.walk_block(3, 1, 2, 0, 0, 128, 64)
    np.testing.assert_array_equal(syn.f32_to_bf16_bits(x).view(np.int16),
                                  torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy())


def test_chunked_generation_matches_per_block_streams():
    # Generation jobs cover several row blocks at once (5 blocks at 3072 columns);
    # every block must still come from its own (tag, step, head, block) stream.
    import synthetic as syn
    from synthetic.gen import TAG, walk_block
    n, cols = 1500, 3072                               # 12 blocks, last one 92 rows
    ref = [np.concatenate([syn.f32_to_bf16_bits(walk_block(5, TAG["X"], t, 0, b, min(n, (b + 1) * 128) - b * 128, cols))
                           for b in range(12)]) for t in range(3)]
    w = syn.activation_walk(5, "X", 3, n, cols)
    for t in range(3):
        np.testing.assert_array_equal(w[t], ref[t])
        np.testing.assert_array_equal(syn.activations(5, "X", t, n, cols), ref[t])
    np.testing.assert_array_equal(syn.activations(5, "X", 2, n, cols, blocks=[11, 3]),
                                  np.concatenate([ref[2][1408:], ref[2][384:512]]))


# ------------------------------------------------------ the parity checker ---
def test_rel_frobenius_hand_values():
    # ||a - b||_F / ||b||_F, worked by hand.  The reference is the second
    # argument: swapping the arguments changes the result.
    from oracle import rel_frobenius
    b = np.array([[3.0, 0.0], [0.0, 4.0]])              # ||b||_F = 5
    assert rel_frobenius(b, b) == 0.0
    assert rel_frobenius(2 * b, b) == 1.0               # ||b|| / ||b||
    assert rel_frobenius(np.zeros_like(b), b) == 1.0    # a dropped output is a 100% error
    assert rel_frobenius(b + np.array([[0.0, 0.5], [0.0, 0.0]]), b) == 0.1
    assert rel_frobenius(b, 2 * b) == 0.5               # ||b|| / ||2b||, not ||b|| / ||b||
    assert rel_frobenius(np.array([1.0, 2.0]), np.array([1.0, 0.0])) == 2.0
    # zero reference: the absolute norm of the difference
    assert rel_frobenius(np.zeros(3), np.zeros(3)) == 0.0
    assert rel_frobenius(np.array([0.0, 3.0, 4.0]), np.zeros(3)) == 5.0


def test_rel_frobenius_matches_linalg_norms():
    # Against numpy's own norms on random arrays of several ranks, float32
    # inputs included (the checker works in float64).
    from oracle import rel_frobenius
    g = np.random.default_rng(5)
    for shape in [(7,), (33, 17), (4, 5, 6)]:
        b = g.standard_normal(shape)
        a = b + 1e-3 * g.standard_normal(shape)
        ref = np.sqrt(np.sum((a - b) ** 2)) / np.sqrt(np.sum(b ** 2))
        assert abs(rel_frobenius(a, b) - ref) <= 1e-12 * ref
        a32, b32 = a.astype(np.float32), b.astype(np.float32)
        ref32 = (np.linalg.norm((a32.astype(np.float64) - b32.astype(np.float64)).ravel())
                 / np.linalg.norm(b32.astype(np.float64).ravel()))
        assert abs(rel_frobenius(a32, b32) - ref32) <= 1e-12 * ref32
    # one wrong column of 3072 columns: about 1/sqrt(3072) of the whole, so a
    # single norm over a tensor dilutes a localized error (the GPU tests also
    # apply their bars per block and per column group)
    b = g.standard_normal((128, 3072))
    a = b.copy()
    a[:, 5] = 0.0
    assert 0.015 < rel_frobenius(a, b) < 0.022


def test_stepwise_walk_matches_whole_walks():
    # The step-at-a-time walker gives the same bits as the whole-walk
    # generators, for several heads, a ragged last block and wide rows.
    import synthetic as syn
    w = syn.Walk(3, "K", 2, 300, 128)
    hw = syn.heads_walk(3, "K", 4, 2, 300)
    for t in range(4):
        np.testing.assert_array_equal(w.advance(), hw[t])
    wx = syn.Walk(5, "X", 1, 1500, 3072)
    aw = syn.activation_walk(5, "X", 3, 1500, 3072)
    for t in range(3):
        np.testing.assert_array_equal(wx.advance()[0], aw[t])
