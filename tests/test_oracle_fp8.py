"""Pins of the oracle's fp8 quantizer (the fp8 variant of the MLP's first
product: x and W1^T rows as e4m3 codes with one power-of-two scale per row).

Fixed outside the oracle: torch's float8_e4m3fn type (decode of all 256 codes,
and its float32 -> e4m3 cast, round to nearest even) on random values and on
every midpoint between neighbouring codes; hand-derived ties; the defining
property of the row exponent (the smallest power of two that brings the row
into [-448, 448]); the half-quantum error bound; values already on the grid
are kept exactly."""
import numpy as np
import torch

from oracle.chipmunk_oracle import (dequantize_fp8_rows, fp8_e4m3_decode, fp8_e4m3_encode, fp8_e4m3_round,
                                    fp8_row_exponent, fp8_rows, quantize_fp8_rows)

CODES = np.arange(256, dtype=np.uint8)


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


def test_decode_all_codes_matches_torch():
    ours, ref = fp8_e4m3_decode(CODES), _torch_decode(CODES)
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    np.testing.assert_array_equal(ours[~np.isnan(ours)], ref[~np.isnan(ref)])
    assert np.isnan(ours[[0x7f, 0xff]]).all() and np.nanmax(ours) == 448.0


def test_encode_matches_torch_cast_and_round_trips():
    vals = fp8_e4m3_decode(CODES)
    fin = ~np.isnan(vals)
    np.testing.assert_array_equal(fp8_e4m3_encode(vals[fin]), CODES[fin])
    g = np.random.default_rng(0)
    v = np.clip((g.standard_normal(100000) * np.exp(g.uniform(-14, 6, 100000))).astype(np.float32), -448, 448)
    pos = np.sort(vals[fin & (vals >= 0)])
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)          # every tie between neighbouring codes
    v = np.concatenate([v, mids, -mids, np.float32([0.0, -0.0, 448.0, -448.0])])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(fp8_e4m3_encode(v.astype(np.float64)), ref)


def test_hand_ties():
    # (value, code): ties go to the even code
    cases = [(448.0, 0x7e), (-448.0, 0xfe), (440.0, 0x7e),   # 440: halfway 416..448 goes to even 448
             (1.0625, 0x38), (1.1875, 0x3a), (-1.0625, 0xb8),
             (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (5 * 2.0 ** -10, 0x02),
             (2.0 ** -9, 0x01), (0.015625, 0x08), (240.0, 0x77), (232.0, 0x76), (248.0, 0x78)]
    for val, code in cases:
        assert int(fp8_e4m3_encode(np.array([val]))[0]) == code, (val, code)
        assert fp8_e4m3_round(np.array([val]))[0] == fp8_e4m3_decode(np.array([code], np.uint8))[0]


def test_row_exponent_is_the_smallest_fitting_power_of_two():
    g = np.random.default_rng(1)
    amax = np.concatenate([np.exp(g.uniform(-60, 60, 5000)),
                           448.0 * np.ldexp(1.0, np.arange(-20, 20)),               # exactly 448 * 2^j
                           np.nextafter(448.0 * np.ldexp(1.0, np.arange(-20, 20)), np.inf),
                           np.ldexp(1.0, np.arange(-40, 40))])
    e = fp8_row_exponent(amax)
    assert np.all(np.ldexp(amax, -e) <= 448.0)
    assert np.all(np.ldexp(amax, -(e - 1)) > 448.0)
    np.testing.assert_array_equal(fp8_row_exponent(448.0 * np.ldexp(1.0, np.arange(-20, 20))), np.arange(-20, 20))
    assert fp8_row_exponent(np.array([0.0]))[0] == 0
    assert fp8_row_exponent(np.array([1e-40]))[0] == -126        # floor of the exponent range


def test_quantize_rows_error_bound_and_grid_values_are_kept():
    g = np.random.default_rng(2)
    a = g.standard_normal((50, 192)) * np.exp(g.uniform(-8, 8, (50, 1)))
    a[3] = 0.0
    codes, sb = quantize_fp8_rows(a)
    assert codes.dtype == np.uint8 and sb.dtype == np.uint8 and sb[3] == 127
    e = sb.astype(np.int64) - 127
    dq = dequantize_fp8_rows(codes, sb)
    # half a quantum: 2^-4 relative in the normal range, 2^-10 * 2^e below it
    bound = np.maximum(np.abs(a) * 2.0 ** -4, np.ldexp(1.0, e - 10)[:, None])
    assert np.all(np.abs(dq - a) <= bound)
    assert np.all(np.abs(dq).max(axis=1) <= np.ldexp(448.0, e))
    # values already on the grid are kept (a row whose maximum rounded down to
    # half the next power of two may take a smaller exponent, same values)
    np.testing.assert_array_equal(fp8_rows(dq), dq)


# ---- blocks (D of the fp8 second product) and columns (W2) -------------------
def test_blocks_reduce_to_rows_and_are_independent():
    from oracle.chipmunk_oracle import fp8_blocks, quantize_fp8_blocks
    g = np.random.default_rng(5)
    a = g.standard_normal((7, 96)) * np.exp(g.uniform(-6, 6, (7, 96)))
    # one block per row is row quantization
    np.testing.assert_array_equal(fp8_blocks(a, 96), fp8_rows(a))
    # each 32-block is quantized on its own, as an explicitly cut-out row would be
    codes, sb = quantize_fp8_blocks(a, 32)
    assert sb.shape == (7, 3)
    for j in range(3):
        c_j, s_j = quantize_fp8_rows(a[:, 32 * j:32 * j + 32])
        np.testing.assert_array_equal(codes[:, 32 * j:32 * j + 32], c_j)
        np.testing.assert_array_equal(sb[:, j], s_j)
    # changing one block leaves the others' values alone
    b = a.copy()
    b[:, 40:50] *= 1000.0
    fa, fb = fp8_blocks(a, 32), fp8_blocks(b, 32)
    np.testing.assert_array_equal(fa[:, :32], fb[:, :32])
    np.testing.assert_array_equal(fa[:, 64:], fb[:, 64:])


def test_blocks_ragged_tail_and_error_bound():
    from oracle.chipmunk_oracle import fp8_blocks, quantize_fp8_blocks
    g = np.random.default_rng(6)
    a = g.standard_normal((5, 70))
    codes, sb = quantize_fp8_blocks(a, 32)
    assert codes.shape == (5, 70) and sb.shape == (5, 3)
    # the 6-element tail block is quantized as if padded with zeros
    c_t, s_t = quantize_fp8_rows(np.concatenate([a[:, 64:], np.zeros((5, 26))], axis=1))
    np.testing.assert_array_equal(codes[:, 64:], c_t[:, :6])
    np.testing.assert_array_equal(sb[:, 2], s_t)
    dq = fp8_blocks(a, 32)
    e = np.repeat(sb.astype(np.int64) - 127, 32, axis=1)[:, :70]
    assert np.all(np.abs(dq - a) <= np.maximum(np.abs(a) * 2.0 ** -4, np.ldexp(1.0, e - 10)))


def test_cols_are_rows_of_the_transpose():
    from oracle.chipmunk_oracle import fp8_cols
    g = np.random.default_rng(7)
    a = g.standard_normal((40, 24)) * np.exp(g.uniform(-5, 5, (1, 24)))   # columns of very different size
    c = fp8_cols(a)
    np.testing.assert_array_equal(c.T, fp8_rows(a.T))
    # every column uses its own range: its largest entry keeps 3 significant bits
    assert np.all(np.abs(c - a).max(axis=0) <= np.abs(a).max(axis=0) * 2.0 ** -4)


def test_sparse_mlp_with_fp8_second_product():
    from oracle import mlp_dense, mlp_sparse
    from oracle.chipmunk_oracle import bf16_round, fp8_blocks, fp8_cols
    g = np.random.default_rng(8)
    n, d, h, k = 200, 64, 96, 40
    x0, x1 = bf16_round(g.standard_normal((n, d))), bf16_round(g.standard_normal((n, d)))
    w1t = bf16_round(g.standard_normal((h, d)) / 8)
    w2 = bf16_round(g.standard_normal((h, d)) / 10)
    a0, y0, sc = mlp_dense(x0, w1t, None, w2, None, np.zeros((n, h)))
    idx = np.stack([np.sort(g.choice(h, k, replace=False)) for _ in range(2)]).astype(np.int32)
    a_ref, y_ref = mlp_sparse(x1, w1t, None, w2, a0, y0, idx)
    w2q = fp8_cols(w2)
    a_q, y_q = mlp_sparse(x1, w1t, None, w2q, a0, y0, idx, d_fp8=True)
    np.testing.assert_array_equal(a_q, a_ref)                 # the cache does not see the fp8 product
    # the change of y departs from the exact one by no more than the operands' rounding
    for b, (r0, r1) in enumerate([(0, 128), (128, 200)]):
        s = idx[b]
        dd = a_ref[r0:r1][:, s] - a0[r0:r1][:, s]
        bound = (np.abs(fp8_blocks(bf16_round(dd), 32) - dd) @ np.abs(w2q[s])
                 + np.abs(dd) @ np.abs(w2q[s] - w2[s]))
        assert np.all(np.abs((y_q - y_ref)[r0:r1]) <= bound * (1 + 1e-9) + 1e-12)
    # no units: nothing changes
    none = np.zeros((2, 0), np.int32)
    a_n, y_n = mlp_sparse(x1, w1t, None, w2q, a0, y0, none, d_fp8=True)
    np.testing.assert_array_equal(y_n, y0)
