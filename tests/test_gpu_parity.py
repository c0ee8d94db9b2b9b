"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bars: top-k index sets bit-exact on the same fp32 score bits; float outputs
within relative Frobenius error 2e-2 (bf16 operands, fp32 accumulation);
k = 0 leaves every buffer bit-unchanged; runs are bit-reproducible.
Sizes span several tiles with ragged tails (300 rows = 2 full blocks + 44)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from tests.gpu_helpers import (attn_s_only, bf16_values, bits_of, cache_to_rows, idx_sets_valid, up_bf16, up_f32,
                               worst_block_error)

pytestmark = pytest.mark.gpu
TOL = 2e-2
SCALE = 1.0 / np.sqrt(128.0)


@pytest.fixture(scope="module")
def L(gpu_lib):
    return gpu_lib


# ------------------------------------------------------------------ top-k ---
@pytest.mark.parametrize("kind", ["normal", "ties", "special", "abs"])
@pytest.mark.parametrize("rows,cols,k", [
    (5, 1, 1), (7, 7, 3), (9, 100, 1), (9, 100, 50), (9, 100, 99), (9, 100, 100),
    (4, 4352, 718), (3, 12288, 3686), (3, 12288, 860), (2, 20000, 1400), (1, 118800, 8316),
    (3, 16384, 5000),    # the longest register-held row (16 keys per thread, 16-byte loads)
    (3, 16380, 4000),    # 16-byte loads with the last group of the row out of range
    (3, 20001, 777),     # long rows not a multiple of 4: 4-byte loads
    (2, 16385, 16385),   # every column of a long row
    (2, 40000, 1),
    (2, 30000, 15000),   # long rows, both index lists in LDS (two reads)
    (2, 30000, 19000),   # long rows whose lists overflow LDS (three reads)
])
def test_topk_bit_exact(L, kind, rows, cols, k):
    print(f"topk kind={kind} rows={rows} cols={cols} k={k}", flush=True)
    s = syn.scores(7, rows, cols, kind)
    idx = torch.full((rows, k), -1, dtype=torch.int32, device="cuda")
    L.chipmunk_identify_topk(up_f32(s), rows, cols, k, idx)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), oracle.identify_topk(s, k))


@pytest.mark.parametrize("rows,cols,k", [(3, 12288, 3686), (9, 100, 50), (4, 4352, 718)])
def test_topk_unaligned_rows_take_scalar_loads(L, rows, cols, k):
    # Scores starting 4 bytes past a 16-byte boundary: the register variant
    # reads them one float at a time; same result.
    print(f"topk unaligned rows={rows} cols={cols} k={k}", flush=True)
    s = syn.scores(11, rows, cols, "normal")
    buf = torch.zeros(rows * cols + 4, dtype=torch.float32, device="cuda")
    view = buf[1:1 + rows * cols]
    view.copy_(up_f32(s).reshape(-1))
    assert view.data_ptr() % 16 == 4
    idx = torch.full((rows, k), -1, dtype=torch.int32, device="cuda")
    L.chipmunk_identify_topk(view, rows, cols, k, idx)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), oracle.identify_topk(s, k))


# -------------------------------------------------------------------- MLP ---
def _mlp_inputs(n, d, h, seed=0, bias=True, steps=2):
    w1t_b, w2_b = syn.mlp_weights(seed, d, h)
    g = np.random.default_rng(seed + 100)
    b1 = (g.standard_normal(h) * 0.1).astype(np.float32) if bias else None
    b2 = (g.standard_normal(d) * 0.1).astype(np.float32) if bias else None
    xs = [syn.activations(seed, "X", t, n, d) for t in range(steps)]
    return w1t_b, w2_b, b1, b2, xs


def _mlp_layer(L, n, d, h, k, w1t_b, w2_b, b1, b2):
    from dynamic_column_sparse_amd.layers import MLPDelta
    return MLPDelta(up_bf16(w1t_b), up_bf16(w2_b), n, k,
                    None if b1 is None else up_f32(b1), None if b2 is None else up_f32(b2))


@pytest.mark.parametrize("n,d,h,k", [(300, 256, 640, 200), (256, 128, 512, 128), (130, 384, 1024, 1000)])
def test_mlp_dense_then_sparse_matches_oracle(L, n, d, h, k):
    print(f"mlp parity n={n} d={d} h={h} k={k}", flush=True)
    w1t_b, w2_b, b1, b2, xs = _mlp_inputs(n, d, h)
    lay = _mlp_layer(L, n, d, h, k, w1t_b, w2_b, b1, b2)
    lay.dense(up_bf16(xs[0]))
    torch.cuda.synchronize()
    w1t, w2 = oracle.from_bf16_bits(w1t_b), oracle.from_bf16_bits(w2_b)
    x0, x1 = oracle.from_bf16_bits(xs[0]), oracle.from_bf16_bits(xs[1])
    a0, y0, sc0 = oracle.mlp_dense(x0, w1t, b1, w2, b2, np.zeros((n, h)))
    a_gpu = cache_to_rows(lay.a_cache, n)
    assert np.mean(a_gpu != a0) < 2e-3              # one-ulp bf16 splits at rounding ties only
    assert oracle.rel_frobenius(a_gpu, a0) < 1e-3
    assert oracle.rel_frobenius(lay.y.cpu().numpy(), y0) < TOL
    assert oracle.rel_frobenius(lay.score.cpu().numpy(), sc0) < 1e-3
    pad = bits_of(lay.a_cache).reshape(lay.nb, h, 128)[-1][:, n - (lay.nb - 1) * 128:]
    assert np.all(pad == 0)

    # sparse step on the oracle's index sets (lockstep)
    idx = oracle.identify_topk(sc0.astype(np.float32), k)
    y_before = lay.y.clone()
    lay.sparse(up_bf16(xs[1]), idx=torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    a1, y1 = oracle.mlp_sparse(x1, w1t, b1, w2, a0, y0, idx)
    y_gpu = lay.y.cpu().numpy()
    assert oracle.rel_frobenius(y_gpu, y1) < TOL
    assert oracle.rel_frobenius(y_gpu - y_before.cpu().numpy(), y1 - y0) < TOL
    assert oracle.rel_frobenius(cache_to_rows(lay.a_cache, n), a1) < 1e-3


def test_mlp_k_zero_is_bit_identity_and_k_h_is_dense(L):
    n, d, h = 300, 256, 640
    w1t_b, w2_b, b1, b2, xs = _mlp_inputs(n, d, h, seed=3)
    lay0 = _mlp_layer(L, n, d, h, 0, w1t_b, w2_b, b1, b2)
    lay0.dense(up_bf16(xs[0]))
    torch.cuda.synchronize()
    ybits, abits = lay0.y.clone(), lay0.a_cache.clone()
    lay0.sparse(up_bf16(xs[1]))
    torch.cuda.synchronize()
    assert torch.equal(lay0.y.view(torch.int32), ybits.view(torch.int32))
    assert torch.equal(lay0.a_cache.view(torch.int16), abits.view(torch.int16))

    layh = _mlp_layer(L, n, d, h, h, w1t_b, w2_b, b1, b2)
    layh.dense(up_bf16(xs[0]))
    every = torch.arange(h, dtype=torch.int32, device="cuda").repeat(layh.nb, 1)
    layh.sparse(up_bf16(xs[1]), idx=every)
    torch.cuda.synchronize()
    w1t, w2 = oracle.from_bf16_bits(w1t_b), oracle.from_bf16_bits(w2_b)
    a0, _, _ = oracle.mlp_dense(oracle.from_bf16_bits(xs[0]), w1t, b1, w2, b2, np.zeros((n, h)))
    _, y1d, _ = oracle.mlp_dense(oracle.from_bf16_bits(xs[1]), w1t, b1, w2, b2, a0)
    assert oracle.rel_frobenius(layh.y.cpu().numpy(), y1d) < TOL


def test_mlp_unfused_writeback_matches_fused_bit_exact(L):
    n, d, h, k = 300, 256, 640, 250
    w1t_b, w2_b, b1, b2, xs = _mlp_inputs(n, d, h, seed=5)
    fa = _mlp_layer(L, n, d, h, k, w1t_b, w2_b, b1, b2)
    fb = _mlp_layer(L, n, d, h, k, w1t_b, w2_b, b1, b2)
    for lay in (fa, fb):
        lay.dense(up_bf16(xs[0]))
        lay.identify()
    fa.sparse(up_bf16(xs[1]))
    packed = torch.zeros(fb.nb, k, 128, dtype=torch.bfloat16, device="cuda")
    a_before = fb.a_cache.clone()
    fb.sparse(up_bf16(xs[1]), a_new_packed=packed)
    torch.cuda.synchronize()
    assert torch.equal(fb.a_cache.view(torch.int16), a_before.view(torch.int16))   # cache untouched
    fb.writeback(packed)
    torch.cuda.synchronize()
    assert torch.equal(fa.a_cache.view(torch.int16), fb.a_cache.view(torch.int16))
    assert torch.equal(fa.y.view(torch.int32), fb.y.view(torch.int32))


def test_mlp_free_running_tiny_workload(L):
    # 256 tokens, d 128, h 512, keep 128 per block, GPU's own identification.
    n, d, h, k = 256, 128, 512, 128
    w1t_b, w2_b, _, _, xs = _mlp_inputs(n, d, h, seed=0, bias=False)
    lay = _mlp_layer(L, n, d, h, k, w1t_b, w2_b, None, None)
    lay.dense(up_bf16(xs[0]))
    lay.identify()
    lay.sparse(up_bf16(xs[1]))
    torch.cuda.synchronize()
    w1t, w2 = oracle.from_bf16_bits(w1t_b), oracle.from_bf16_bits(w2_b)
    a0, y0, sc0 = oracle.mlp_dense(oracle.from_bf16_bits(xs[0]), w1t, None, w2, None, np.zeros((n, h)))
    ridx = oracle.identify_topk(sc0.astype(np.float32), k)
    jac = idx_sets_valid(lay.idx.cpu().numpy(), ridx, sc0.astype(np.float32))
    print(f"tiny workload index-set Jaccard {jac:.4f}")
    _, y1 = oracle.mlp_sparse(oracle.from_bf16_bits(xs[1]), w1t, None, w2, a0, y0, ridx)
    assert oracle.rel_frobenius(lay.y.cpu().numpy(), y1) < TOL


def test_mlp_deterministic(L):
    n, d, h, k = 300, 256, 640, 200
    w1t_b, w2_b, b1, b2, xs = _mlp_inputs(n, d, h, seed=9, steps=3)
    outs = []
    for _ in range(2):
        lay = _mlp_layer(L, n, d, h, k, w1t_b, w2_b, b1, b2)
        lay.step(up_bf16(xs[0]), True)
        lay.step(up_bf16(xs[1]), False)
        lay.step(up_bf16(xs[2]), False)
        torch.cuda.synchronize()
        outs.append((lay.y.clone(), lay.a_cache.clone(), lay.idx.clone(), lay.score.clone()))
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


# -------------------------------------------------------------- attention ---
def _qkv(H, n, step, seed=0):
    return [syn.heads_activations(seed, t, step, H, n) for t in "QKV"]


@pytest.mark.parametrize("n,H,kk,sc", [
    (300, 2, 100, SCALE), (256, 8, 64, SCALE), (200, 1, 200, SCALE),
    (33, 3, 5, SCALE),          # one full 32-key chunk and a 1-key tail
    (1, 1, 1, SCALE),           # a single token
    (300, 2, 100, -0.5 * SCALE),  # negative scale: the row max is the minimum raw score
    # more than 256 keys: the 8-slot key-id ring wraps, and the steady-state
    # loop (at least 8 chunks) runs
    (1000, 2, 300, SCALE),
    (600, 2, 600, SCALE),       # every key of the layer, 19 chunks (last one partial)
    (2000, 8, 718, SCALE),      # the FLUX keep count, 8 heads (XCD head mapping)
])
def test_attention_refresh_and_sparse_match_oracle(L, n, H, kk, sc):
    print(f"attention parity n={n} H={H} kk={kk} scale={sc}", flush=True)
    from dynamic_column_sparse_amd.layers import AttnDelta
    b0, b1_ = _qkv(H, n, 0), _qkv(H, n, 1)
    att = AttnDelta(n, H, kk, "cuda", scale=sc)
    g0 = [up_bf16(a) for a in b0]
    g1 = [up_bf16(a) for a in b1_]
    att.dense(*g0)
    torch.cuda.synchronize()
    m_g, den_g, num_g = att.m.cpu().numpy(), att.den.cpu().numpy(), att.num.cpu().numpy()
    o_g, sc_g = att.o.cpu().numpy(), att.score.cpu().numpy()
    refs = []
    for hh in range(H):
        q0, k0, v0 = (oracle.from_bf16_bits(a[hh]) for a in b0)
        m, den, num, o, score = oracle.attn_dense(q0, k0, v0, sc)
        np.testing.assert_allclose(m_g[hh], m, rtol=1e-5, atol=1e-5)
        assert oracle.rel_frobenius(den_g[hh], den) < 1e-3
        assert oracle.rel_frobenius(num_g[hh], num) < TOL
        assert oracle.rel_frobenius(o_g[hh], o) < TOL
        assert oracle.rel_frobenius(sc_g[hh], score) < 1e-3
        refs.append((m, score))
    # refresh with the oracle's index sets, then a sparse step on drifted inputs
    idx = np.concatenate([oracle.identify_topk(refs[hh][1].astype(np.float32), kk) for hh in range(H)], axis=0)
    idx_g = torch.from_numpy(idx).cuda()
    att.refresh_rest(*g0, idx=idx_g)
    att.sparse(*g1, idx=idx_g)
    o_s_g = attn_s_only(L, att, *g1, idx=idx_g).cpu().numpy()
    torch.cuda.synchronize()
    nb = (n + 127) // 128
    sizes = [min(n, (b + 1) * 128) - b * 128 for b in range(nb)]
    num_r, den_r, o_g = att.num.cpu().numpy(), att.den.cpu().numpy(), att.o.cpu().numpy()
    for hh in range(H):
        q0, k0, v0 = (oracle.from_bf16_bits(a[hh]) for a in b0)
        q1, k1, v1 = (oracle.from_bf16_bits(a[hh]) for a in b1_)
        sidx = idx[hh * nb:(hh + 1) * nb]
        m = refs[hh][0]
        _, den, num, _, _ = oracle.attn_dense(q0, k0, v0, sc)
        nr, dr = oracle.attn_rest(q0, k0, v0, m, sidx, sc)
        # bars per query block: the rest state, the part REFRESH took out (the
        # chosen keys alone), the sparse output, and the output over S alone
        z = np.zeros_like(nr)
        o1 = oracle.attn_sparse(q1, k1, v1, m, nr, dr, sidx, sc)
        o_s = oracle.attn_sparse(q1, k1, v1, m, z, np.zeros_like(dr), sidx, sc)
        for name, g, r, tol in (("den_rest", den_r[hh][:, None], dr[:, None], 1e-3), ("num_rest", num_r[hh], nr, TOL),
                                ("den_S", (den_g[hh] - den_r[hh])[:, None], (den - dr)[:, None], 1e-3),
                                ("num_S", num_g[hh] - num_r[hh], num - nr, TOL),
                                ("o", o_g[hh], o1, TOL), ("o over S alone", o_s_g[hh], o_s, TOL)):
            e, i, _ = worst_block_error(g, r, sizes)
            assert e < tol, f"head {hh} block {i}: {name} rel-F {e:.2e}"


def test_attention_free_running_and_deterministic(L):
    from dynamic_column_sparse_amd.layers import AttnDelta
    n, H, kk = 300, 8, 50
    b0, b1_ = _qkv(H, n, 0, seed=4), _qkv(H, n, 1, seed=4)
    outs = []
    for _ in range(2):
        att = AttnDelta(n, H, kk, "cuda")
        att.step(*[up_bf16(a) for a in b0], refresh=True)
        att.step(*[up_bf16(a) for a in b1_], refresh=False)
        torch.cuda.synchronize()
        outs.append((att.o.clone(), att.idx.clone()))
    assert torch.equal(outs[0][0].view(torch.int32), outs[1][0].view(torch.int32))
    assert torch.equal(outs[0][1], outs[1][1])
    nb = (n + 127) // 128
    gidx = outs[0][1].cpu().numpy()
    o_g = outs[0][0].cpu().numpy()
    for hh in range(H):
        q0, k0, v0 = (oracle.from_bf16_bits(a[hh]) for a in b0)
        q1, k1, v1 = (oracle.from_bf16_bits(a[hh]) for a in b1_)
        m, den, num, o, score = oracle.attn_dense(q0, k0, v0, SCALE)
        ridx = oracle.identify_topk(score.astype(np.float32), kk)
        idx_sets_valid(gidx[hh * nb:(hh + 1) * nb], ridx, score.astype(np.float32))
        nr, dr = oracle.attn_rest(q0, k0, v0, m, ridx, SCALE)
        o1 = oracle.attn_sparse(q1, k1, v1, m, nr, dr, ridx, SCALE)
        assert oracle.rel_frobenius(o_g[hh], o1) < TOL


def test_attention_no_keys_returns_cached_output(L):
    from dynamic_column_sparse_amd.layers import AttnDelta
    n, H = 300, 2
    b0, b1_ = _qkv(H, n, 0, seed=6), _qkv(H, n, 1, seed=6)
    att = AttnDelta(n, H, 0, "cuda")
    att.dense(*[up_bf16(a) for a in b0])
    torch.cuda.synchronize()
    o_ref = att.o.clone()
    num_b, den_b = att.num.clone(), att.den.clone()
    att.refresh_rest(*[up_bf16(a) for a in b0])       # kk = 0: nothing subtracted
    att.sparse(*[up_bf16(a) for a in b1_])
    torch.cuda.synchronize()
    assert torch.equal(att.num.view(torch.int32), num_b.view(torch.int32))
    assert torch.equal(att.den.view(torch.int32), den_b.view(torch.int32))
    assert torch.equal(att.o.view(torch.int32), o_ref.view(torch.int32))


@pytest.mark.parametrize("order", ["rising", "falling", "wide"])
def test_attention_statistics_over_wide_score_ranges(L, order):
    """Row max and denominator of the refresh when the scores span a wide range
    along the keys: rising scores move the running maximum on nearly every
    chunk (the statistics pass re-bases its sum many times), falling scores
    never after the first chunk, and wide Gaussian scores (inputs x 6) put
    single keys far above the rest.  m, den and the key-mass score are checked
    against the oracle per query block, on 1000 tokens (7 full blocks and a
    104-row tail) and two heads."""
    from dynamic_column_sparse_amd.layers import AttnDelta
    n, H = 1000, 2
    g = np.random.default_rng(7)
    q = 0.5 + 0.05 * g.standard_normal((H, n, 128))
    ramp = np.arange(n, dtype=np.float64)[None, :, None] / 40.0
    if order == "rising":
        k = ramp * (1.0 + 0.05 * g.standard_normal((H, n, 128)))
    elif order == "falling":
        k = ramp[:, ::-1] * (1.0 + 0.05 * g.standard_normal((H, n, 128)))
    else:
        q = 6.0 * g.standard_normal((H, n, 128))
        k = 6.0 * g.standard_normal((H, n, 128))
    v = g.standard_normal((H, n, 128))
    qb, kb, vb = (syn.f32_to_bf16_bits(a.astype(np.float32)) for a in (q, k, v))
    att = AttnDelta(n, H, 64, "cuda")
    att.dense(up_bf16(qb), up_bf16(kb), up_bf16(vb))
    torch.cuda.synchronize()
    m_g, den_g, sc_g = att.m.cpu().numpy(), att.den.cpu().numpy(), att.score.cpu().numpy()
    sizes = [min(n, (b + 1) * 128) - b * 128 for b in range((n + 127) // 128)]
    for hh in range(H):
        q0, k0, v0 = (oracle.from_bf16_bits(a[hh]) for a in (qb, kb, vb))
        m, den, _, _, score = oracle.attn_dense(q0, k0, v0, SCALE)
        np.testing.assert_allclose(m_g[hh], m, rtol=1e-5, atol=1e-5)
        e, i, _ = worst_block_error(den_g[hh][:, None], den[:, None], sizes)
        assert e < 1e-3, f"{order} head {hh} block {i}: den rel-F {e:.2e}"
        e_s = oracle.rel_frobenius(sc_g[hh], score)
        assert e_s < 1e-3, f"{order} head {hh}: score rel-F {e_s:.2e}"
