"""chipmunk_sparse_step: the MLP's phase 2 and the attention delta in one grid.

  * Against the separate calls (chipmunk_sparse_mlp_delta, then
    chipmunk_sparse_attn_delta): bit-identical y, cache, index sets and o, over
    several sparse steps.  The shapes cover ragged row blocks, both phase-2
    tile widths (d a multiple of 256, and not), head counts with and without
    the XCD head mapping (heads % 8), k = 0, kk = 0, and an attention layer
    whose token count differs from the MLP's; layers with bf16 products, both
    products on fp8, and the fp8 second product with per-step rescoring.
  * Against the oracle at the FLUX.1-dev shapes (1280x768 and 2304x1280), in
    the launch configuration the benchmark times: sampled row blocks (MLP) and
    (head, query block) slices (attention), each recomputed on its own (exact,
    as every block depends only on its own rows and the shared weights or
    keys).  Bars as for the separate calls: rel. Frobenius <= 2e-2 on y and on
    its change per step, per sampled row block and per (block, 256 columns)
    tile; on o per slice and on o over the chosen keys alone; 1e-3 on the
    cache.
  * Overlapping buffers are refused before anything is launched.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from tests.gpu_helpers import attn_s_only, block_sizes, up_bf16, worst_block_error
from tests.test_gpu_fullsize import RB, SCALE, TOL, _cache_rows, _rows_of, _sample_blocks

pytestmark = pytest.mark.gpu


def _bits(t):
    if t.dtype == torch.int32:
        return t
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def _pair(n, d, h, k, na, H, kk, seed, steps, **mlp_kw):
    from dynamic_column_sparse_amd.layers import AttnDelta, MLPDelta
    w1t_b, w2_b = syn.mlp_weights(seed, d, h)
    xs = [up_bf16(x) for x in syn.activation_walk(seed, "X", steps, n, d)]
    qkv = [[up_bf16(a) for a in st] for st in zip(*[syn.heads_walk(seed, t, steps, H, na) for t in "QKV"])]
    layers = []
    for _ in range(2):
        mlp = MLPDelta(up_bf16(w1t_b), up_bf16(w2_b), n, k, **mlp_kw)
        att = AttnDelta(na, H, kk, "cuda")
        mlp.step(xs[0], refresh=True)
        att.step(*qkv[0], refresh=True)
        layers.append((mlp, att))
    return layers, xs, qkv


@pytest.mark.parametrize("n,d,h,k,na,H,kk,mode", [
    (300, 256, 640, 200, 300, 2, 100, "bf16"),      # ragged, 256-wide phase-2 tiles, 2 heads
    (1000, 384, 1024, 130, 1000, 8, 300, "bf16"),   # 128-wide tiles (d % 256 != 0), XCD head mapping
    (300, 256, 640, 0, 517, 3, 64, "bf16"),         # k = 0: attention units only; other token count
    (517, 256, 512, 64, 300, 8, 0, "bf16"),         # kk = 0: o = num / den beside the MLP tiles
    (129, 128, 64, 64, 129, 1, 129, "bf16"),        # one unit each side, every column / key kept
    (300, 256, 640, 200, 300, 2, 100, "fp8"),       # both MLP products on fp8 operands
    (1000, 384, 1024, 130, 1000, 8, 300, "fp8"),    # the same with 128-wide phase-2 tiles
    (517, 256, 512, 64, 300, 8, 0, "fp8w2"),        # fp8 second product only, rescoring on
])
def test_fused_step_matches_separate_calls(gpu_lib, n, d, h, k, na, H, kk, mode):
    from dynamic_column_sparse_amd.layers import sparse_step
    print(f"fused step vs separate calls n={n} d={d} h={h} k={k} na={na} H={H} kk={kk} {mode}", flush=True)
    steps = 4
    kw = {"bf16": {}, "fp8": dict(fp8=True, fp8_w2=True), "fp8w2": dict(fp8_w2=True, rescore=True)}[mode]
    ((m_s, a_s), (m_f, a_f)), xs, qkv = _pair(n, d, h, k, na, H, kk, 5, steps, **kw)
    torch.cuda.synchronize()
    for t in range(1, steps):
        m_s.step(xs[t], refresh=False)
        a_s.step(*qkv[t], refresh=False)
        sparse_step(m_f, a_f, xs[t], *qkv[t])
        torch.cuda.synchronize()
        for name, a, b in (("y", m_s.y, m_f.y), ("a_cache", m_s.a_cache, m_f.a_cache), ("idx", m_s.idx, m_f.idx),
                           ("o", a_s.o, a_f.o)):
            assert torch.equal(_bits(a), _bits(b)), f"step {t}: {name}"
    assert torch.isfinite(a_f.o).all() and torch.isfinite(m_f.y).all()


def test_fused_step_refuses_overlap(gpu_lib):
    from dynamic_column_sparse_amd import lib
    from dynamic_column_sparse_amd.layers import AttnDelta, MLPDelta
    n, d, h, k, H, kk = 256, 256, 512, 64, 2, 64
    w1t_b, w2_b = syn.mlp_weights(0, d, h)
    mlp = MLPDelta(up_bf16(w1t_b), up_bf16(w2_b), n, k)
    att = AttnDelta(n, H, kk, "cuda")
    x = torch.zeros(n, d, dtype=torch.bfloat16, device="cuda")
    q = torch.zeros(H, n, 128, dtype=torch.bfloat16, device="cuda")
    y_before = mlp.y.clone()
    # o aliases y: refused, and nothing ran.
    alias = mlp.y.view(H, n, 128)            # y is [256, 256] fp32: the same bytes as o [2, 256, 128]
    with pytest.raises(lib.ChipmunkError) as e:
        lib.chipmunk_sparse_step(mlp.layer, x, mlp.idx, k, mlp.y, None, mlp.ws, att.layer, q, q, q, att.idx, kk,
                                 alias)
    assert e.value.code == 2 and "overlaps" in str(e.value)
    torch.cuda.synchronize()
    assert torch.equal(mlp.y, y_before)


@pytest.mark.parametrize("n,kk", [
    (4352, 718),     # FLUX.1-dev at 1280x768: 3840 image + 512 text tokens, keep 16.5% of keys
    (12032, 1985),   # FLUX.1-dev at 2304x1280: 11520 image + 512 text tokens, same sparsity
])
def test_flux_fused_step_against_oracle(gpu_lib, n, kk):
    # MLP d 3072, h 12288, keep 3686 per block; 24 heads x 128: refresh at step
    # 0, then three sparse steps through the shared-grid call.
    from dynamic_column_sparse_amd.layers import AttnDelta, MLPDelta, sparse_step
    d, h, k, H, steps, seed = 3072, 12288, 3686, 24, 4, 0
    nb = (n + RB - 1) // RB
    blocks = _sample_blocks(nb, 3, seed + 11, n)
    rows = _rows_of(blocks, n)
    rows_t = torch.from_numpy(rows).cuda()
    g = np.random.default_rng(21)
    slices = [(int(g.integers(H)), int(g.integers(nb))) for _ in range(3)] + [(H - 1, nb - 1)]
    print(f"flux fused step n={n} kk={kk}: blocks {blocks}, slices {slices}", flush=True)

    w1t_b, w2_b = syn.mlp_weights(seed, d, h)
    mlp = MLPDelta(up_bf16(w1t_b), up_bf16(w2_b), n, k)
    w1t, w2 = oracle.from_bf16_bits(w1t_b), oracle.from_bf16_bits(w2_b)
    del w1t_b, w2_b
    xs = syn.activation_walk(seed, "X", steps, n, d)
    walks = [syn.heads_walk(seed, tag, steps, H, n) for tag in "QKV"]
    att = AttnDelta(n, H, kk, "cuda")

    a_s = np.zeros((len(rows), h))
    state = {}
    y_s = None
    for t in range(steps):
        x_g = up_bf16(xs[t])
        qkv_g = [up_bf16(w[t]) for w in walks]
        x_s = oracle.from_bf16_bits(xs[t][rows])
        if t == 0:
            mlp.step(x_g, refresh=True)
            att.step(*qkv_g, refresh=True)
            torch.cuda.synchronize()
            a_s, y_s, _ = oracle.mlp_dense(x_s, w1t, None, w2, None, a_s)
            assert oracle.rel_frobenius(mlp.y[rows_t].cpu().numpy(), y_s) < TOL, "dense y"
            for (hh, b) in slices:
                r0, r1 = b * RB, min(n, (b + 1) * RB)
                q = oracle.from_bf16_bits(walks[0][t][hh, r0:r1])
                kx = oracle.from_bf16_bits(walks[1][t][hh])
                vx = oracle.from_bf16_bits(walks[2][t][hh])
                m, _, _, _, _ = oracle.attn_dense(q, kx, vx, SCALE)
                g_idx = att.idx[hh * nb + b].cpu().numpy()[None]
                nr, dr = oracle.attn_rest(q, kx, vx, m, g_idx, SCALE)
                state[(hh, b)] = (m, nr, dr, g_idx)
            continue
        y_prev = mlp.y[rows_t].cpu().numpy()
        sparse_step(mlp, att, x_g, *qkv_g)
        o_s_only = attn_s_only(gpu_lib, att, *qkv_g)
        torch.cuda.synchronize()
        del qkv_g
        g_idx = mlp.idx[torch.tensor(blocks, device="cuda")].cpu().numpy()
        g_score = mlp.score[torch.tensor(blocks, device="cuda")].cpu().numpy()
        np.testing.assert_array_equal(g_idx, oracle.identify_topk(g_score, k))
        y_old = y_s
        a_s, y_s = oracle.mlp_sparse(x_s, w1t, None, w2, a_s, y_s, g_idx)
        y_g = mlp.y[rows_t].cpu().numpy()
        # bars per sampled row block and per (block, 256 columns) tile, on y and
        # on the step's change of y
        e_y, i, c = worst_block_error(y_g, y_s, block_sizes(blocks, n), 256)
        assert e_y < TOL, f"step {t}: y {e_y:.2e} in block {blocks[i]} column group {c}"
        e_dy, i, c = worst_block_error(y_g - y_prev, y_s - y_old, block_sizes(blocks, n), 256)
        assert e_dy < TOL, f"step {t}: delta of y {e_dy:.2e} in block {blocks[i]} column group {c}"
        assert oracle.rel_frobenius(_cache_rows(mlp.a_cache, blocks, n), a_s) < 1e-3, f"step {t}: cache"
        for (hh, b) in slices:
            r0, r1 = b * RB, min(n, (b + 1) * RB)
            m, nr, dr, s_idx = state[(hh, b)]
            q = oracle.from_bf16_bits(walks[0][t][hh, r0:r1])
            kx = oracle.from_bf16_bits(walks[1][t][hh])
            vx = oracle.from_bf16_bits(walks[2][t][hh])
            o1 = oracle.attn_sparse(q, kx, vx, m, nr, dr, s_idx, SCALE)
            e = oracle.rel_frobenius(att.o[hh, r0:r1].cpu().numpy(), o1)
            assert e < TOL, f"step {t} head {hh} block {b}: o {e:.2e}"
            o_s = oracle.attn_sparse(q, kx, vx, m, np.zeros_like(nr), np.zeros_like(dr), s_idx, SCALE)
            e_s = oracle.rel_frobenius(o_s_only[hh, r0:r1].cpu().numpy(), o_s)
            assert e_s < TOL, f"step {t} head {hh} block {b}: o over S alone {e_s:.2e}"
        print(f"  step {t}: MLP worst block/tile rel-F y {e_y:.2e}, delta {e_dy:.2e}; attention slices ok",
              flush=True)
