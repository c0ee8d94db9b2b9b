"""Per-step rescoring of the MLP (CHIPMUNK_MLP_RESCORE, reading R12) on the GPU.

Every sparse step rewrites the scores of the units it recomputed with that
step's column L1 of D, so the next identification can pick a different S.
  * Against the oracle over several steps (small, FLUX.1-dev and HunyuanVideo
    shapes, the large ones on seeded blocks and the tail block): the GPU's index sets equal the
    oracle's top-k of the GPU's own score bits (bit-exact); the GPU's scores
    after each step equal the oracle's rescored scores within 1e-3 (rel.
    Frobenius; the sums run in a different order); y and the cache within the
    usual bars.  The oracle follows the GPU's index sets, so both stay in step.
  * S does change from step to step (the point of the mode).
  * The shared-grid call gives the same bits as the separate calls.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from tests.gpu_helpers import up_bf16
from tests.test_gpu_fullsize import RB, TOL, _cache_rows, _rows_of, _sample_blocks

pytestmark = pytest.mark.gpu


def _loop(n, d, h, k, steps, blocks=None, seed=3):
    from dynamic_column_sparse_amd.layers import MLPDelta
    nb = (n + RB - 1) // RB
    blocks = list(range(nb)) if blocks is None else blocks
    rows = _rows_of(blocks, n)
    rows_t = torch.from_numpy(rows).cuda()
    bt = torch.tensor(blocks, device="cuda")
    w1t_b, w2_b = syn.mlp_weights(seed, d, h)
    lay = MLPDelta(up_bf16(w1t_b), up_bf16(w2_b), n, k, rescore=True)
    w1t, w2 = oracle.from_bf16_bits(w1t_b), oracle.from_bf16_bits(w2_b)
    xs = syn.activation_walk(seed, "X", steps, n, d)
    a_s = np.zeros((len(rows), h))
    idx_prev = None
    changed = 0
    for t in range(steps):
        x_g = up_bf16(xs[t])
        x_s = oracle.from_bf16_bits(xs[t][rows])
        if t == 0:
            lay.dense(x_g)
            torch.cuda.synchronize()
            a_s, y_s, sc_s = oracle.mlp_dense(x_s, w1t, None, w2, None, a_s)
            continue
        g_sc_before = lay.score[bt].cpu().numpy()
        lay.identify()
        lay.sparse(x_g)
        torch.cuda.synchronize()
        g_idx = lay.idx[bt].cpu().numpy()
        # identification ranks exactly the GPU's score bits (rescored last step)
        np.testing.assert_array_equal(g_idx, oracle.identify_topk(g_sc_before, k))
        y_old = y_s
        a_s, y_s, sc_s = oracle.mlp_sparse(x_s, w1t, None, w2, a_s, y_s, g_idx, score=sc_s)
        g_sc = lay.score[bt].cpu().numpy()
        e_sc = oracle.rel_frobenius(g_sc, sc_s)
        e_y = oracle.rel_frobenius(lay.y[rows_t].cpu().numpy(), y_s)
        assert e_sc < 1e-3, f"step {t}: score {e_sc:.2e}"
        assert e_y < TOL, f"step {t}: y {e_y:.2e}"
        assert oracle.rel_frobenius(_cache_rows(lay.a_cache, blocks, n), a_s) < 1e-3, f"step {t}: cache"
        if idx_prev is not None:
            changed += int(np.any(idx_prev != g_idx))
        idx_prev = g_idx
        print(f"  step {t}: score rel-F {e_sc:.2e}, y rel-F {e_y:.2e}", flush=True)
    return changed


def test_rescore_small_matches_oracle(gpu_lib):
    # Ragged (300 rows: blocks of 128, 128, 44); S must move between steps.
    changed = _loop(300, 256, 640, 200, steps=5)
    assert changed >= 1


def test_rescore_flux_sampled(gpu_lib):
    # FLUX.1-dev MLP shape, 3 seeded blocks followed by the oracle.
    n = 4352
    blocks = _sample_blocks(34, 3, 17, n)
    _loop(n, 3072, 12288, 3686, steps=4, blocks=blocks, seed=0)


def test_rescore_shared_grid_matches_separate_calls(gpu_lib):
    from dynamic_column_sparse_amd.layers import AttnDelta, MLPDelta, sparse_step
    n, d, h, k, H, kk, steps = 300, 256, 640, 200, 2, 100, 4
    w1t_b, w2_b = syn.mlp_weights(5, d, h)
    xs = [up_bf16(x) for x in syn.activation_walk(5, "X", steps, n, d)]
    qkv = [[up_bf16(a) for a in st] for st in zip(*[syn.heads_walk(5, t, steps, H, n) for t in "QKV"])]
    pairs = []
    for _ in range(2):
        mlp = MLPDelta(up_bf16(w1t_b), up_bf16(w2_b), n, k, rescore=True)
        att = AttnDelta(n, H, kk, "cuda")
        mlp.step(xs[0], refresh=True)
        att.step(*qkv[0], refresh=True)
        pairs.append((mlp, att))
    (m_s, a_s), (m_f, a_f) = pairs
    for t in range(1, steps):
        m_s.step(xs[t], refresh=False)
        a_s.step(*qkv[t], refresh=False)
        sparse_step(m_f, a_f, xs[t], *qkv[t])
        torch.cuda.synchronize()
        for name, a, b in (("y", m_s.y, m_f.y), ("score", m_s.score, m_f.score), ("idx", m_s.idx, m_f.idx),
                           ("a_cache", m_s.a_cache.view(torch.int16), m_f.a_cache.view(torch.int16)),
                           ("o", a_s.o, a_f.o)):
            if a.dtype == torch.float32:
                a, b = a.view(torch.int32), b.view(torch.int32)
            assert torch.equal(a, b), f"step {t}: {name}"


def test_rescore_hunyuan_sampled(gpu_lib):
    # HunyuanVideo MLP shape (118 800 tokens, 16-row tail block, keep 860 of
    # 12 288 units), seeded blocks and the tail followed by the oracle.
    n = 118800
    blocks = _sample_blocks(929, 3, 41, n)
    _loop(n, 3072, 12288, 860, steps=3, blocks=blocks, seed=0)
