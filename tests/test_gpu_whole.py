"""chipmunk_sparse_step_whole: the MLP's identification and both sparse deltas
in one launch.

  * Against the separate calls (chipmunk_identify_topk, then
    chipmunk_sparse_mlp_delta and chipmunk_sparse_attn_delta): bit-identical
    y, cache, index sets and o over several sparse steps.  The shapes cover
    ragged row blocks, both phase-1 tile widths, both phase-2 tile widths,
    head counts with and without the XCD head mapping, k = 0, kk = 0, k = h,
    and the longest identification row (h = 16384).
  * Against the oracle at a small shape over several steps (index sets
    bit-exact on the layer's own scores, y and o within rel. Frobenius 2e-2,
    the cache within 1e-3).
  * After every call the sync block is zero again and its status word is 0
    (no wait between work items gave up).
  * At the FLUX.1-dev shape (1280x768), in the launch configuration the
    benchmark times: bit-identical to the shared-grid step.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from tests.gpu_helpers import cache_to_rows, up_bf16

pytestmark = pytest.mark.gpu

RB = 128
SCALE = 1.0 / np.sqrt(128.0)
TOL = 2e-2


def _bits(t):
    if t.dtype == torch.int32:
        return t
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def _layers(n, d, h, k, na, H, kk, seed, steps, copies=2):
    from dynamic_column_sparse_amd.layers import AttnDelta, MLPDelta
    w1t_b, w2_b = syn.mlp_weights(seed, d, h)
    xs = [up_bf16(x) for x in syn.activation_walk(seed, "X", steps, n, d)]
    qkv = [[up_bf16(a) for a in st] for st in zip(*[syn.heads_walk(seed, t, steps, H, na) for t in "QKV"])]
    layers = []
    for _ in range(copies):
        mlp = MLPDelta(up_bf16(w1t_b), up_bf16(w2_b), n, k)
        att = AttnDelta(na, H, kk, "cuda")
        mlp.step(xs[0], refresh=True)
        att.step(*qkv[0], refresh=True)
        layers.append((mlp, att))
    return layers, xs, qkv, (w1t_b, w2_b)


def _check_sync(mlp):
    from dynamic_column_sparse_amd import lib
    s = mlp.sync.cpu()
    assert int(s[lib.SYNC_STATUS_WORD]) == 0, "a wait between work items gave up"
    assert int(s.abs().sum()) == 0, "sync block not cleared"


@pytest.mark.parametrize("n,d,h,k,na,H,kk", [
    (300, 256, 640, 200, 300, 2, 100),       # ragged; 128-wide phase-1, 256-wide phase-2 tiles
    (1000, 384, 1024, 520, 1000, 8, 300),    # 128-wide phase-2 tiles (d % 256 != 0), XCD head mapping
    (600, 256, 2048, 1000, 600, 3, 200),     # 256-wide phase-1 tiles, 3 heads
    (300, 256, 640, 0, 517, 3, 64),          # k = 0: attention units only; other token count
    (517, 256, 512, 64, 300, 8, 0),          # kk = 0: o = num / den beside the MLP items
    (129, 128, 64, 64, 129, 1, 129),         # every unit and key kept
    (256, 128, 16384, 5000, 256, 1, 64),     # the longest identification row (64 scores per thread)
])
def test_whole_step_matches_separate_calls(gpu_lib, n, d, h, k, na, H, kk):
    from dynamic_column_sparse_amd.layers import sparse_step
    print(f"whole step vs separate calls n={n} d={d} h={h} k={k} na={na} H={H} kk={kk}", flush=True)
    steps = 4
    ((m_s, a_s), (m_w, a_w)), xs, qkv, _ = _layers(n, d, h, k, na, H, kk, 7, steps)
    torch.cuda.synchronize()
    for t in range(1, steps):
        m_s.step(xs[t], refresh=False)
        a_s.step(*qkv[t], refresh=False)
        sparse_step(m_w, a_w, xs[t], *qkv[t], whole=True)
        torch.cuda.synchronize()
        names = [("y", m_s.y, m_w.y), ("a_cache", m_s.a_cache, m_w.a_cache), ("o", a_s.o, a_w.o)]
        if k > 0:
            names.append(("idx", m_s.idx, m_w.idx))
        for name, a, b in names:
            assert torch.equal(_bits(a), _bits(b)), f"step {t}: {name}"
        _check_sync(m_w)
    assert torch.isfinite(a_w.o).all() and torch.isfinite(m_w.y).all()


def test_whole_step_against_oracle(gpu_lib):
    from dynamic_column_sparse_amd.layers import sparse_step
    n, d, h, k, H, kk, steps, seed = 400, 256, 1024, 300, 2, 120, 4, 3
    nb = (n + RB - 1) // RB
    print(f"whole step against the oracle n={n} d={d} h={h} k={k} H={H} kk={kk}", flush=True)
    ((mlp, att),), xs, qkv, (w1t_b, w2_b) = _layers(n, d, h, k, n, H, kk, seed, steps, copies=1)
    w1t, w2 = oracle.from_bf16_bits(w1t_b), oracle.from_bf16_bits(w2_b)
    xs_np = syn.activation_walk(seed, "X", steps, n, d)
    walks = [syn.heads_walk(seed, tag, steps, H, n) for tag in "QKV"]
    torch.cuda.synchronize()
    a_o = np.zeros((n, h))
    a_o, y_o, _ = oracle.mlp_dense(oracle.from_bf16_bits(xs_np[0]), w1t, None, w2, None, a_o)
    state = {}
    for hh in range(H):
        q = oracle.from_bf16_bits(walks[0][0][hh])
        kx = oracle.from_bf16_bits(walks[1][0][hh])
        vx = oracle.from_bf16_bits(walks[2][0][hh])
        for b in range(nb):
            r0, r1 = b * RB, min(n, (b + 1) * RB)
            m, _, _, _, _ = oracle.attn_dense(q[r0:r1], kx, vx, SCALE)
            g_idx = att.idx[hh * nb + b].cpu().numpy()[None]
            nr, dr = oracle.attn_rest(q[r0:r1], kx, vx, m, g_idx, SCALE)
            state[(hh, b)] = (m, nr, dr, g_idx)
    for t in range(1, steps):
        sparse_step(mlp, att, xs[t], *qkv[t], whole=True)
        torch.cuda.synchronize()
        _check_sync(mlp)
        g_idx = mlp.idx.cpu().numpy()
        np.testing.assert_array_equal(g_idx, oracle.identify_topk(mlp.score.cpu().numpy(), k))
        a_o, y_o = oracle.mlp_sparse(oracle.from_bf16_bits(xs_np[t]), w1t, None, w2, a_o, y_o, g_idx)
        e_y = oracle.rel_frobenius(mlp.y.cpu().numpy(), y_o)
        assert e_y < TOL, f"step {t}: y {e_y:.2e}"
        assert oracle.rel_frobenius(cache_to_rows(mlp.a_cache, n), a_o) < 1e-3, f"step {t}: cache"
        for (hh, b), (m, nr, dr, s_idx) in state.items():
            r0, r1 = b * RB, min(n, (b + 1) * RB)
            q = oracle.from_bf16_bits(walks[0][t][hh, r0:r1])
            kx = oracle.from_bf16_bits(walks[1][t][hh])
            vx = oracle.from_bf16_bits(walks[2][t][hh])
            o1 = oracle.attn_sparse(q, kx, vx, m, nr, dr, s_idx, SCALE)
            e = oracle.rel_frobenius(att.o[hh, r0:r1].cpu().numpy(), o1)
            assert e < TOL, f"step {t} head {hh} block {b}: o {e:.2e}"
        print(f"  step {t}: y rel-F {e_y:.2e}", flush=True)


def test_flux_whole_step_matches_shared_grid(gpu_lib):
    # FLUX.1-dev at 1280x768: 4352 tokens, MLP 3072 -> 12288 keeping 3686 units
    # per block, 24 heads keeping 718 keys per query block.
    from dynamic_column_sparse_amd.layers import sparse_step
    n, d, h, k, H, kk, steps = 4352, 3072, 12288, 3686, 24, 718, 3
    print(f"flux whole step vs shared grid n={n}", flush=True)
    ((m_s, a_s), (m_w, a_w)), xs, qkv, _ = _layers(n, d, h, k, n, H, kk, 0, steps)
    torch.cuda.synchronize()
    for t in range(1, steps):
        sparse_step(m_s, a_s, xs[t], *qkv[t])
        sparse_step(m_w, a_w, xs[t], *qkv[t], whole=True)
        torch.cuda.synchronize()
        for name, a, b in (("y", m_s.y, m_w.y), ("a_cache", m_s.a_cache, m_w.a_cache), ("idx", m_s.idx, m_w.idx),
                           ("o", a_s.o, a_w.o)):
            assert torch.equal(_bits(a), _bits(b)), f"step {t}: {name}"
        _check_sync(m_w)
