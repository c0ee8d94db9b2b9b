"""GPU parity at the full workload sizes, in the launch configuration the bench times.

The kernels run on whole tensors of the real shapes.  The oracle recomputes
sampled row blocks (MLP) or sampled (head, query block) slices (attention), one
at a time.  That is exact, not an approximation: every MLP row block and every
attention (head, query block) depends only on its own rows and the shared
weights or keys, so a sampled block's state follows from that block alone.

Index sets:
  * the GPU's top-k must equal the oracle's top-k of the GPU's own fp32 score
    bits (bit-exact);
  * against the oracle's top-k of the oracle's own scores, the two may differ
    only between near-tied columns (the scores are sums in different orders).
The oracle then continues with the GPU's index sets, so both sides stay in
lockstep through the loop.

Bars: relative Frobenius error <= 2e-2 on every step's output rows and on the
step's change of them; scores within 1e-3.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from tests.gpu_helpers import bf16_values, idx_sets_valid, up_bf16

pytestmark = pytest.mark.gpu
TOL = 2e-2
SCALE = 1.0 / np.sqrt(128.0)
RB = 128


def _rows_of(blocks, n):
    return np.concatenate([np.arange(b * RB, min(n, (b + 1) * RB)) for b in blocks])


def _sample_blocks(nb, count, seed, n):
    """`count` seeded full blocks, ascending, then the last block if it is partial."""
    full = nb if n % RB == 0 else nb - 1
    g = np.random.default_rng(seed)
    pick = sorted(g.choice(full, size=min(count, full), replace=False).tolist())
    if full < nb:
        pick.append(nb - 1)
    return pick


def _cache_rows(a_cache, blocks, n):
    """Sampled blocks of the [nb][h][128] cache as [rows, h] float64 values."""
    sel = a_cache[torch.tensor(blocks, device=a_cache.device)]
    v = bf16_values(sel).reshape(len(blocks), -1, RB).transpose(0, 2, 1)
    return np.concatenate([v[i][: min(n, (b + 1) * RB) - b * RB] for i, b in enumerate(blocks)], axis=0)


# -------------------------------------------------------------------- MLP ---
def _mlp_loop(L, n, d, h, k, steps, dense_every, nsample, seed=0, fp8=False):
    # fp8: both products on fp8 operands; the oracle runs on the values those
    # operands carry (fp8_rows of x and W1^T; fp8_cols of W2 and fp8 blocks of
    # D in the sparse steps).
    from dynamic_column_sparse_amd.layers import MLPDelta
    nb = (n + RB - 1) // RB
    blocks = _sample_blocks(nb, nsample, seed + 11, n)
    rows = _rows_of(blocks, n)
    rows_t = torch.from_numpy(rows).cuda()
    print(f"mlp full size n={n} d={d} h={h} k={k} steps={steps} sampled blocks={len(blocks)} fp8={fp8}", flush=True)

    w1t_b, w2_b = syn.mlp_weights(seed, d, h)
    lay = MLPDelta(up_bf16(w1t_b), up_bf16(w2_b), n, k, **(dict(fp8=True, fp8_w2=True) if fp8 else {}))
    w1t, w2 = oracle.from_bf16_bits(w1t_b), oracle.from_bf16_bits(w2_b)
    del w1t_b, w2_b
    w2_sparse = w2
    if fp8:
        w1t = oracle.fp8_rows(w1t)
        w2_sparse = oracle.fp8_cols(w2)
    xs = syn.activation_walk(seed, "X", steps, n, d)

    a_s = np.zeros((len(rows), h))
    y_s = None
    sc_s = None
    for t in range(steps):
        x_g = up_bf16(xs[t])
        x_s = oracle.from_bf16_bits(xs[t][rows])
        if fp8:
            x_s = oracle.fp8_rows(x_s)
        if t % dense_every == 0:
            lay.dense(x_g)
            torch.cuda.synchronize()
            a_s, y_s, sc_s = oracle.mlp_dense(x_s, w1t, None, w2, None, a_s)
            g_score = lay.score[torch.tensor(blocks, device="cuda")].cpu().numpy()
            assert oracle.rel_frobenius(g_score, sc_s) < 1e-3, f"step {t}: score"
            assert oracle.rel_frobenius(lay.y[rows_t].cpu().numpy(), y_s) < TOL, f"step {t}: dense y"
            assert oracle.rel_frobenius(_cache_rows(lay.a_cache, blocks, n), a_s) < 1e-3, f"step {t}: cache"
            print(f"  step {t}: dense ok", flush=True)
            continue
        y_prev = lay.y[rows_t].cpu().numpy()
        lay.identify()
        lay.sparse(x_g)
        torch.cuda.synchronize()
        bt = torch.tensor(blocks, device="cuda")
        g_idx = lay.idx[bt].cpu().numpy()
        g_score = lay.score[bt].cpu().numpy()
        np.testing.assert_array_equal(g_idx, oracle.identify_topk(g_score, k))
        jac = idx_sets_valid(g_idx, oracle.identify_topk(sc_s.astype(np.float32), k), sc_s.astype(np.float32))
        y_old = y_s
        a_s, y_s = oracle.mlp_sparse(x_s, w1t, None, w2_sparse, a_s, y_s, g_idx, d_fp8=fp8)
        y_g = lay.y[rows_t].cpu().numpy()
        e_y = oracle.rel_frobenius(y_g, y_s)
        e_dy = oracle.rel_frobenius(y_g - y_prev, y_s - y_old)
        assert e_y < TOL and e_dy < TOL, f"step {t}: y {e_y:.2e}, delta {e_dy:.2e}"
        assert oracle.rel_frobenius(_cache_rows(lay.a_cache, blocks, n), a_s) < 1e-3, f"step {t}: cache"
        print(f"  step {t}: sparse ok (rel-F y {e_y:.2e}, delta {e_dy:.2e}, index Jaccard {jac:.4f})", flush=True)


def test_flux_mlp_ten_step_loop(gpu_lib):
    # FLUX.1-dev shape: 4352 tokens, d 3072, h 12288, keep 3686 per block; dense
    # at step 0, sparse steps 1..9.
    _mlp_loop(gpu_lib, 4352, 3072, 12288, 3686, steps=10, dense_every=10, nsample=3)


def test_hunyuan_mlp_sampled(gpu_lib):
    # HunyuanVideo shape: 118800 tokens (last block 16 rows), keep 860 per block;
    # the first three steps of the loop (dense, then sparse); the oracle follows
    # 32 seeded blocks (4096 rows) plus the 16-row tail block.
    _mlp_loop(gpu_lib, 118800, 3072, 12288, 860, steps=3, dense_every=10, nsample=32)


def test_hunyuan_mlp_fp8_sampled(gpu_lib):
    # The same shape with both products on fp8 operands (16 seeded blocks and
    # the 16-row tail block).
    _mlp_loop(gpu_lib, 118800, 3072, 12288, 860, steps=3, dense_every=10, nsample=16, fp8=True)


# -------------------------------------------------------------- attention ---
def _attn_loop(L, n, H, kk, steps, dense_at, slices, seed=0):
    from dynamic_column_sparse_amd.layers import AttnDelta
    nb = (n + RB - 1) // RB
    print(f"attention full size n={n} H={H} kk={kk} steps={steps} slices={slices}", flush=True)
    walks = [syn.heads_walk(seed, tag, steps, H, n) for tag in "QKV"]
    att = AttnDelta(n, H, kk, "cuda")
    state = {}
    for t in range(steps):
        g = [up_bf16(w[t]) for w in walks]
        refresh = t in dense_at
        att.step(*g, refresh=refresh)
        torch.cuda.synchronize()
        del g
        for (hh, b) in slices:
            r0, r1 = b * RB, min(n, (b + 1) * RB)
            q = oracle.from_bf16_bits(walks[0][t][hh, r0:r1])
            kx = oracle.from_bf16_bits(walks[1][t][hh])
            vx = oracle.from_bf16_bits(walks[2][t][hh])
            if refresh:
                m, den, num, o, score = oracle.attn_dense(q, kx, vx, SCALE)
                np.testing.assert_allclose(att.m[hh, r0:r1].cpu().numpy(), m, rtol=1e-5, atol=1e-5)
                assert oracle.rel_frobenius(att.o[hh, r0:r1].cpu().numpy(), o) < TOL, f"step {t}: dense o"
                g_score = att.score[hh, b].cpu().numpy()[None]
                assert oracle.rel_frobenius(g_score, score) < 1e-3, f"step {t}: score"
                g_idx = att.idx[hh * nb + b].cpu().numpy()[None]
                np.testing.assert_array_equal(g_idx, oracle.identify_topk(g_score, kk))
                jac = idx_sets_valid(g_idx, oracle.identify_topk(score.astype(np.float32), kk), score.astype(np.float32))
                nr, dr = oracle.attn_rest(q, kx, vx, m, g_idx, SCALE)
                assert oracle.rel_frobenius(att.num[hh, r0:r1].cpu().numpy(), nr) < TOL, f"step {t}: num_rest"
                assert oracle.rel_frobenius(att.den[hh, r0:r1].cpu().numpy(), dr) < 1e-3, f"step {t}: den_rest"
                state[(hh, b)] = (m, nr, dr, g_idx)
                print(f"  step {t} head {hh} block {b}: refresh ok (index Jaccard {jac:.4f})", flush=True)
            else:
                m, nr, dr, g_idx = state[(hh, b)]
                o1 = oracle.attn_sparse(q, kx, vx, m, nr, dr, g_idx, SCALE)
                e = oracle.rel_frobenius(att.o[hh, r0:r1].cpu().numpy(), o1)
                assert e < TOL, f"step {t} head {hh} block {b}: o {e:.2e}"
                print(f"  step {t} head {hh} block {b}: sparse ok (rel-F {e:.2e})", flush=True)


def test_flux_attention_ten_step_loop(gpu_lib):
    # FLUX.1-dev shape: 4352 tokens, 24 heads x 128, keep 718 keys per query
    # block; refresh at step 0, sparse steps 1..9.
    g = np.random.default_rng(21)
    slices = [(int(g.integers(24)), int(g.integers(34))) for _ in range(3)] + [(23, 33)]
    _attn_loop(gpu_lib, 4352, 24, 718, steps=10, dense_at={0}, slices=slices)


def test_hunyuan_attention_sampled(gpu_lib):
    # HunyuanVideo shape: 118800 tokens (last block 16 rows), 24 heads, keep 8316
    # keys per query block; the refresh step and the first sparse step, checked on
    # 2 seeded query blocks x 2 seeded heads plus one head's 16-row tail block.
    g = np.random.default_rng(31)
    heads = sorted(g.choice(24, size=2, replace=False).tolist())
    blocks = sorted(g.choice(928, size=2, replace=False).tolist())
    slices = [(hh, b) for hh in heads for b in blocks] + [(heads[0], 928)]
    _attn_loop(gpu_lib, 118800, 24, 8316, steps=2, dense_at={0}, slices=slices)
