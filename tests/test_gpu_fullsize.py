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
step's change of them, applied to each sampled row block on its own (the
16-row tail block of 118 800 tokens included) and to each (row block, 256
columns) tile of the MLP output, so that a localized error is not averaged
away by the rest; scores within 1e-3.  The loops follow the workloads'
schedules: the HunyuanVideo MLP refreshes every 10 steps, so the refresh at
step 10 scores the new activations against a cache that nine sparse steps
have written; the HunyuanVideo attention refreshes at steps 0 and 9.  The
attention is also checked on the chosen keys alone: the part REFRESH takes
out of num and den, and the sparse call on zero rest caches (o = num_S / den_S),
where one missing or doubled key chunk moves the result by several percent.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from tests.gpu_helpers import attn_s_only, bf16_values, block_sizes, idx_sets_valid, up_bf16, worst_block_error

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
    sizes = block_sizes(blocks, n)
    rows = _rows_of(blocks, n)
    rows_t = torch.from_numpy(rows).cuda()
    bt = torch.tensor(blocks, device="cuda")
    print(f"mlp full size n={n} d={d} h={h} k={k} steps={steps} dense every {dense_every} "
          f"sampled blocks={len(blocks)} fp8={fp8}", flush=True)

    w1t_b, w2_b = syn.mlp_weights(seed, d, h)
    lay = MLPDelta(up_bf16(w1t_b), up_bf16(w2_b), n, k, **(dict(fp8=True, fp8_w2=True) if fp8 else {}))
    w1t, w2 = oracle.from_bf16_bits(w1t_b), oracle.from_bf16_bits(w2_b)
    del w1t_b, w2_b
    w2_sparse = w2
    if fp8:
        w1t = oracle.fp8_rows(w1t)
        w2_sparse = oracle.fp8_cols(w2)
    walk = syn.Walk(seed, "X", 1, n, d)

    def check(name, g, ref, t, col_group=256):
        e, i, c = worst_block_error(g, ref, sizes, col_group)
        assert e < TOL, f"step {t}: {name} rel-F {e:.2e} in sampled block {blocks[i]} column group {c}"
        return e

    a_s = np.zeros((len(rows), h))
    y_s = None
    sc_s = None
    refreshes_after_sparse = 0
    for t in range(steps):
        xb = walk.advance()[0]
        x_g = up_bf16(xb)
        x_s = oracle.from_bf16_bits(xb[rows])
        del xb
        if fp8:
            x_s = oracle.fp8_rows(x_s)
        y_prev = lay.y[rows_t].cpu().numpy() if y_s is not None else None
        if t % dense_every == 0:
            lay.dense(x_g)
            torch.cuda.synchronize()
            # the score compares the new activations with the cache as the
            # previous steps left it (zero before the first refresh)
            y_old = y_s
            a_s, y_s, sc_s = oracle.mlp_dense(x_s, w1t, None, w2, None, a_s)
            g_score = lay.score[bt].cpu().numpy()
            e_sc, i, _ = worst_block_error(g_score, sc_s, [1] * len(blocks))
            assert e_sc < 1e-3, f"step {t}: score of sampled block {blocks[i]} rel-F {e_sc:.2e}"
            y_g = lay.y[rows_t].cpu().numpy()
            e_y = check("dense y", y_g, y_s, t)
            if y_old is not None:
                check("dense step's change of y", y_g - y_prev, y_s - y_old, t)
                refreshes_after_sparse += 1
            assert oracle.rel_frobenius(_cache_rows(lay.a_cache, blocks, n), a_s) < 1e-3, f"step {t}: cache"
            print(f"  step {t}: dense ok (worst block rel-F y {e_y:.2e}, score {e_sc:.2e})", flush=True)
            continue
        lay.identify()
        lay.sparse(x_g)
        torch.cuda.synchronize()
        g_idx = lay.idx[bt].cpu().numpy()
        g_score = lay.score[bt].cpu().numpy()
        np.testing.assert_array_equal(g_idx, oracle.identify_topk(g_score, k))
        jac = idx_sets_valid(g_idx, oracle.identify_topk(sc_s.astype(np.float32), k), sc_s.astype(np.float32),
                             gpu_score=g_score)
        y_old = y_s
        a_s, y_s = oracle.mlp_sparse(x_s, w1t, None, w2_sparse, a_s, y_s, g_idx, d_fp8=fp8)
        y_g = lay.y[rows_t].cpu().numpy()
        e_y = check("y", y_g, y_s, t)
        e_dy = check("delta of y", y_g - y_prev, y_s - y_old, t)
        assert oracle.rel_frobenius(_cache_rows(lay.a_cache, blocks, n), a_s) < 1e-3, f"step {t}: cache"
        print(f"  step {t}: sparse ok (worst block/tile rel-F y {e_y:.2e}, delta {e_dy:.2e}, "
              f"index Jaccard {jac:.4f})", flush=True)
    return refreshes_after_sparse


def test_flux_mlp_ten_step_loop(gpu_lib):
    # FLUX.1-dev shape: 4352 tokens, d 3072, h 12288, keep 3686 per block; dense
    # at step 0, sparse steps 1..9.
    _mlp_loop(gpu_lib, 4352, 3072, 12288, 3686, steps=10, dense_every=10, nsample=3)


def test_flux_mlp_refresh_after_sparse_steps(gpu_lib):
    # The same shape with refreshes at steps 0, 4 and 8: both later refreshes
    # score and overwrite a cache that sparse steps have written.
    assert _mlp_loop(gpu_lib, 4352, 3072, 12288, 3686, steps=10, dense_every=4, nsample=3) == 2


def test_hunyuan_mlp_schedule(gpu_lib):
    # HunyuanVideo shape: 118800 tokens (last block 16 rows), keep 860 per block,
    # refresh every 10 steps: steps 0..11 of the 50-step loop (dense at 0 and
    # 10).  The oracle follows 32 seeded blocks (4096 rows) plus the 16-row tail
    # block; the step-10 refresh scores against the oracle's cache after step 9.
    assert _mlp_loop(gpu_lib, 118800, 3072, 12288, 860, steps=12, dense_every=10, nsample=32) == 1


def test_hunyuan_mlp_fp8_sampled(gpu_lib):
    # The same shape with both products on fp8 operands (16 seeded blocks and
    # the 16-row tail block).
    _mlp_loop(gpu_lib, 118800, 3072, 12288, 860, steps=3, dense_every=10, nsample=16, fp8=True)


# -------------------------------------------------------------- attention ---
def _attn_loop(L, n, H, kk, steps, dense_at, slices, seed=0):
    from dynamic_column_sparse_amd.layers import AttnDelta
    nb = (n + RB - 1) // RB
    print(f"attention full size n={n} H={H} kk={kk} steps={steps} dense at {sorted(dense_at)} slices={slices}",
          flush=True)
    walks = [syn.Walk(seed, tag, H, n, 128) for tag in "QKV"]
    att = AttnDelta(n, H, kk, "cuda")
    state = {}
    for t in range(steps):
        host = [w.advance() for w in walks]
        g = [up_bf16(a) for a in host]
        refresh = t in dense_at
        if refresh:
            att.dense(*g)
            att.identify()
            torch.cuda.synchronize()
            num_dense, den_dense = att.num.clone(), att.den.clone()
            att.refresh_rest(*g)
            torch.cuda.synchronize()
            o_s_only = None
        else:
            att.sparse(*g)
            o_s_only = attn_s_only(L, att, *g)
            torch.cuda.synchronize()
        del g
        for (hh, b) in slices:
            r0, r1 = b * RB, min(n, (b + 1) * RB)
            q = oracle.from_bf16_bits(host[0][hh, r0:r1])
            kx = oracle.from_bf16_bits(host[1][hh])
            vx = oracle.from_bf16_bits(host[2][hh])
            if refresh:
                m, den, num, o, score = oracle.attn_dense(q, kx, vx, SCALE)
                np.testing.assert_allclose(att.m[hh, r0:r1].cpu().numpy(), m, rtol=1e-5, atol=1e-5)
                assert oracle.rel_frobenius(att.o[hh, r0:r1].cpu().numpy(), o) < TOL, f"step {t}: dense o"
                g_score = att.score[hh, b].cpu().numpy()[None]
                assert oracle.rel_frobenius(g_score, score) < 1e-3, f"step {t}: score"
                g_idx = att.idx[hh * nb + b].cpu().numpy()[None]
                np.testing.assert_array_equal(g_idx, oracle.identify_topk(g_score, kk))
                jac = idx_sets_valid(g_idx, oracle.identify_topk(score.astype(np.float32), kk), score.astype(np.float32),
                                     gpu_score=g_score)
                nr, dr = oracle.attn_rest(q, kx, vx, m, g_idx, SCALE)
                num_g, den_g = att.num[hh, r0:r1].cpu().numpy(), att.den[hh, r0:r1].cpu().numpy()
                assert oracle.rel_frobenius(num_g, nr) < TOL, f"step {t}: num_rest"
                assert oracle.rel_frobenius(den_g, dr) < 1e-3, f"step {t}: den_rest"
                # the part REFRESH took out: the chosen keys' share alone
                num_s_g = num_dense[hh, r0:r1].cpu().numpy() - num_g
                den_s_g = den_dense[hh, r0:r1].cpu().numpy() - den_g
                e_num = oracle.rel_frobenius(num_s_g, num - nr)
                e_den = oracle.rel_frobenius(den_s_g, den - dr)
                assert e_num < TOL and e_den < 1e-3, f"step {t}: S part num {e_num:.2e} den {e_den:.2e}"
                state[(hh, b)] = (m, nr, dr, g_idx)
                print(f"  step {t} head {hh} block {b}: refresh ok (S part num {e_num:.2e}, den {e_den:.2e}; "
                      f"index Jaccard {jac:.4f})", flush=True)
            else:
                m, nr, dr, g_idx = state[(hh, b)]
                o1 = oracle.attn_sparse(q, kx, vx, m, nr, dr, g_idx, SCALE)
                e = oracle.rel_frobenius(att.o[hh, r0:r1].cpu().numpy(), o1)
                assert e < TOL, f"step {t} head {hh} block {b}: o {e:.2e}"
                z = np.zeros_like(nr)
                o_s = oracle.attn_sparse(q, kx, vx, m, z, np.zeros_like(dr), g_idx, SCALE)
                e_s = oracle.rel_frobenius(o_s_only[hh, r0:r1].cpu().numpy(), o_s)
                assert e_s < TOL, f"step {t} head {hh} block {b}: o over S alone {e_s:.2e}"
                print(f"  step {t} head {hh} block {b}: sparse ok (rel-F {e:.2e}, S alone {e_s:.2e})", flush=True)
        del host


def test_flux_attention_ten_step_loop(gpu_lib):
    # FLUX.1-dev shape: 4352 tokens, 24 heads x 128, keep 718 keys per query
    # block; refresh at step 0, sparse steps 1..9.
    g = np.random.default_rng(21)
    slices = [(int(g.integers(24)), int(g.integers(34))) for _ in range(3)] + [(23, 33)]
    _attn_loop(gpu_lib, 4352, 24, 718, steps=10, dense_at={0}, slices=slices)


def test_hunyuan_attention_schedule(gpu_lib):
    # HunyuanVideo shape: 118800 tokens (last block 16 rows), 24 heads, keep 8316
    # keys per query block; steps 0..10 of the 50-step loop whose dense steps
    # fall at t mod 9 = 0 (refresh at 0 and 9, sparse 1..8 and 10), checked on 2
    # seeded query blocks x 2 seeded heads plus one head's 16-row tail block.
    g = np.random.default_rng(31)
    heads = sorted(g.choice(24, size=2, replace=False).tolist())
    blocks = sorted(g.choice(928, size=2, replace=False).tolist())
    slices = [(hh, b) for hh in heads for b in blocks] + [(heads[0], 928)]
    _attn_loop(gpu_lib, 118800, 24, 8316, steps=11, dense_at={0, 9}, slices=slices)
