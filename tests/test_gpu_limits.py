"""GPU parity at the largest sizes the C-ABI accepts, through the C-ABI.

Attention: n = 2^24 - 1 tokens, the largest the header allows (gathered K and
V rows are addressed by 32-bit byte offsets from each head's base, so the key
n - 1 sits 512 bytes below 2^32).  Two heads, so the second head's base lies
beyond 4 GiB; 300 keys per query block (the id ring wraps); every index set
holds the 32 highest keys and 268 keys spread over the rest of the range; the
last query block has 127 rows.  The rest caches (m, num, den) are seeded
inputs: the sparse step reads them and nothing else of the refresh, so no
dense step (whose score array would take 2 x 131 072 x n floats) is needed.

MLP: 720 077 rows of d = 3072, so x and y hold more than 2^31 elements and the
sampled blocks past row 699 051 sit beyond 32-bit element offsets (and the
activation cache beyond 2^31 elements too); the last block has 77 rows.  One
refresh, then one sparse step on drifted inputs, as the workloads run.

Inputs are drawn on the device with seeded torch generators (the arrays are
too large to draw on the host); the oracle gets the sampled rows of those
inputs, never an output of the library.  Bars as in the full-size tests:
relative Frobenius error <= 2e-2 per sampled block (per 256-column tile for
the MLP output), scores within 1e-3, index sets bit-exact against the
oracle's top-k of the library's own scores.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from tests.gpu_helpers import bf16_values, block_sizes, idx_sets_valid, up_bf16, worst_block_error

pytestmark = pytest.mark.gpu
TOL = 2e-2
RB = 128
SCALE = 1.0 / np.sqrt(128.0)


def _randn_bf16(shape, gen):
    """A seeded bf16 device tensor, drawn one leading slice at a time."""
    out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    for i in range(shape[0]):
        out[i].copy_(torch.randn(shape[1:], device="cuda", generator=gen))
    return out


def _host(t):
    """bf16 device tensor -> float64 host values."""
    return bf16_values(t.contiguous())


def test_attention_at_the_largest_token_count(gpu_lib):
    n, H, kk = (1 << 24) - 1, 2, 300
    nb = (n + RB - 1) // RB
    top = 32
    print(f"attention limits: n={n} heads={H} kk={kk} blocks={nb} (last block {n - (nb - 1) * RB} rows)", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(41)
    q = _randn_bf16((H, n, 128), gen)
    k = _randn_bf16((H, n, 128), gen)
    v = _randn_bf16((H, n, 128), gen)
    # Index sets: 268 keys a + i * stride (a seeded per row), then the top 32.
    spread = kk - top
    stride = (n - top) // spread
    a0 = torch.randint(0, stride, (H * nb, 1), device="cuda", generator=gen, dtype=torch.int64)
    low = a0 + torch.arange(spread, device="cuda", dtype=torch.int64)[None] * stride
    high = torch.arange(n - top, n, device="cuda", dtype=torch.int64)[None].expand(H * nb, top)
    idx = torch.cat([low, high], dim=1).to(torch.int32).contiguous()
    del a0, low, high
    res = torch.empty(2, dtype=torch.int64, device="cuda")
    gpu_lib.chipmunk_check_index_sets(idx, H * nb, kk, n, res)
    # Rest caches as a refresh would leave them: m near the row maxima of these
    # scores, positive den, num of matching size.
    m = 3.0 + torch.rand(H, n, device="cuda", generator=gen)
    den = 5.0 + 10.0 * torch.rand(H, n, device="cuda", generator=gen)
    num = torch.empty(H, n, 128, device="cuda")
    for hh in range(H):
        num[hh].copy_(0.5 * torch.randn(n, 128, device="cuda", generator=gen))
    o = torch.empty(H, n, 128, device="cuda")
    layer = gpu_lib.attn_layer(n, H, m, num, den, None, SCALE)
    gpu_lib.chipmunk_sparse_attn_delta(layer, q, k, v, idx, kk, gpu_lib.ATTN_SPARSE, o)
    torch.cuda.synchronize()
    assert res.cpu().tolist() == [0, H * nb], "index sets break the contract"
    # The chosen keys alone: zero rest caches, o = num_S / den_S.
    o_s = torch.empty_like(o)
    num_z, den_z = torch.zeros_like(num), torch.zeros_like(den)
    layer_z = gpu_lib.attn_layer(n, H, m, num_z, den_z, None, SCALE)
    gpu_lib.chipmunk_sparse_attn_delta(layer_z, q, k, v, idx, kk, gpu_lib.ATTN_SPARSE, o_s)
    torch.cuda.synchronize()
    del num_z, den_z

    g = np.random.default_rng(43)
    slices = [(0, 0), (0, int(g.integers(nb - 1))), (1, int(g.integers(nb - 1))), (1, nb - 2), (0, nb - 1),
              (1, nb - 1)]
    for hh, b in slices:
        r0, r1 = b * RB, min(n, (b + 1) * RB)
        s = idx[hh * nb + b].long()
        assert int(s[-1]) == n - 1
        # The oracle sees the block's rows and the chosen keys' rows only; its
        # index set then names those rows in order.
        qs, ks, vs = _host(q[hh, r0:r1]), _host(k[hh, s]), _host(v[hh, s])
        ms, ns, ds = (m[hh, r0:r1].double().cpu().numpy(), num[hh, r0:r1].double().cpu().numpy(),
                      den[hh, r0:r1].double().cpu().numpy())
        local = [np.arange(kk)]
        ref = oracle.attn_sparse(qs, ks, vs, ms, ns, ds, local, SCALE)
        e = oracle.rel_frobenius(o[hh, r0:r1].cpu().numpy(), ref)
        ref_s = oracle.attn_sparse(qs, ks, vs, ms, np.zeros_like(ns), np.zeros_like(ds), local, SCALE)
        e_s = oracle.rel_frobenius(o_s[hh, r0:r1].cpu().numpy(), ref_s)
        print(f"  head {hh} block {b} ({r1 - r0} rows): o rel-F {e:.2e}, chosen keys alone {e_s:.2e}", flush=True)
        assert e < TOL and e_s < TOL, f"head {hh} block {b}: o {e:.2e}, S alone {e_s:.2e}"
    del q, k, v, idx, m, den, num, o, o_s
    torch.cuda.empty_cache()


def test_mlp_beyond_32_bit_element_offsets(gpu_lib):
    from dynamic_column_sparse_amd.layers import MLPDelta
    n, d, h, k = 720_077, 3072, 12288, 860
    nb = (n + RB - 1) // RB
    assert n * d > 2 ** 31 and nb * h * RB > 2 ** 31
    first_far = (2 ** 31 + d - 1) // d // RB + 1          # first block wholly past 2^31 elements of x
    g = np.random.default_rng(47)
    blocks = sorted({0, int(g.integers(1, first_far)), first_far, int(g.integers(first_far + 1, nb - 1)), nb - 1})
    sizes = block_sizes(blocks, n)
    rows = np.concatenate([np.arange(b * RB, min(n, (b + 1) * RB)) for b in blocks])
    rows_t = torch.from_numpy(rows).cuda()
    bt = torch.tensor(blocks, device="cuda")
    print(f"mlp limits: n={n} d={d} h={h} k={k} blocks={nb} (last block {n - (nb - 1) * RB} rows), "
          f"sampled {blocks}", flush=True)

    w1t_b, w2_b = syn.mlp_weights(5, d, h)
    lay = MLPDelta(up_bf16(w1t_b), up_bf16(w2_b), n, k)
    w1t, w2 = oracle.from_bf16_bits(w1t_b), oracle.from_bf16_bits(w2_b)
    del w1t_b, w2_b
    gen = torch.Generator(device="cuda").manual_seed(53)
    x0 = torch.empty(n, d, dtype=torch.bfloat16, device="cuda")
    x1 = torch.empty_like(x0)
    step = 1 << 16
    for r in range(0, n, step):
        e = min(n, r + step)
        w = torch.randn(e - r, d, device="cuda", generator=gen)
        x0[r:e].copy_(w)
        x1[r:e].copy_(w + 0.05 * torch.randn(e - r, d, device="cuda", generator=gen))
    del w

    def check(name, got, ref, col_group=256):
        err, i, c = worst_block_error(got, ref, sizes, col_group)
        assert err < TOL, f"{name} rel-F {err:.2e} in sampled block {blocks[i]} column group {c}"
        return err

    # Refresh, then its index sets.
    lay.step(x0, refresh=True)
    torch.cuda.synchronize()
    x_s = _host(x0[rows_t])
    a_s, y_s, sc_s = oracle.mlp_dense(x_s, w1t, None, w2, None, np.zeros((len(rows), h)))
    g_score = lay.score[bt].cpu().numpy()
    e_sc, i, _ = worst_block_error(g_score, sc_s, [1] * len(blocks))
    assert e_sc < 1e-3, f"score of sampled block {blocks[i]} rel-F {e_sc:.2e}"
    y_prev = lay.y[rows_t].cpu().numpy()
    e_y = check("dense y", y_prev, y_s)
    g_idx = lay.idx[bt].cpu().numpy()
    np.testing.assert_array_equal(g_idx, oracle.identify_topk(g_score, k))
    jac = idx_sets_valid(g_idx, oracle.identify_topk(sc_s.astype(np.float32), k), sc_s.astype(np.float32),
                         gpu_score=g_score)
    print(f"  refresh ok (worst block rel-F y {e_y:.2e}, score {e_sc:.2e}, index Jaccard {jac:.4f})", flush=True)

    # One sparse step on the drifted inputs.
    lay.step(x1, refresh=False)
    torch.cuda.synchronize()
    y_old = y_s
    a_s, y_s = oracle.mlp_sparse(_host(x1[rows_t]), w1t, None, w2, a_s, y_s, g_idx)
    y_g = lay.y[rows_t].cpu().numpy()
    e_y = check("y", y_g, y_s)
    e_dy = check("delta of y", y_g - y_prev, y_s - y_old)
    print(f"  sparse ok (worst block/tile rel-F y {e_y:.2e}, delta {e_dy:.2e})", flush=True)
    del lay, x0, x1
    torch.cuda.empty_cache()
