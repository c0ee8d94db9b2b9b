"""Step caching on the GPU (reading R16): a cached step launches nothing and
leaves every output and cache bit for bit as the latest computed step left
them; the computed steps of a schedule with cached steps match the oracle's
schedule (the oracle follows the GPU's index sets, which are checked bit for
bit against the oracle's top-k of the GPU's scores).  Bars as elsewhere:
rel. Frobenius <= 2e-2 per row block on y and o."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from tests.gpu_helpers import up_bf16, worst_block_error

pytestmark = pytest.mark.gpu
TOL = 2e-2
SCALE = 1.0 / np.sqrt(128.0)
D, S, C = "dense", "sparse", "cached"


def _bits(t):
    return t.view(torch.int32) if t.dtype in (torch.float32, torch.int32) else t.view(torch.int16)


@pytest.mark.parametrize("n,d,h,k,H,kk,fused", [
    (300, 256, 640, 200, 2, 100, True),      # ragged blocks, shared-grid sparse steps
    (300, 256, 640, 200, 2, 100, False),     # separate calls
    (4352, 3072, 12288, 3686, 24, 718, True),   # FLUX.1-dev shape (sampled blocks / slices)
])
def test_schedule_with_cached_steps_matches_oracle(gpu_lib, n, d, h, k, H, kk, fused):
    from dynamic_column_sparse_amd.layers import AttnDelta, MLPDelta, schedule_step
    sched = [D, S, C, S, C, C, S, D, C, S]
    print(f"step caching n={n} d={d} h={h} k={k} H={H} kk={kk} fused={fused}: {sched}", flush=True)
    T = len(sched)
    nb = (n + 127) // 128
    blocks = [0, nb - 1] if n > 1000 else list(range(nb))
    rows = np.concatenate([np.arange(b * 128, min(n, b * 128 + 128)) for b in blocks])
    sizes = [min(n, b * 128 + 128) - b * 128 for b in blocks]
    heads_chk = [0, H - 1]
    w1t_b, w2_b = syn.mlp_weights(5, d, h)
    mlp = MLPDelta(up_bf16(w1t_b), up_bf16(w2_b), n, k)
    att = AttnDelta(n, H, kk, "cuda")
    w1t, w2 = oracle.from_bf16_bits(w1t_b), oracle.from_bf16_bits(w2_b)
    xw, qw, kw, vw = (syn.Walk(5, tag, hd, n, dim) for tag, hd, dim in
                      (("X", 1, d), ("Q", H, 128), ("K", H, 128), ("V", H, 128)))
    a_s = np.zeros((len(rows), h))
    y_s = score_s = None
    at_state = {}
    o_s = {}
    for t, kind in enumerate(sched):
        x_b, q_b, k_b, v_b = xw.advance()[0], qw.advance(), kw.advance(), vw.advance()
        before = [getattr(mlp, nm).clone() for nm in mlp.STATE] + [getattr(att, nm).clone() for nm in att.STATE]
        schedule_step(kind, mlp, att, up_bf16(x_b), up_bf16(q_b), up_bf16(k_b), up_bf16(v_b), fused=fused)
        torch.cuda.synchronize()
        if kind == C:
            after = [getattr(mlp, nm) for nm in mlp.STATE] + [getattr(att, nm) for nm in att.STATE]
            for i, (a_, b_) in enumerate(zip(before, after)):
                assert torch.equal(_bits(a_), _bits(b_)), f"step {t}: cached step changed buffer {i}"
            continue
        x_s = oracle.from_bf16_bits(x_b[rows])
        if kind == D:
            a_s, y_s, score_s = oracle.mlp_dense(x_s, w1t, None, w2, None, a_s)
        else:
            g_idx = mlp.idx[torch.tensor(blocks, device="cuda")].cpu().numpy()
            g_score = mlp.score[torch.tensor(blocks, device="cuda")].cpu().numpy()
            np.testing.assert_array_equal(g_idx, oracle.identify_topk(g_score, k))
            a_s, y_s = oracle.mlp_sparse(x_s, w1t, None, w2, a_s, y_s, g_idx)
        e, i, c = worst_block_error(mlp.y[torch.from_numpy(rows).cuda()].cpu().numpy(), y_s, sizes, 256)
        assert e < TOL, f"step {t} ({kind}): y rel-F {e:.2e} in block {blocks[i]} column group {c}"
        for hh in heads_chk:
            qh, kh, vh = (oracle.from_bf16_bits(a[hh]) for a in (q_b, k_b, v_b))
            for b in blocks:
                r0, r1 = b * 128, min(n, b * 128 + 128)
                if kind == D:
                    m, _, _, o, _ = oracle.attn_dense(qh[r0:r1], kh, vh, SCALE)
                    g_idx = att.idx[hh * nb + b].cpu().numpy()[None]
                    nr, dr = oracle.attn_rest(qh[r0:r1], kh, vh, m, g_idx, SCALE)
                    at_state[(hh, b)] = (m, nr, dr, g_idx)
                else:
                    m, nr, dr, g_idx = at_state[(hh, b)]
                    o = oracle.attn_sparse(qh[r0:r1], kh, vh, m, nr, dr, g_idx, SCALE)
                e = oracle.rel_frobenius(att.o[hh, r0:r1].cpu().numpy(), o)
                assert e < TOL, f"step {t} ({kind}): o head {hh} block {b} rel-F {e:.2e}"
        print(f"  step {t} ({kind}) ok", flush=True)
