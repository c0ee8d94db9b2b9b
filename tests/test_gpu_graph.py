"""A sparse step captured as a HIP graph and replayed gives the same bits as the
same step run eagerly.

Two identical layers start from the same refresh.  One steps eagerly, the other
replays a captured graph of the same calls.  Unrelated eager work and
synchronizations sit between the replays.  After every step the two states must
be bit-identical.  The kernels are deterministic, so any difference would come
from the capture."""
import numpy as np
import pytest
import torch

import synthetic as syn
from tests.gpu_helpers import up_bf16

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


@pytest.mark.parametrize("mode", ["bf16", "fp8", "reident"])
def test_sparse_step_graph_replay_matches_eager(gpu_lib, mode):
    # bf16: the default layers; fp8: both MLP products on fp8 (the quantize
    # kernel of x runs inside the graph); reident: attention identifying its
    # keys every step (the previous step's q, k, v are baked into each captured
    # step, so the eager side is given the same ones).
    from dynamic_column_sparse_amd.layers import AttnDelta, MLPDelta
    print(f"graph replay {mode}", flush=True)
    n, d, h, k, H, kk = 300, 256, 640, 200, 2, 100
    w1t_b, w2_b = syn.mlp_weights(1, d, h)
    xs = [up_bf16(x) for x in syn.activation_walk(1, "X", 4, n, d)]
    qkv = [[up_bf16(a) for a in step] for step in zip(*[syn.heads_walk(1, t, 4, H, n) for t in "QKV"])]

    layers = []
    for _ in range(2):
        mlp = MLPDelta(up_bf16(w1t_b), up_bf16(w2_b), n, k, **(dict(fp8=True, fp8_w2=True) if mode == "fp8" else {}))
        att = AttnDelta(n, H, kk, "cuda", reident=mode == "reident")
        mlp.step(xs[0], refresh=True)
        att.step(*qkv[0], refresh=True)
        layers.append((mlp, att))
    torch.cuda.synchronize()
    (m_e, a_e), (m_g, a_g) = layers

    def step(mlp, att, t):
        if att.reident:
            att.prev = tuple(qkv[t - 1])
        mlp.step(xs[t], refresh=False)
        att.step(*qkv[t], refresh=False)

    graphs = {}
    side = torch.cuda.Stream()
    for t in (1, 2, 3):
        g = torch.cuda.CUDAGraph()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                step(m_g, a_g, t)
        torch.cuda.current_stream().wait_stream(side)
        graphs[t] = g
    torch.cuda.synchronize()
    # Capture records the launches without running them, so the captured
    # layer is still at its refresh state.
    assert torch.equal(_bits(m_g.y), _bits(m_e.y))

    scratch = torch.zeros(1 << 20, device="cuda")
    for rep in range(3):
        for t in (1, 2, 3):
            step(m_e, a_e, t)
            scratch.add_(1.0)                      # unrelated eager work between replays
            graphs[t].replay()
            torch.cuda.synchronize()
            for a, b in ((m_e.y, m_g.y), (m_e.a_cache, m_g.a_cache), (m_e.idx, m_g.idx), (a_e.o, a_g.o),
                         (a_e.num, a_g.num), (a_e.score, a_g.score), (a_e.idx, a_g.idx)):
                assert torch.equal(_bits(a) if a.dtype != torch.int32 else a, _bits(b) if b.dtype != torch.int32 else b), \
                    f"replay {rep} step {t}"
    assert float(scratch[0]) == 9.0
