"""Layer state across a checkpoint and after a corrupted cache.

  * Checkpoint / resume: the cached state of an MLP and an attention layer is
    saved after a refresh and two sparse steps, written to a file, read back
    (torch.load with weights_only=True) into new layers, and both the original
    and the resumed layers run two more sparse steps and a refresh: every
    buffer must agree bit for bit.
  * Corrupted caches: the activation cache, output cache, scores and the
    attention numerator / denominator filled with garbage (NaN and huge
    values).  A refresh rewrites y, the activation cache and all attention
    state from the inputs alone, bit-identical to a new layer's refresh; the
    MLP scores compare the new activations with the old (corrupted) cache, so
    reset() first (zero caches, as a new layer) makes every following step,
    scores and index sets included, bit-identical to a new layer's.
"""
import os
import tempfile

import numpy as np
import pytest
import torch

import synthetic as syn
from tests.gpu_helpers import up_bf16

pytestmark = pytest.mark.gpu


def _bits(t):
    if t.dtype in (torch.float32, torch.int32):
        return t.view(torch.int32)
    return t.view(torch.int16)


def _equal(a_layer, b_layer, what):
    for name in a_layer.STATE:
        a, b = getattr(a_layer, name), getattr(b_layer, name)
        assert torch.equal(_bits(a), _bits(b)), f"{what}: {name}"


def _layers(n, d, h, k, na, H, kk, seed):
    from dynamic_column_sparse_amd.layers import AttnDelta, MLPDelta
    w1t_b, w2_b = syn.mlp_weights(seed, d, h)
    w1t, w2 = up_bf16(w1t_b), up_bf16(w2_b)

    def make():
        return MLPDelta(w1t, w2, n, k), AttnDelta(na, H, kk, "cuda")
    return make


def _inputs(n, d, na, H, steps, seed):
    xs = [up_bf16(x) for x in syn.activation_walk(seed, "X", steps, n, d)]
    qkv = [[up_bf16(a) for a in st] for st in zip(*[syn.heads_walk(seed, t, steps, H, na) for t in "QKV"])]
    return xs, qkv


def test_checkpoint_resume_is_bit_identical(gpu_lib):
    from dynamic_column_sparse_amd.layers import sparse_step
    n, d, h, k, na, H, kk = 1000, 384, 1024, 300, 1000, 8, 300
    print(f"checkpoint/resume n={n} d={d} h={h} k={k} H={H} kk={kk}", flush=True)
    make = _layers(n, d, h, k, na, H, kk, seed=13)
    xs, qkv = _inputs(n, d, na, H, 6, seed=13)
    mlp, att = make()
    mlp.step(xs[0], refresh=True)
    att.step(*qkv[0], refresh=True)
    for t in (1, 2):
        sparse_step(mlp, att, xs[t], *qkv[t])
    torch.cuda.synchronize()
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "state.pt")
        torch.save({"mlp": mlp.state_dict(), "attn": att.state_dict()}, path)
        state = torch.load(path, weights_only=True)
    mlp2, att2 = make()
    mlp2.load_state_dict(state["mlp"])
    att2.load_state_dict(state["attn"])
    torch.cuda.synchronize()
    _equal(mlp, mlp2, "restored MLP")
    _equal(att, att2, "restored attention")
    for t in (3, 4):
        sparse_step(mlp, att, xs[t], *qkv[t])
        sparse_step(mlp2, att2, xs[t], *qkv[t])
        torch.cuda.synchronize()
        _equal(mlp, mlp2, f"MLP step {t}")
        _equal(att, att2, f"attention step {t}")
    for m_, a_ in ((mlp, att), (mlp2, att2)):
        m_.step(xs[5], refresh=True)
        a_.step(*qkv[5], refresh=True)
    torch.cuda.synchronize()
    _equal(mlp, mlp2, "MLP refresh after resume")
    _equal(att, att2, "attention refresh after resume")


def test_refresh_recovers_from_corrupted_caches(gpu_lib):
    from dynamic_column_sparse_amd.layers import sparse_step
    n, d, h, k, na, H, kk = 300, 256, 640, 200, 300, 2, 100
    print(f"corrupted caches n={n} d={d} h={h} k={k} H={H} kk={kk}", flush=True)
    make = _layers(n, d, h, k, na, H, kk, seed=17)
    xs, qkv = _inputs(n, d, na, H, 4, seed=17)
    fresh_m, fresh_a = make()
    bad_m, bad_a = make()
    # a few steps, then garbage in every cache
    bad_m.step(xs[0], refresh=True)
    bad_a.step(*qkv[0], refresh=True)
    sparse_step(bad_m, bad_a, xs[1], *qkv[1])
    g = torch.Generator(device="cpu").manual_seed(5)
    for t in (bad_m.a_cache, bad_m.y, bad_m.score, bad_a.num, bad_a.den, bad_a.m, bad_a.score, bad_a.o):
        junk = torch.randint(-2**15, 2**15, t.shape, generator=g, dtype=torch.int32)
        if t.dtype == torch.bfloat16:
            t.view(torch.int16).copy_(junk.to(torch.int16))
        else:
            t.view(torch.int32).copy_(junk * 65536 + 0x7fc0)     # NaNs and large values
    assert not torch.isfinite(bad_m.a_cache.float()).all()
    # refresh alone: everything written from the inputs is clean
    fresh_m.step(xs[2], refresh=True)
    fresh_a.step(*qkv[2], refresh=True)
    bad_m.step(xs[2], refresh=True)
    bad_a.step(*qkv[2], refresh=True)
    torch.cuda.synchronize()
    for name in ("a_cache", "y"):
        assert torch.equal(_bits(getattr(bad_m, name)), _bits(getattr(fresh_m, name))), f"refresh: {name}"
    _equal(bad_a, fresh_a, "attention refresh")
    # reset() and a refresh: identical to a new layer in every buffer and step
    fresh_m, fresh_a = make()
    bad_m.reset()
    bad_a.reset()
    for m_, a_ in ((fresh_m, fresh_a), (bad_m, bad_a)):
        m_.step(xs[2], refresh=True)
        a_.step(*qkv[2], refresh=True)
        sparse_step(m_, a_, xs[3], *qkv[3])
    torch.cuda.synchronize()
    _equal(bad_m, fresh_m, "MLP after reset")
    _equal(bad_a, fresh_a, "attention after reset")
    assert torch.isfinite(bad_m.y).all() and torch.isfinite(bad_a.o).all()


def test_loading_bad_index_sets_is_refused(gpu_lib):
    # A checkpoint whose index sets break the contract (a repeated unit, a key
    # past n) is refused when loaded, naming the first bad row.
    from dynamic_column_sparse_amd.layers import AttnDelta, MLPDelta
    n, d, h, k, H, kk = 300, 256, 640, 64, 2, 40
    w1t_b, w2_b = syn.mlp_weights(2, d, h)
    mlp = MLPDelta(up_bf16(w1t_b), up_bf16(w2_b), n, k)
    att = AttnDelta(n, H, kk, "cuda")
    x = up_bf16(syn.activations(2, "X", 0, n, d))
    qkv = [up_bf16(syn.heads_activations(2, t, 0, H, n)) for t in "QKV"]
    mlp.step(x, refresh=True)
    att.step(*qkv, refresh=True)
    torch.cuda.synchronize()
    sm, sa = mlp.state_dict(), att.state_dict()
    mlp.load_state_dict(sm)                       # a sound state loads
    att.load_state_dict(sa)
    bad_m = {key: v.clone() for key, v in sm.items()}
    bad_m["idx"][1, 5] = bad_m["idx"][1, 4]
    with pytest.raises(ValueError, match="row 1"):
        mlp.load_state_dict(bad_m)
    bad_a = {key: v.clone() for key, v in sa.items()}
    bad_a["idx"][4, kk - 1] = n
    bad_a["idx"][5, 0] = -3
    with pytest.raises(ValueError, match="2 of 6 rows.*row 4"):
        att.load_state_dict(bad_a)
