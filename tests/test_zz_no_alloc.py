"""chipmunk_sparse_mlp_delta_noalloc (the entry point for callers that cannot
allocate) against chipmunk_sparse_mlp_delta with a caller workspace: the same
kernels, so y, the activation cache and the packed activations must agree bit
for bit.  Two calls in a row on the library's scratch array, the second with
a smaller input (the array keeps the first call's contents)."""
import numpy as np
import pytest
import torch

import synthetic as syn
from tests.gpu_helpers import up_bf16

pytestmark = pytest.mark.gpu


def _pair(n, d, h, k, seed):
    from dynamic_column_sparse_amd.layers import MLPDelta
    w1t_b, w2_b = syn.mlp_weights(seed, d, h)
    xs = [up_bf16(x) for x in syn.activation_walk(seed, "X", 2, n, d)]
    lays = []
    for _ in range(2):
        lay = MLPDelta(up_bf16(w1t_b), up_bf16(w2_b), n, k)
        lay.dense(xs[0])
        lay.identify()
        lays.append(lay)
    return lays, xs[1]


def _same(a, b):
    return torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                       b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16))


@pytest.mark.parametrize("first,second", [
    # FLUX.1-dev 1280x768 (32.3 MB of D tiles), then a ragged small layer
    ((4352, 3072, 12288, 3686, False), (300, 256, 640, 200, True)),
])
def test_noalloc_matches_workspace_entry_point(gpu_lib, first, second):
    L = gpu_lib
    for i, (n, d, h, k, packed) in enumerate((first, second)):
        print(f"no-alloc call {i}: n={n} d={d} h={h} k={k} packed={packed}", flush=True)
        (ref, new), x = _pair(n, d, h, k, seed=7 + i)
        assert L.chipmunk_workspace_bytes(L.OP_SPARSE_MLP, n, d, h, k) <= L.NOALLOC_SCRATCH_BYTES
        pk_ref = pk_new = None
        if packed:
            pk_ref = torch.zeros(ref.nb, k, 128, dtype=torch.bfloat16, device="cuda")
            pk_new = torch.zeros_like(pk_ref)
        L.chipmunk_sparse_mlp_delta(ref.layer, x, ref.idx, k, ref.y, pk_ref, ref.ws)
        L.chipmunk_sparse_mlp_delta_noalloc(new.layer, x, new.idx, k, new.y, pk_new)
        torch.cuda.synchronize()
        assert _same(ref.y, new.y), f"call {i}: y"
        assert _same(ref.a_cache, new.a_cache), f"call {i}: a_cache"
        if packed:
            assert _same(pk_ref, pk_new), f"call {i}: packed activations"
        assert torch.isfinite(new.y).all()


def test_noalloc_refuses_oversize_before_launch(gpu_lib):
    # HunyuanVideo-sized D tiles exceed the scratch array: refused, y untouched.
    L = gpu_lib
    n, d, h, k = 118800, 256, 1024, 512
    need = L.chipmunk_workspace_bytes(L.OP_SPARSE_MLP, n, d, h, k)
    assert need > L.NOALLOC_SCRATCH_BYTES
    from dynamic_column_sparse_amd.layers import MLPDelta
    w1t_b, w2_b = syn.mlp_weights(3, d, h)
    lay = MLPDelta(up_bf16(w1t_b), up_bf16(w2_b), n, k)
    x = torch.zeros(n, d, dtype=torch.bfloat16, device="cuda")
    y0 = lay.y.clone()
    with pytest.raises(L.ChipmunkError) as e:
        L.chipmunk_sparse_mlp_delta_noalloc(lay.layer, x, lay.idx, k, lay.y)
    assert e.value.code == 5
    torch.cuda.synchronize()
    assert _same(lay.y, y0)
