"""Per-layer device state for a sampler loop: buffers plus the order of C-ABI
calls.  Allocation and call sequencing only; every computation is a call into
``libchipmunk.so``.

Schedule per layer and diffusion step (the Chipmunk post, section "Activation
Deltas Across Diffusion Steps are Very Sparse": cache the value vectors and
their coefficients, then recompute a chosen subset each step):
  MLP        refresh: dense step (fills the activation cache, output cache and
             per-block column scores), then identify the top-k columns per
             block; sparse: the sparse delta with fused cache writeback.  The
             scores change only at a refresh, so the index sets are found once
             there; with rescore=True the sparse delta updates the scores of
             the units it recomputed, and each sparse step identifies first.
  attention  refresh: dense step (m, num, den, o, key-mass scores), identify the
             top-k keys per query block, then REFRESH (num, den keep only the
             part outside S); sparse: the sparse delta writes o.
             With reident=True: the refresh is the dense step alone (num, den
             keep totals); each sparse step identifies S from the latest
             scores, then swaps S's previous-step share for this step's and
             rescores S (chipmunk_sparse_attn_reident).
  cached     (step caching, stacked on the deltas in the post's Results
             section): nothing is recomputed and nothing is launched; the
             layer's output buffer keeps the latest computed output and every
             cache keeps its value.
"""
from __future__ import annotations

import math

import torch

from . import lib

ROW_BLOCK = lib.ROW_BLOCK


def row_blocks(n: int) -> int:
    return (n + ROW_BLOCK - 1) // ROW_BLOCK


def check_index_sets(idx: torch.Tensor, cols: int, what: str = "index sets"):
    """Raise ValueError unless every row of idx [rows][k] (int32, on the
    device) is strictly ascending with values in [0, cols): the contract the
    kernels assume (they clamp bad values rather than fault).  Synchronizes."""
    rows, k = idx.shape
    res = torch.empty(2, dtype=torch.int64, device=idx.device)
    lib.chipmunk_check_index_sets(idx, rows, k, cols, res)
    bad, first = res.tolist()
    if bad:
        raise ValueError(f"{what}: {bad} of {rows} rows are not ascending sets of [0, {cols}) (first: row {first})")


class MLPDelta:
    """One MLP layer: w1t [h,d], w2 [h,d] bf16 device tensors; k kept columns per block.
    rescore=True: every sparse step rescores the units it recomputed, so the set
    S can change from step to step (CHIPMUNK_MLP_RESCORE).
    fp8=True: the first product runs on fp8 operands (CHIPMUNK_MLP_FP8); W1^T is
    quantized once here, x by every call.  fp8_w2=True: the sparse delta's
    second product runs on fp8 operands too (CHIPMUNK_MLP_FP8_W2); W2 is
    quantized once here, column by column."""

    def __init__(self, w1t: torch.Tensor, w2: torch.Tensor, n: int, k: int, b1=None, b2=None, rescore=False,
                 fp8=False, fp8_w2=False):
        h, d = w1t.shape
        assert w2.shape == (h, d) and w1t.dtype == torch.bfloat16 and w2.dtype == torch.bfloat16
        dev = w1t.device
        self.n, self.d, self.h, self.k = n, d, h, k
        self.nb = row_blocks(n)
        self.w1t, self.w2, self.b1, self.b2 = w1t, w2, b1, b2
        self.a_cache = torch.zeros(self.nb, h, ROW_BLOCK, dtype=torch.bfloat16, device=dev)
        self.score = torch.zeros(self.nb, h, dtype=torch.float32, device=dev)
        self.y = torch.zeros(n, d, dtype=torch.float32, device=dev)
        self.idx = torch.zeros(self.nb, max(k, 1), dtype=torch.int32, device=dev)
        self.w1t_f8 = self.w1t_scale = None
        if fp8:
            self.w1t_f8 = torch.empty(h, d, dtype=torch.uint8, device=dev)
            self.w1t_scale = torch.empty(h, dtype=torch.uint8, device=dev)
            lib.chipmunk_quantize_fp8(w1t, h, d, self.w1t_f8, self.w1t_scale)
            ws = max(lib.chipmunk_workspace_bytes(lib.OP_SPARSE_MLP_FP8, n, d, h, k),
                     lib.chipmunk_workspace_bytes(lib.OP_DENSE_MLP_FP8, n, d, h, 0))
        else:
            ws = lib.chipmunk_workspace_bytes(lib.OP_SPARSE_MLP, n, d, h, k)
        self.ws = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)
        self.w2_f8 = self.w2_scale = None
        if fp8_w2:
            self.w2_f8 = torch.empty(h, d, dtype=torch.uint8, device=dev)
            self.w2_scale = torch.empty(d, dtype=torch.uint8, device=dev)
            lib.chipmunk_quantize_fp8_cols(w2, h, d, self.w2_f8, self.w2_scale)
        flags = ((lib.MLP_RESCORE if rescore else 0) | (lib.MLP_FP8 if fp8 else 0)
                 | (lib.MLP_FP8_W2 if fp8_w2 else 0))
        self.rescore = rescore
        self.layer = lib.mlp_layer(n, d, h, w1t, w2, self.a_cache, self.score, b1, b2, flags, self.w1t_f8,
                                   self.w1t_scale, self.w2_f8, self.w2_scale)
        # index sets of the (zero) scores, so that idx always holds valid sets
        self.identify()

    STATE = ("a_cache", "score", "y", "idx")

    def state_dict(self) -> dict:
        """The layer's cached state (activation cache, scores, output cache and
        the current index sets) as host tensors, for a checkpoint."""
        return {name: getattr(self, name).detach().cpu() for name in self.STATE}

    def load_state_dict(self, state: dict):
        """Restore a state_dict() of a layer of the same shape, in place (the C
        layer keeps pointing at the same buffers).  The index sets are checked
        on the device (ValueError if a row is not an ascending set of hidden
        units)."""
        for name in self.STATE:
            dst = getattr(self, name)
            src = state[name]
            assert src.shape == dst.shape and src.dtype == dst.dtype, name
            dst.copy_(src)
        if self.k:
            check_index_sets(self.idx, self.h, "MLP index sets")

    def reset(self):
        """Back to the state of a new layer: zero caches, so the next dense
        step scores its activations against zero, as the first one does."""
        for name in self.STATE:
            getattr(self, name).zero_()
        self.identify()

    def dense(self, x: torch.Tensor, stream=None):
        lib.chipmunk_dense_step(lib.MLP, self.layer, x, None, None, self.y, self.ws, stream=stream)

    def identify(self, stream=None):
        lib.chipmunk_identify_topk(self.score, self.nb, self.h, self.k, self.idx, stream=stream)

    def sparse(self, x: torch.Tensor, idx=None, a_new_packed=None, stream=None):
        lib.chipmunk_sparse_mlp_delta(self.layer, x, self.idx if idx is None else idx, self.k, self.y,
                                      a_new_packed, self.ws, stream=stream)

    def writeback(self, a_new_packed, idx=None, stream=None):
        lib.chipmunk_cache_writeback(self.layer, a_new_packed, self.idx if idx is None else idx, self.k,
                                     stream=stream)

    def step(self, x: torch.Tensor, refresh: bool, stream=None):
        if refresh:
            self.dense(x, stream)
            if not self.rescore:
                self.identify(stream)
        else:
            if self.rescore:
                self.identify(stream)
            self.sparse(x, stream=stream)


class AttnDelta:
    """One attention layer (all heads), head_dim 128; kk kept keys per query block.
    reident=True: S is identified anew at every sparse step; the layer then
    keeps references to the previous step's q, k, v, which the caller must
    leave unmodified until the next step."""

    def __init__(self, n: int, heads: int, kk: int, device, scale=None, reident=False):
        self.n, self.heads, self.kk = n, heads, kk
        self.reident = reident
        self.prev = None
        self.nb = row_blocks(n)
        self.scale = 1.0 / math.sqrt(lib.HEAD_DIM) if scale is None else scale
        f32 = dict(dtype=torch.float32, device=device)
        self.m = torch.zeros(heads, n, **f32)
        self.den = torch.zeros(heads, n, **f32)
        self.num = torch.zeros(heads, n, lib.HEAD_DIM, **f32)
        self.score = torch.zeros(heads, self.nb, n, **f32)
        self.o = torch.zeros(heads, n, lib.HEAD_DIM, **f32)
        self.idx = torch.zeros(heads * self.nb, max(kk, 1), dtype=torch.int32, device=device)
        self.layer = lib.attn_layer(n, heads, self.m, self.num, self.den, self.score, self.scale)

    STATE = ("m", "den", "num", "score", "o", "idx")

    def state_dict(self) -> dict:
        """The layer's cached state (row max, numerator, denominator, key-mass
        scores, output and index sets) as host tensors, for a checkpoint.  A
        re-identifying layer also needs the previous step's q, k, v, which the
        caller owns."""
        return {name: getattr(self, name).detach().cpu() for name in self.STATE}

    def load_state_dict(self, state: dict):
        """As MLPDelta.load_state_dict; the index sets are checked against the
        key range."""
        for name in self.STATE:
            dst = getattr(self, name)
            src = state[name]
            assert src.shape == dst.shape and src.dtype == dst.dtype, name
            dst.copy_(src)
        if self.kk:
            check_index_sets(self.idx, self.n, "attention index sets")

    def reset(self):
        for name in self.STATE:
            getattr(self, name).zero_()
        self.prev = None

    def dense(self, q, k, v, stream=None):
        lib.chipmunk_dense_step(lib.ATTN, self.layer, q, k, v, self.o, stream=stream)

    def identify(self, stream=None):
        lib.chipmunk_identify_topk(self.score, self.heads * self.nb, self.n, self.kk, self.idx, stream=stream)

    def refresh_rest(self, q, k, v, idx=None, stream=None):
        lib.chipmunk_sparse_attn_delta(self.layer, q, k, v, self.idx if idx is None else idx, self.kk,
                                       lib.ATTN_REFRESH, None, stream=stream)

    def sparse(self, q, k, v, idx=None, stream=None):
        lib.chipmunk_sparse_attn_delta(self.layer, q, k, v, self.idx if idx is None else idx, self.kk,
                                       lib.ATTN_SPARSE, self.o, stream=stream)

    def reident_sparse(self, q, k, v, idx=None, stream=None):
        qp, kp, vp = self.prev
        lib.chipmunk_sparse_attn_reident(self.layer, qp, kp, vp, q, k, v, self.idx if idx is None else idx,
                                         self.kk, self.o, stream=stream)
        self.prev = (q, k, v)

    def step(self, q, k, v, refresh: bool, stream=None):
        if self.reident:
            if refresh:
                self.dense(q, k, v, stream)
                self.prev = (q, k, v)
            else:
                self.identify(stream)
                self.reident_sparse(q, k, v, stream=stream)
        elif refresh:
            self.dense(q, k, v, stream)
            self.identify(stream)
            self.refresh_rest(q, k, v, stream=stream)
        else:
            self.sparse(q, k, v, stream=stream)


DENSE, SPARSE, CACHED = "dense", "sparse", "cached"


def schedule_step(kind: str, mlp: MLPDelta = None, att: AttnDelta = None, x=None, q=None, k=None, v=None,
                  fused: bool = True, stream=None):
    """One step of a sampler loop for a block's MLP and / or attention layer:
    kind DENSE (refresh), SPARSE (the delta; through the shared-grid call when
    both layers are given and fused) or CACHED (step caching: nothing runs, the
    output buffers keep the latest computed outputs)."""
    if kind == CACHED:
        return
    if kind not in (DENSE, SPARSE):
        raise ValueError(kind)
    if kind == SPARSE and fused and mlp is not None and att is not None:
        sparse_step(mlp, att, x, q, k, v, stream=stream)
        return
    if mlp is not None:
        mlp.step(x, refresh=kind == DENSE, stream=stream)
    if att is not None:
        att.step(q, k, v, refresh=kind == DENSE, stream=stream)


def sparse_step(mlp: MLPDelta, att: AttnDelta, x, q, k, v, stream=None):
    """One sparse step of a block whose attention and MLP deltas are independent
    (both read the block's input): the top-k of a layer that re-identifies
    every step (MLP rescoring, re-identifying attention), then both deltas
    through chipmunk_sparse_step (or chipmunk_sparse_step_reident).  Same
    results as ``mlp.step(x, False)`` followed by ``att.step(q, k, v, False)``."""
    if mlp.rescore:
        mlp.identify(stream)
    if att.reident:
        att.identify(stream)
        qp, kp, vp = att.prev
        lib.chipmunk_sparse_step_reident(mlp.layer, x, mlp.idx, mlp.k, mlp.y, None, mlp.ws, att.layer, qp, kp, vp,
                                         q, k, v, att.idx, att.kk, att.o, stream=stream)
        att.prev = (q, k, v)
    else:
        lib.chipmunk_sparse_step(mlp.layer, x, mlp.idx, mlp.k, mlp.y, None, mlp.ws, att.layer, q, k, v, att.idx,
                                 att.kk, att.o, stream=stream)
