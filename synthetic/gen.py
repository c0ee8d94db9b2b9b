"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers and stores them in the bf16 bit layout the
kernels and the oracle both accept.  It holds none of the column-sparse delta's
arithmetic: no GELU, no matmul, no softmax, no top-k.

Every tensor is cut into independent streams, one per (tensor tag, diffusion step,
head, 128-row block), each a numpy ``Generator(PCG64(SeedSequence([seed, tag, step,
head, block])))`` drawing ``standard_normal`` in float32.  Any slice can therefore
be regenerated bit-identically without generating the rest, and host threads can
generate blocks in parallel.

Diffusion-step drift follows the workloads' recipe: a float32 master random walk
``X_t = X_{t-1} + 0.05 * eps_t`` with ``X_0 = eps_0``; each step hands out the
bf16 (round-to-nearest-even) rounding of the walk.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROW_BLOCK = 128
DRIFT = np.float32(0.05)

TAG = {"X": 1, "W1": 2, "W2": 3, "Q": 4, "K": 5, "V": 6, "SCORE": 7}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def stream(seed: int, tag: int, step: int, head: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, step, head, block])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest, ties to even.

    Inputs here are finite Gaussian draws, so NaN handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _block_rows(n: int, block: int) -> tuple[int, int]:
    r0 = block * ROW_BLOCK
    return r0, min(n, r0 + ROW_BLOCK)


def walk_block(seed: int, tag: int, step: int, head: int, block: int, rows: int, cols: int) -> np.ndarray:
    """float32 master walk of one (head, row-block) slice at diffusion step ``step``."""
    x = stream(seed, tag, 0, head, block).standard_normal((rows, cols), dtype=np.float32)
    for s in range(1, step + 1):
        eps = stream(seed, tag, s, head, block).standard_normal((rows, cols), dtype=np.float32)
        x = x + DRIFT * eps
    return x


def _chunk_blocks(cols: int) -> int:
    """Row blocks per generation job: about 2M floats, so a job's buffers stay small
    while its draws are large enough to run outside the interpreter lock."""
    return max(1, (1 << 21) // (ROW_BLOCK * cols))


def _walk_rows(seed: int, t: int, head: int, n: int, cols: int, b0: int, b1: int, steps: int, emit) -> None:
    """Advance the master walk of row blocks b0..b1-1 (one contiguous row range)
    through steps 0..steps-1, calling ``emit(step, r0, r1, x)`` with the float32
    walk after each step.  Same values as ``walk_block`` on every block."""
    r0, r1 = b0 * ROW_BLOCK, min(n, b1 * ROW_BLOCK)
    x = np.empty((r1 - r0, cols), np.float32)
    eps = np.empty_like(x) if steps > 1 else None
    for s in range(steps):
        dst = x if s == 0 else eps
        for b in range(b0, b1):
            a, c = _block_rows(n, b)
            stream(seed, t, s, head, b).standard_normal(out=dst[a - r0:c - r0], dtype=np.float32)
        if s:
            np.multiply(eps, DRIFT, out=eps)
            np.add(x, eps, out=x)
        emit(s, r0, r1, x)


def _run_walks(seed: int, t: int, heads: int, n: int, cols: int, steps: int, emit) -> None:
    nb = (n + ROW_BLOCK - 1) // ROW_BLOCK
    ch = _chunk_blocks(cols)
    jobs = [(h, b, min(nb, b + ch)) for h in range(heads) for b in range(0, nb, ch)]

    def one(job):
        h, b0, b1 = job
        _walk_rows(seed, t, h, n, cols, b0, b1, steps, lambda s, r0, r1, x: emit(h, s, r0, r1, x))

    if len(jobs) > 1:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, jobs))
    else:
        for j in jobs:
            one(j)


def activations(seed: int, tag: str, step: int, n: int, cols: int, head: int = 0,
                blocks=None) -> np.ndarray:
    """bf16 bits [rows, cols] of a drifting activation (X, or one head of Q/K/V).

    ``blocks``: iterable of 128-row block indices to generate (default: all).  The
    result stacks the requested blocks' rows in the given order.
    """
    t = TAG[tag]
    if blocks is None:
        out = np.empty((n, cols), np.uint16)

        def emit(h, s, r0, r1, x):
            if s == step:
                out[r0:r1] = f32_to_bf16_bits(x)

        nb = (n + ROW_BLOCK - 1) // ROW_BLOCK
        ch = _chunk_blocks(cols)
        jobs = [(b, min(nb, b + ch)) for b in range(0, nb, ch)]

        def one(job):
            _walk_rows(seed, t, head, n, cols, job[0], job[1], step + 1, lambda s, r0, r1, x: emit(head, s, r0, r1, x))

        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, jobs))
        return out
    parts = []
    for b in blocks:
        r0, r1 = _block_rows(n, b)
        parts.append(f32_to_bf16_bits(walk_block(seed, t, step, head, b, r1 - r0, cols)))
    return np.concatenate(parts, axis=0) if parts else np.zeros((0, cols), np.uint16)


def heads_activations(seed: int, tag: str, step: int, heads: int, n: int, dim: int = 128) -> np.ndarray:
    """bf16 bits [heads, n, dim] for Q, K or V."""
    out = np.empty((heads, n, dim), np.uint16)

    def emit(h, s, r0, r1, x):
        if s == step:
            out[h, r0:r1] = f32_to_bf16_bits(x)

    _run_walks(seed, TAG[tag], heads, n, dim, step + 1, emit)
    return out


def activation_walk(seed: int, tag: str, steps: int, n: int, cols: int, head: int = 0) -> list:
    """bf16 bits [n, cols] of a drifting activation at steps 0 .. steps-1, generated
    incrementally (same values as ``activations`` at each step)."""
    out = [np.empty((n, cols), np.uint16) for _ in range(steps)]

    def emit(h, s, r0, r1, x):
        out[s][r0:r1] = f32_to_bf16_bits(x)

    nb = (n + ROW_BLOCK - 1) // ROW_BLOCK
    ch = _chunk_blocks(cols)
    jobs = [(b, min(nb, b + ch)) for b in range(0, nb, ch)]

    def one(job):
        _walk_rows(seed, TAG[tag], head, n, cols, job[0], job[1], steps, lambda s, r0, r1, x: emit(head, s, r0, r1, x))

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, jobs))
    return out


def heads_walk(seed: int, tag: str, steps: int, heads: int, n: int, dim: int = 128) -> list:
    """bf16 bits [heads, n, dim] of Q, K or V at steps 0 .. steps-1 (incremental)."""
    out = [np.empty((heads, n, dim), np.uint16) for _ in range(steps)]

    def emit(h, s, r0, r1, x):
        out[s][h, r0:r1] = f32_to_bf16_bits(x)

    _run_walks(seed, TAG[tag], heads, n, dim, steps, emit)
    return out


class Walk:
    """The master walk of one drifting tensor ([heads, n, cols]), advanced one
    diffusion step at a time: ``advance()`` returns the bf16 bits of the next
    step.  Same values as ``heads_walk`` / ``activation_walk`` at every step,
    holding one float32 copy of the walk instead of every step's bits."""

    def __init__(self, seed: int, tag: str, heads: int, n: int, cols: int):
        self.seed, self.tag, self.heads, self.n, self.cols = seed, TAG[tag], heads, n, cols
        self.x = np.empty((heads, n, cols), np.float32)
        self.t = -1

    def advance(self) -> np.ndarray:
        """bf16 bits [heads, n, cols] of step t + 1 (step 0 on the first call)."""
        self.t += 1
        s, n, cols = self.t, self.n, self.cols
        nb = (n + ROW_BLOCK - 1) // ROW_BLOCK
        ch = _chunk_blocks(cols)
        jobs = [(h, b, min(nb, b + ch)) for h in range(self.heads) for b in range(0, nb, ch)]
        out = np.empty((self.heads, n, cols), np.uint16)

        def one(job):
            h, b0, b1 = job
            r0, r1 = b0 * ROW_BLOCK, min(n, b1 * ROW_BLOCK)
            x = self.x[h, r0:r1]
            dst = x if s == 0 else np.empty_like(x)
            for b in range(b0, b1):
                a, c = _block_rows(n, b)
                stream(self.seed, self.tag, s, h, b).standard_normal(out=dst[a - r0:c - r0], dtype=np.float32)
            if s:
                np.multiply(dst, DRIFT, out=dst)
                np.add(x, dst, out=x)
            out[h, r0:r1] = f32_to_bf16_bits(x)

        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, jobs))
        return out


def weight(seed: int, tag: str, rows: int, cols: int, fan_in: int) -> np.ndarray:
    """bf16 bits [rows, cols] of N(0,1) * 1/sqrt(fan_in) (standard deviation 1/sqrt(fan_in))."""
    nb = (rows + ROW_BLOCK - 1) // ROW_BLOCK
    scale = np.float32(1.0 / np.sqrt(np.float64(fan_in)))
    out = np.empty((rows, cols), np.uint16)
    t = TAG[tag]

    def one(b):
        r0, r1 = _block_rows(rows, b)
        g = stream(seed, t, 0, 0, b).standard_normal((r1 - r0, cols), dtype=np.float32)
        out[r0:r1] = f32_to_bf16_bits(g * scale)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(nb)))
    return out


def mlp_weights(seed: int, d: int, h: int):
    """(W1t [h,d], W2 [h,d]) bf16 bits.  W1t row j is hidden unit j's input weights
    (fan_in d); W2 row j is hidden unit j's output vector (fan_in h)."""
    return weight(seed, "W1", h, d, d), weight(seed, "W2", h, d, h)


def scores(seed: int, rows: int, cols: int, kind: str = "normal", step: int = 0) -> np.ndarray:
    """float32 score rows for top-k tests.

    kinds: ``normal`` (continuous, no ties), ``ties`` (integers in {0,1,2}: heavy
    ties), ``special`` (mix of +-0, +-inf, NaN and a few repeated values), ``abs``
    (|N(0,1)|, the shape of an L1 or probability-mass score).
    """
    out = np.empty((rows, cols), np.float32)
    for r in range(rows):
        g = stream(seed, TAG["SCORE"], step, 0, r)
        if kind == "normal":
            out[r] = g.standard_normal(cols, dtype=np.float32)
        elif kind == "abs":
            out[r] = np.abs(g.standard_normal(cols, dtype=np.float32))
        elif kind == "ties":
            out[r] = g.integers(0, 3, cols).astype(np.float32)
        elif kind == "special":
            base = np.round(g.standard_normal(cols, dtype=np.float32) * 4) / 4
            pick = g.integers(0, 10, cols)
            base = np.where(pick == 0, np.float32(0.0), base)
            base = np.where(pick == 1, np.float32(-0.0), base)
            base = np.where(pick == 2, np.float32(np.inf), base)
            base = np.where(pick == 3, np.float32(-np.inf), base)
            base = np.where(pick == 4, np.float32(np.nan), base)
            out[r] = base.astype(np.float32)
        else:
            raise ValueError(kind)
    return out
