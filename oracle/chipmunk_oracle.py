"""CPU oracle for the column-sparse cross-step delta.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package.
The product path (``dynamic_column_sparse_amd`` and its HIP library) never imports
it and shares no code with it.

Source of the method: "Chipmunk: Training-Free Acceleration of Diffusion
Transformers with Dynamic Column-Sparse Deltas" (Silveria, Govande, Fu; Together AI
research post, 2025), called "the Chipmunk post" below.  Its section "Activation
Deltas Across Diffusion Steps are Very Sparse" gives

* the two ops: attention ``softmax(Q K^T) V`` and MLP ``gelu(x W1) W2``;
* the reading of each as a linear combination of value vectors (rows of V for
  attention, rows of W2 plus one static bias vector for the MLP);
* the cache of value vectors and scalar coefficients, with a per-step choice of
  which ones to recompute;
* the delta reformulation: with an output cache, a dense step n is the same as
  taking every one of step n-1's output vectors out of the cache and putting every
  one of step n's in; the sparse step swaps only a chosen subset (single hidden
  units or single keys) and keeps the others from the earlier step.

The row-block granularity (128 tokens), top-k per block, GELU in its tanh form and
the cached attention state (row max, numerator, denominator) are the workloads'
operational definition of that method.

Arithmetic is float64 throughout.  Values the kernels store in bfloat16 (inputs,
weights, the MLP activation cache) are rounded to bf16 (nearest, ties to even) at
exactly those storage points, so both sides start from the same bits.  Scores are
handed to top-k as float32, the precision the kernels rank in.

Readings of points the post leaves open (each is listed with its reason in the
design notes of this repository):
  R1 MLP score = per-block column L1 of (A_new - A_cache) at the latest dense step
     (cache starts at zero).
  R2 attention score = per-block key probability mass sum_i p_ij / den_i at the
     dense refresh.
  R3 S is fixed from a refresh to the next; the attention "old" S-part is the
     refresh step's, so the refresh stores num_rest / den_rest.
  R4 top-k order: score descending, then index ascending; -0 == +0; NaN lowest;
     output ascending.
  R6 softmax scale 1/sqrt(head_dim).
  R8 D is the exact difference of the stored bf16 values (no rounding of D here).
  R9 a partial last row block is scored over its real rows only.
  R10 sparse attention steps keep the refresh-step row max (no re-normalisation).
  R12 optional per-step rescoring of the MLP: a sparse step sets the score of each
      unit it recomputed to that step's column L1 of D; other units keep theirs.
  R13 optional per-step re-identification of attention: the cache keeps the total
      numerator and denominator of the dense step; a sparse step takes the chosen
      keys' share as computed from the previous step's q, k, v out of them and puts
      the share from this step's q, k, v in, and sets those keys' scores to this
      step's probability mass over the denominator held at the start of the step.
  R14 optional fp8 variant of the MLP's first product: x and W1^T become e4m3 codes
      row by row, each row with the smallest power-of-two scale that brings its
      largest magnitude within 448, rounded to nearest even; the product (dense and
      sparse) takes those values, and everything after it is unchanged.  The fp8
      MLP is mlp_dense / mlp_sparse applied to fp8_rows(x) and fp8_rows(w1t).
  R16 step caching: a cached step recomputes nothing for the layer -- its output
      is the output cache as the latest computed step left it, and every cache
      keeps its value (the delta over an empty set of vectors, for the whole
      layer).  Which steps are cached is the schedule's choice.
  R15 optional fp8 second product of the sparse delta (with R14): D, rounded to
      bf16 as the bf16 path stores it, becomes e4m3 codes per (row, 32 consecutive
      units of S) block, and W2 per column (output feature); each block and column
      takes its own smallest fitting power-of-two scale.  The dense step's second
      product stays bf16.  mlp_sparse(..., w2=fp8_cols(w2), d_fp8=True).

Parity pins for every function live in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import numpy as np

ROW_BLOCK = 128


# --------------------------------------------------------------------------- #
# Storage rounding
# --------------------------------------------------------------------------- #
def bf16_round(x) -> np.ndarray:
    """Nearest bfloat16 value of each element (ties to even), returned as float64.

    bfloat16 = 1 sign, 8 exponent, 7 stored mantissa bits.  Normal numbers keep 8
    significant bits; below 2**-126 the spacing is 2**-133 (subnormals); a result
    at or above 2**128 overflows to infinity.  NaN and infinities pass through.
    """
    x = np.asarray(x, dtype=np.float64)
    mant, expo = np.frexp(x)                      # x = mant * 2**expo, 0.5 <= |mant| < 1
    r = np.ldexp(np.rint(np.ldexp(mant, 8)), expo - 8)   # np.rint rounds half to even
    tiny = np.abs(x) < 2.0 ** -126
    r = np.where(tiny, np.ldexp(np.rint(np.ldexp(x, 133)), -133), r)
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)


def bf16_bits(x) -> np.ndarray:
    """bf16 bit patterns (uint16) of ``bf16_round(x)``."""
    v = bf16_round(x).astype(np.float32)          # exact: every bf16 value is an fp32 value
    return (v.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def from_bf16_bits(b) -> np.ndarray:
    """float64 values of bf16 bit patterns."""
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------- #
# FP8 operands (the fp8 variant of the MLP's first product)
# --------------------------------------------------------------------------- #
E4M3_MAX = 448.0


def fp8_e4m3_round(v) -> np.ndarray:
    """Nearest OCP fp8 e4m3 ("fn": 4 exponent bits with bias 7, 3 mantissa bits,
    no infinities, largest finite value 448) value of each element, ties to the
    even code, as float64.  Normal values are 2**(E-7) (1 + m/8) for E in 1..15;
    below 2**-6 the spacing is 2**-9 (subnormals).  Inputs must satisfy
    |v| <= 448 (the quantizer scales rows into that range)."""
    v = np.asarray(v, dtype=np.float64)
    assert np.all(np.abs(v) <= E4M3_MAX), "value outside the e4m3 range"
    a = np.abs(v)
    _, ex = np.frexp(a)                          # a = mant * 2**ex, 0.5 <= mant < 1: binade 2**(ex-1)
    # quantum: 2**(ex-1-3) in a normal binade, 2**-9 below 2**-6
    q = np.where(a >= 2.0 ** -6, np.ldexp(1.0, ex - 4), 2.0 ** -9)
    r = np.rint(a / q) * q                       # np.rint: half to even (even quotient = even code)
    return np.copysign(r, v)


def fp8_e4m3_decode(codes) -> np.ndarray:
    """float64 values of e4m3 codes (0x7f / 0xff are NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return s * mag


def fp8_e4m3_encode(v) -> np.ndarray:
    """e4m3 codes (uint8) of fp8_e4m3_round(v); -0 keeps its sign bit."""
    r = fp8_e4m3_round(v)
    a = np.abs(r)
    mant, ex = np.frexp(a)
    normal = a >= 2.0 ** -6
    eb = np.where(normal, ex - 1 + 7, 0)
    m = np.where(normal, np.rint((2.0 * mant - 1.0) * 8), np.rint(a * 2.0 ** 9)).astype(np.int64)
    sign = np.signbit(r).astype(np.int64) << 7
    return (sign | (eb.astype(np.int64) << 3) | m).astype(np.uint8)


def fp8_row_exponent(amax) -> np.ndarray:
    """Per-row scale exponent e: the smallest integer with amax * 2**-e <= 448,
    at least -126; e = 0 for an all-zero row.  With amax = mant * 2**ex
    (0.5 <= mant < 1) and 448 = 0.875 * 2**9 that is ex - 9, plus one when
    mant > 0.875."""
    amax = np.asarray(amax, dtype=np.float64)
    assert np.all(np.isfinite(amax)) and np.all(amax >= 0)
    mant, ex = np.frexp(amax)
    e = ex.astype(np.int64) - 9 + (mant > 0.875)
    e = np.maximum(e, -126)
    return np.where(amax > 0, e, 0)


def quantize_fp8_rows(a):
    """Row-wise fp8 quantization: each row gets the power-of-two scale 2**e of
    fp8_row_exponent(max |row|) and its elements become e4m3 codes of
    a * 2**-e (exact scaling, then round to nearest even).  Returns (codes uint8
    [rows, cols], scale bytes uint8 [rows] = 127 + e, the E8M0 encoding of 2**e)."""
    a = np.asarray(a, dtype=np.float64)
    e = fp8_row_exponent(np.abs(a).max(axis=1) if a.shape[1] else np.zeros(a.shape[0]))
    codes = fp8_e4m3_encode(np.ldexp(a, -e[:, None]))
    return codes, (e + 127).astype(np.uint8)


def dequantize_fp8_rows(codes, scale_bytes) -> np.ndarray:
    """float64 values code * 2**(scale byte - 127), row by row."""
    e = np.asarray(scale_bytes, dtype=np.int64) - 127
    return np.ldexp(fp8_e4m3_decode(codes), e[:, None])


def fp8_rows(a) -> np.ndarray:
    """The values an fp8 operand carries: dequantize_fp8_rows(quantize_fp8_rows(a))."""
    return dequantize_fp8_rows(*quantize_fp8_rows(a))


def quantize_fp8_blocks(a, block: int = 32):
    """Each row cut into consecutive blocks of `block` elements (the last one
    padded with zeros), every block quantized as one row of quantize_fp8_rows.
    Returns (codes [rows, cols] uint8, scale bytes [rows, ceil(cols/block)])."""
    a = np.asarray(a, dtype=np.float64)
    rows, cols = a.shape
    nblk = (cols + block - 1) // block
    padded = np.zeros((rows, nblk * block))
    padded[:, :cols] = a
    codes, sb = quantize_fp8_rows(padded.reshape(rows * nblk, block))
    return codes.reshape(rows, nblk * block)[:, :cols], sb.reshape(rows, nblk)


def fp8_blocks(a, block: int = 32) -> np.ndarray:
    """The values of quantize_fp8_blocks(a, block), dequantized."""
    codes, sb = quantize_fp8_blocks(a, block)
    rows, cols = codes.shape
    e = np.repeat(sb.astype(np.int64) - 127, block, axis=1)[:, :cols]
    return np.ldexp(fp8_e4m3_decode(codes), e)


def fp8_cols(a) -> np.ndarray:
    """Column-wise fp8 values: each column with its own power-of-two scale."""
    return fp8_rows(np.asarray(a, dtype=np.float64).T).T


# --------------------------------------------------------------------------- #
# Non-linearity
# --------------------------------------------------------------------------- #
def gelu_tanh(z) -> np.ndarray:
    """GELU in its tanh form (Hendrycks & Gimpel 2016):
    0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))).

    The Chipmunk post writes the MLP as gelu(x W1) W2; the workloads name the tanh
    form.
    """
    z = np.asarray(z, dtype=np.float64)
    c = np.sqrt(2.0 / np.pi)
    return 0.5 * z * (1.0 + np.tanh(c * (z + 0.044715 * z * z * z)))


def _blocks(n: int):
    for b in range((n + ROW_BLOCK - 1) // ROW_BLOCK):
        r0 = b * ROW_BLOCK
        yield b, r0, min(n, r0 + ROW_BLOCK)


# --------------------------------------------------------------------------- #
# Sparsity identification
# --------------------------------------------------------------------------- #
def identify_topk(score, k: int) -> np.ndarray:
    """Per row, the k columns to recompute: largest score first, ties to the lower
    column index; returned ascending, int32 [rows, k].

    The post says each step chooses which vectors to recompute; the workloads fix
    the choice as top-k per 128-token block.  Ranking is on float32 values (the
    kernels' precision), -0 equals +0, NaN ranks below everything, +inf above
    every finite value.
    """
    s = np.asarray(score, dtype=np.float32)
    if s.ndim != 2:
        raise ValueError("score must be 2-D [rows, cols]")
    rows, cols = s.shape
    if not 0 <= k <= cols:
        raise ValueError("k out of range")
    out = np.empty((rows, k), dtype=np.int32)
    col = np.arange(cols)
    for r in range(rows):
        v = s[r].astype(np.float64)
        nan = np.isnan(v)
        v = np.where(nan, 0.0, v) + 0.0             # + 0.0 maps -0 to +0
        order = np.lexsort((col, -v, nan))          # NaN last, then score desc, then index asc
        out[r] = np.sort(order[:k])
    return out


# --------------------------------------------------------------------------- #
# MLP
# --------------------------------------------------------------------------- #
def mlp_dense(x, w1t, b1, w2, b2, a_old):
    """Dense refresh step of the MLP: the ordinary full forward pass, which also
    fills the caches (Chipmunk post, Activation Deltas section).

    x [n,d] (bf16 values), w1t [h,d] (row j = hidden unit j's input weights),
    w2 [h,d] (row j = hidden unit j's output vector), b1 [h] / b2 [d] or None,
    a_old [n,h] = the activation cache before this step.

    Returns (a_new [n,h] bf16 values, y [n,d], score [nb,h]) where
      z = x w1t^T + b1, a_new = bf16(gelu(z)), y = a_new w2 + b2 and
      score[b,j] = sum over the block's real rows of |a_new - a_old| (reading R1).
    """
    x = np.asarray(x, np.float64)
    w1t = np.asarray(w1t, np.float64)
    w2 = np.asarray(w2, np.float64)
    z = x @ w1t.T
    if b1 is not None:
        z = z + np.asarray(b1, np.float64)[None, :]
    a_new = bf16_round(gelu_tanh(z))
    n, h = a_new.shape
    score = np.zeros(((n + ROW_BLOCK - 1) // ROW_BLOCK, h))
    diff = np.abs(a_new - np.asarray(a_old, np.float64))
    for b, r0, r1 in _blocks(n):
        score[b] = diff[r0:r1].sum(axis=0)
    y = a_new @ w2
    if b2 is not None:
        y = y + np.asarray(b2, np.float64)[None, :]
    return a_new, y, score


def mlp_sparse(x, w1t, b1, w2, a, y, idx, score=None, d_fp8=False):
    """One sparse MLP step (Chipmunk post, Activation Deltas section: only the
    chosen output vectors are swapped for new ones, the others are kept).

    The MLP output is a sum over hidden units j of coefficient a[i,j] times the
    static vector w2[j] (plus a bias that every step shares, so it cancels).  Per
    128-row block b with column set S = idx[b]:
      a_S   = bf16(gelu(x_b w1t[S]^T + b1[S]))     recompute only the chosen units
      D     = a_S - a[b rows, S]                    exact difference of stored values (R8)
      y_b  += D w2[S]                               swap old vectors for new ones
      a[b rows, S] = a_S                            cache writeback
    Returns new copies (a, y); the inputs are not modified.

    With ``score`` [nb,h] given (the per-step rescoring variant, reading R12:
    the post chooses the recomputed vectors in each step), also returns a new
    score in which score[b, S] = sum over the block's real rows of |D| -- the
    dense step's score formula (R1) applied to this step's recomputed units --
    and every other entry is unchanged: (a, y, score).

    With ``d_fp8`` (the fp8 second product, reading R15) the product takes D
    rounded to bf16 (as the bf16 path stores it) and then to e4m3 codes per
    (row, 32 consecutive units of S) block, fp8_blocks(bf16(D)); pass w2 as the
    values the fp8 operand carries, fp8_cols(w2).
    """
    x = np.asarray(x, np.float64)
    w1t = np.asarray(w1t, np.float64)
    w2 = np.asarray(w2, np.float64)
    a = np.array(a, dtype=np.float64, copy=True)
    y = np.array(y, dtype=np.float64, copy=True)
    idx = np.asarray(idx)
    sc = None if score is None else np.array(score, dtype=np.float64, copy=True)
    n = x.shape[0]
    for b, r0, r1 in _blocks(n):
        s = idx[b]
        if s.size == 0:
            continue
        z = x[r0:r1] @ w1t[s].T
        if b1 is not None:
            z = z + np.asarray(b1, np.float64)[s][None, :]
        a_s = bf16_round(gelu_tanh(z))
        d = a_s - a[r0:r1][:, s]
        y[r0:r1] += (fp8_blocks(bf16_round(d), 32) if d_fp8 else d) @ w2[s]
        a[r0:r1, s] = a_s
        if sc is not None:
            sc[b, s] = np.abs(d).sum(axis=0)
    if sc is not None:
        return a, y, sc
    return a, y


# --------------------------------------------------------------------------- #
# Attention (one head; any set of whole query blocks against all keys)
# --------------------------------------------------------------------------- #
def attn_dense(q, k, v, scale: float):
    """Dense refresh of one head (Chipmunk post, Activation Deltas section: the
    output is a sum of rows of V weighted by softmax(Q K^T)).

    q [nq,hd] query rows of whole 128-row blocks (nq may end in a partial block),
    k, v [n,hd] all keys of the head.  With s = scale q k^T:
      m = rowmax(s), p = exp(s - m), den = sum_j p, num = p v, o = num / den,
      score[b, j] = sum over the block's rows of p_ij / den_i   (reading R2).
    Returns (m [nq], den [nq], num [nq,hd], o [nq,hd], score [nbq, n]).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    s = scale * (q @ k.T)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    den = p.sum(axis=1)
    num = p @ v
    o = num / den[:, None]
    nq = q.shape[0]
    score = np.zeros(((nq + ROW_BLOCK - 1) // ROW_BLOCK, k.shape[0]))
    pn = p / den[:, None]
    for b, r0, r1 in _blocks(nq):
        score[b] = pn[r0:r1].sum(axis=0)
    return m, den, num, o, score


def attn_rest(q, k, v, m, idx, scale: float):
    """What the refresh leaves in the attention cache (reading R3): for each query
    row i of block b, the numerator and denominator over the keys NOT in S_b,
    num_rest = sum_{j not in S_b} p_ij v_j and den_rest = sum_{j not in S_b} p_ij,
    with p from the refresh inputs and the refresh row max m.  Computed directly
    as masked sums.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    m = np.asarray(m, np.float64)
    nq, n = q.shape[0], k.shape[0]
    num_rest = np.zeros((nq, v.shape[1]))
    den_rest = np.zeros(nq)
    for b, r0, r1 in _blocks(nq):
        keep = np.ones(n, dtype=bool)
        keep[np.asarray(idx[b])] = False
        p = np.exp(scale * (q[r0:r1] @ k[keep].T) - m[r0:r1, None])
        num_rest[r0:r1] = p @ v[keep]
        den_rest[r0:r1] = p.sum(axis=1)
    return num_rest, den_rest


def attn_sparse(q, k, v, m, num_rest, den_rest, idx, scale: float):
    """One sparse attention step: recompute only the chosen keys' vectors and
    keep the other keys' share from the refresh (Chipmunk post, Activation Deltas section),
    with the refresh row max kept fixed (reading R10):
      p_S = exp(scale q_b k[S_b]^T - m_b)
      o_b = (num_rest_b + p_S v[S_b]) / (den_rest_b + sum_j p_S).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    m = np.asarray(m, np.float64)
    nq = q.shape[0]
    o = np.zeros((nq, v.shape[1]))
    for b, r0, r1 in _blocks(nq):
        s = np.asarray(idx[b])
        p = np.exp(scale * (q[r0:r1] @ k[s].T) - m[r0:r1, None])
        o[r0:r1] = (num_rest[r0:r1] + p @ v[s]) / (den_rest[r0:r1] + p.sum(axis=1))[:, None]
    return o


def attn_reident(q_prev, k_prev, v_prev, q, k, v, m, num, den, score, idx, scale: float):
    """One sparse attention step that lets S change from step to step (reading
    R13; Chipmunk post, Activation Deltas section: the subset of vectors to
    recompute is chosen anew in each step, and a step swaps the chosen vectors of
    the earlier step for this step's).

    The cache (num, den) holds totals over all keys, as the dense step leaves them.
    For each block b with S = idx[b], and the row max m kept from the refresh:
      p_old = exp(scale q_prev_b k_prev[S]^T - m_b)      (the previous step's share)
      p_new = exp(scale q_b k[S]^T - m_b)                (this step's share)
      num_b <- num_b - p_old v_prev[S] + p_new v[S]
      den_b <- den_b - sum_j p_old + sum_j p_new
      o_b    = num_b / den_b
      score[b, S] <- sum over the block's rows of p_new / den_b (den before the step)
    Scores of keys outside S are kept.  Returns (o, num, den, score), new arrays.
    """
    f = lambda a: np.asarray(a, np.float64)
    q_prev, k_prev, v_prev, q, k, v, m = map(f, (q_prev, k_prev, v_prev, q, k, v, m))
    num = f(num).copy()
    den = f(den).copy()
    score = f(score).copy()
    nq = q.shape[0]
    o = np.zeros((nq, v.shape[1]))
    for b, r0, r1 in _blocks(nq):
        s = np.asarray(idx[b])
        mb = m[r0:r1, None]
        p_old = np.exp(scale * (q_prev[r0:r1] @ k_prev[s].T) - mb)
        p_new = np.exp(scale * (q[r0:r1] @ k[s].T) - mb)
        score[b, s] = (p_new / den[r0:r1, None]).sum(axis=0)
        num[r0:r1] += p_new @ v[s] - p_old @ v_prev[s]
        den[r0:r1] += p_new.sum(axis=1) - p_old.sum(axis=1)
        o[r0:r1] = num[r0:r1] / den[r0:r1, None]
    return o, num, den, score


# --------------------------------------------------------------------------- #
# Step caching (reading R16): schedules of dense, sparse and cached steps
# --------------------------------------------------------------------------- #
DENSE, SPARSE, CACHED = "dense", "sparse", "cached"


def mlp_schedule(xs, w1t, b1, w2, b2, k: int, schedule):
    """The MLP over a sampler loop.  schedule[t] is DENSE (mlp_dense, the
    cache starting at zero), SPARSE (top-k of the latest dense step's scores,
    then mlp_sparse on xs[t]) or CACHED (nothing is recomputed: the output of
    step t is the output cache left by the latest computed step, and the
    activation cache is kept).  The Chipmunk post stacks step caching on the
    deltas (Results section) without describing it; reading R16 takes a cached
    step as the delta over the empty set for the whole layer.  Returns the
    output of every step (list of [n,d])."""
    n, h = np.asarray(xs[0]).shape[0], np.asarray(w1t).shape[0]
    a = np.zeros((n, h))
    y = score = None
    out = []
    for t, kind in enumerate(schedule):
        if kind == DENSE:
            a, y, score = mlp_dense(xs[t], w1t, b1, w2, b2, a)
        elif kind == SPARSE:
            if y is None:
                raise ValueError("a sparse step needs an earlier dense step")
            a, y = mlp_sparse(xs[t], w1t, b1, w2, a, y, identify_topk(score.astype(np.float32), k))
        elif kind == CACHED:
            if y is None:
                raise ValueError("a cached step needs an earlier computed step")
        else:
            raise ValueError(kind)
        out.append(y.copy())
    return out


def attn_schedule(qs, ks, vs, scale: float, kk: int, schedule):
    """One attention head over a sampler loop: DENSE (attn_dense, top-kk of its
    key-mass scores per query block, the rest state of attn_rest), SPARSE
    (attn_sparse with the latest refresh's sets and rest state) or CACHED (the
    output of step t is the latest computed output; nothing is recomputed and
    the caches keep their values, reading R16).  Returns the output of every
    step (list of [nq,hd])."""
    o = m = nr = dr = idx = None
    out = []
    for t, kind in enumerate(schedule):
        if kind == DENSE:
            m, _, _, o, score = attn_dense(qs[t], ks[t], vs[t], scale)
            idx = identify_topk(score.astype(np.float32), kk)
            nr, dr = attn_rest(qs[t], ks[t], vs[t], m, idx, scale)
        elif kind == SPARSE:
            if m is None:
                raise ValueError("a sparse step needs an earlier dense step")
            o = attn_sparse(qs[t], ks[t], vs[t], m, nr, dr, idx, scale)
        elif kind == CACHED:
            if o is None:
                raise ValueError("a cached step needs an earlier computed step")
        else:
            raise ValueError(kind)
        out.append(o.copy())
    return out


def rel_frobenius(a, b) -> float:
    """||a - b||_F / ||b||_F (0 when both are zero)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    na = np.linalg.norm(a - b)
    return float(na / nb) if nb > 0 else float(na)
