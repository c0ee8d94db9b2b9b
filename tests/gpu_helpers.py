"""Shared plumbing for the GPU parity tests: uploads of the seeded bf16 inputs
and layout conversions of what the kernels write, for comparison with the
oracle.  No arithmetic of the method lives here."""
import numpy as np
import torch

ROW_BLOCK = 128


def up_bf16(bits: np.ndarray, dev="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def up_f32(a: np.ndarray, dev="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_values(t: torch.Tensor) -> np.ndarray:
    u = bits_of(t).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def cache_to_rows(a_cache: torch.Tensor, n: int) -> np.ndarray:
    """[nb][h][128] block-column-major cache -> [n][h] values (float64)."""
    nb, h, _ = a_cache.shape
    v = bf16_values(a_cache).reshape(nb, h, ROW_BLOCK).transpose(0, 2, 1).reshape(nb * ROW_BLOCK, h)
    return v[:n]


def rows_to_cache_bits(a_rows_bits: np.ndarray, nb: int) -> np.ndarray:
    """[n][h] bf16 bits -> [nb][h][128] bits (pad rows zero)."""
    n, h = a_rows_bits.shape
    out = np.zeros((nb * ROW_BLOCK, h), np.uint16)
    out[:n] = a_rows_bits
    return np.ascontiguousarray(out.reshape(nb, ROW_BLOCK, h).transpose(0, 2, 1))


def idx_sets_valid(gpu_idx: np.ndarray, ref_idx: np.ndarray, ref_score: np.ndarray, rtol=1e-3, gpu_score=None):
    """Index sets chosen from scores computed in a different summation order may
    differ only between near-tied columns: every column in one set but not the
    other must score within rtol of the row's k-th largest oracle score.  With
    ``gpu_score`` (the scores the GPU ranked), a column may also lie within
    2 * eps of that threshold, eps = the row's largest |gpu_score - ref_score|:
    if two score rows differ by at most eps everywhere, their top-k sets can
    differ only in columns whose score is within 2 * eps of the k-th largest
    (the k-th largest itself moves by at most eps).  Returns the mean Jaccard
    index."""
    jac = []
    for r in range(gpu_idx.shape[0]):
        a, b = set(gpu_idx[r].tolist()), set(ref_idx[r].tolist())
        assert len(a) == gpu_idx.shape[1], "GPU index set has duplicates"
        assert np.all(np.diff(gpu_idx[r]) > 0), "GPU index set not ascending"
        k = len(b)
        if k == 0:
            continue
        tau = np.sort(ref_score[r])[::-1][k - 1]
        eps = 0.0
        if gpu_score is not None:
            eps = float(np.max(np.abs(np.asarray(gpu_score[r], np.float64) - np.asarray(ref_score[r], np.float64))))
        for c in a ^ b:
            gap = abs(float(ref_score[r][c]) - float(tau))
            assert gap <= max(rtol * max(abs(float(tau)), 1e-30), 2.0 * eps), (r, c, ref_score[r][c], tau, eps)
        jac.append(len(a & b) / len(a | b))
    return float(np.mean(jac)) if jac else 1.0


def block_sizes(blocks, n: int) -> list:
    """Row counts of the sampled row blocks (the last block of n may be partial)."""
    return [min(n, (b + 1) * ROW_BLOCK) - b * ROW_BLOCK for b in blocks]


def worst_block_error(g: np.ndarray, ref: np.ndarray, sizes, col_group: int = 0):
    """Largest relative Frobenius error over the row blocks of stacked rows
    (``sizes`` rows each, in order) and, with ``col_group``, over every (row
    block, group of col_group columns) tile of them: one bar per tile, so a
    wrong tile or a wrong short tail block is not averaged away by the rest.
    Returns (error, row block position, column group)."""
    import oracle
    worst = (0.0, -1, -1)
    r0 = 0
    for i, s in enumerate(sizes):
        gb, rb = g[r0:r0 + s], ref[r0:r0 + s]
        r0 += s
        e = oracle.rel_frobenius(gb, rb)
        if e > worst[0]:
            worst = (e, i, -1)
        if col_group:
            for c in range(0, rb.shape[1], col_group):
                e = oracle.rel_frobenius(gb[:, c:c + col_group], rb[:, c:c + col_group])
                if e > worst[0]:
                    worst = (e, i, c // col_group)
    return worst


def attn_s_only(lib, att, q, k, v, idx=None):
    """The sparse attention call on a copy of the layer whose rest caches (num,
    den) are zero: o = num_S / den_S over the chosen keys alone.  The layer's
    own caches are left as they were."""
    num, den = torch.zeros_like(att.num), torch.zeros_like(att.den)
    o = torch.empty_like(att.o)
    layer = lib.attn_layer(att.n, att.heads, att.m, num, den, att.score, att.scale)
    lib.chipmunk_sparse_attn_delta(layer, q, k, v, att.idx if idx is None else idx, att.kk, lib.ATTN_SPARSE, o)
    return o
