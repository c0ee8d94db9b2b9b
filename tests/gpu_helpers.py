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


def idx_sets_valid(gpu_idx: np.ndarray, ref_idx: np.ndarray, ref_score: np.ndarray, rtol=1e-3):
    """Index sets chosen from scores computed in a different summation order may
    differ only between near-tied columns: every column in one set but not the
    other must score within rtol of the row's k-th largest oracle score.
    Returns the mean Jaccard index."""
    jac = []
    for r in range(gpu_idx.shape[0]):
        a, b = set(gpu_idx[r].tolist()), set(ref_idx[r].tolist())
        assert len(a) == gpu_idx.shape[1], "GPU index set has duplicates"
        assert np.all(np.diff(gpu_idx[r]) > 0), "GPU index set not ascending"
        k = len(b)
        if k == 0:
            continue
        tau = np.sort(ref_score[r])[::-1][k - 1]
        for c in a ^ b:
            assert abs(ref_score[r][c] - tau) <= rtol * max(abs(tau), 1e-30), (r, c, ref_score[r][c], tau)
        jac.append(len(a & b) / len(a | b))
    return float(np.mean(jac)) if jac else 1.0
