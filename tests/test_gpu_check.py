"""chipmunk_check_index_sets on the GPU against the contract written out here:
a row breaks it when a value lies outside [0, cols) or the row is not strictly
ascending.  Valid sets (the library's own top-k output included) give
{0, rows}; planted mistakes in chosen rows give their count and the smallest."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _bad_rows(idx, cols):
    idx = np.asarray(idx, dtype=np.int64)
    out_of_range = ((idx < 0) | (idx >= cols)).any(axis=1)
    not_ascending = (np.diff(idx, axis=1) <= 0).any(axis=1) if idx.shape[1] > 1 else np.zeros(len(idx), bool)
    return np.flatnonzero(out_of_range | not_ascending)


def _check(lib, idx_np, cols):
    rows, k = idx_np.shape
    idx = torch.from_numpy(np.ascontiguousarray(idx_np, dtype=np.int32)).cuda()
    res = torch.full((2,), -7, dtype=torch.int64, device="cuda")
    lib.chipmunk_check_index_sets(idx, rows, k, cols, res)
    torch.cuda.synchronize()
    return res.cpu().tolist()


def test_valid_sets_pass(gpu_lib):
    g = np.random.default_rng(3)
    for rows, k, cols in [(1, 1, 1), (5, 64, 64), (37, 130, 1000), (300, 718, 4352)]:
        idx = np.stack([np.sort(g.choice(cols, size=k, replace=False)) for _ in range(rows)])
        print(f"valid rows={rows} k={k} cols={cols}", flush=True)
        assert _check(gpu_lib, idx, cols) == [0, rows]


def test_library_topk_output_passes(gpu_lib):
    rows, cols, k = 929, 12288, 860
    score = torch.randn(rows, cols, device="cuda")
    score[:, ::7] = 0.5                            # ties
    idx = torch.empty(rows, k, dtype=torch.int32, device="cuda")
    gpu_lib.chipmunk_identify_topk(score, rows, cols, k, idx)
    res = torch.zeros(2, dtype=torch.int64, device="cuda")
    gpu_lib.chipmunk_check_index_sets(idx, rows, k, cols, res)
    torch.cuda.synchronize()
    assert res.cpu().tolist() == [0, rows]


@pytest.mark.parametrize("k", [1, 63, 64, 65, 300])
def test_planted_mistakes_are_found(gpu_lib, k):
    g = np.random.default_rng(k)
    rows, cols = 200, 5000
    idx = np.stack([np.sort(g.choice(cols, size=k, replace=False)) for _ in range(rows)]).astype(np.int64)
    idx[17, k // 2] = cols                         # out of range (high)
    idx[90, 0] = -1                                # out of range (low)
    if k > 1:
        idx[120, k - 1] = idx[120, k - 2]          # duplicate: not strictly ascending
        idx[151, [0, k - 1]] = idx[151, [k - 1, 0]]  # swapped: descending pair
    idx[199, :] = idx[199, ::-1]                   # reversed row (k = 1: still valid)
    expect = _bad_rows(idx, cols)
    print(f"k={k}: planted rows {expect.tolist()}", flush=True)
    got = _check(gpu_lib, idx, cols)
    assert got == [len(expect), int(expect.min()) if len(expect) else rows]


def test_empty_calls_write_the_no_mistake_result(gpu_lib):
    assert _check(gpu_lib, np.zeros((0, 5), np.int32), 10) == [0, 0]
    res = torch.full((2,), -7, dtype=torch.int64, device="cuda")
    gpu_lib.chipmunk_check_index_sets(None, 12, 0, 10, res)
    torch.cuda.synchronize()
    assert res.cpu().tolist() == [0, 12]
