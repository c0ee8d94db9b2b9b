"""Pins of the oracle's top-k: a pairwise brute force of the ranking rule,
exhaustive subset enumeration on tiny rows, and hand-derived golden rows."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import identify_topk
from synthetic import scores

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "topk_cases.json")


def _beats(a: float, i: int, b: float, j: int) -> bool:
    """Does column i (score a) rank above column j (score b)?  NaN lowest,
    -0 == +0, ties to the lower index."""
    an, bn = np.isnan(a), np.isnan(b)
    if an and bn:
        return i < j
    if an:
        return False
    if bn:
        return True
    if a != b:           # float compare: -0 == +0, inf ordered
        return a > b
    return i < j


def _brute(row: np.ndarray, k: int) -> list:
    cols = len(row)
    chosen = []
    for i in range(cols):
        above = sum(1 for j in range(cols) if j != i and _beats(float(row[j]), j, float(row[i]), i))
        if above < k:
            chosen.append(i)
    return chosen


@pytest.mark.parametrize("kind", ["normal", "ties", "special", "abs"])
@pytest.mark.parametrize("cols", [1, 7, 33, 64])
def test_topk_matches_pairwise_brute_force(kind, cols):
    s = scores(3, 6, cols, kind)
    for k in sorted({0, 1, cols // 3, cols // 2, max(cols - 1, 0), cols}):
        got = identify_topk(s, k)
        assert got.dtype == np.int32 and got.shape == (6, k)
        for r in range(6):
            assert list(got[r]) == _brute(s[r], k), (kind, cols, k, r)


def test_topk_exhaustive_subsets_tiny():
    # The chosen set is the unique k-subset in which every member ranks above
    # every non-member.  Enumerate all subsets and check exactly one qualifies.
    s = scores(5, 20, 8, "ties")
    s[:, 3] = np.float32(np.nan)
    for r in range(s.shape[0]):
        row = s[r]
        for k in range(0, 9):
            ok = [c for c in itertools.combinations(range(8), k)
                  if all(_beats(float(row[i]), i, float(row[j]), j)
                         for i in c for j in range(8) if j not in c)]
            assert len(ok) == 1
            assert list(identify_topk(row[None, :], k)[0]) == list(ok[0])


def test_topk_golden_rows():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        row = np.array([float(v) for v in c["row"]], dtype=np.float32)
        got = identify_topk(row[None, :], c["k"])[0]
        assert list(got) == c["expect"], c["why"]


def test_topk_long_row_and_ascending():
    s = scores(11, 2, 118800, "abs")
    got = identify_topk(s, 8316)
    for r in range(2):
        assert np.all(np.diff(got[r]) > 0)
        thr = np.sort(s[r])[::-1][8315]
        assert np.all(s[r][got[r]] >= thr)
        assert np.sum(s[r] > thr) <= 8316


def test_topk_rejects_bad_k():
    with pytest.raises(ValueError):
        identify_topk(np.zeros((1, 4), np.float32), 5)
    with pytest.raises(ValueError):
        identify_topk(np.zeros((1, 4), np.float32), -1)
