"""CPU checks of the test-side acceptance helpers: the oracle-free structural
check of index rows accepts rows the oracle produces and rejects each kind
of malformed row (wrong count, padding inside, duplicates, descending order,
an entry inside the window or negative)."""
import numpy as np
import pytest
import torch

import oracle as orc
from parity import check_idx_structure


def oracle_rows(n, k, W, seed=0):
    rng = np.random.default_rng(seed)
    rows = []
    for p in range(n):
        s = rng.standard_normal(orc.candidate_count(p, W))
        rows.append(orc.topk_select(s, k)[0])
    return torch.tensor(np.stack(rows), dtype=torch.int32)[:, None, :], torch.arange(n)


def test_structure_accepts_oracle_rows():
    idx, pos = oracle_rows(90, 16, 8)
    assert check_idx_structure(idx, pos, 8, 16, chunk=7) == 90


@pytest.mark.parametrize("corrupt", ["count", "hole", "dup", "order", "window", "negative"])
def test_structure_rejects_malformed_rows(corrupt):
    idx, pos = oracle_rows(90, 16, 8)
    r = 60  # |C(p)| = 53 > k: a full row
    row = idx[r, 0]
    if corrupt == "count":
        row[-1] = -1
    elif corrupt == "hole":
        row[3] = -1
    elif corrupt == "dup":
        row[5] = row[4]
    elif corrupt == "order":
        row[4], row[5] = int(row[5]), int(row[4])
    elif corrupt == "window":
        row[-1] = pos[r] - 8 + 1
    elif corrupt == "negative":
        row[0] = -5
    with pytest.raises(AssertionError):
        check_idx_structure(idx, pos, 8, 16, chunk=32)


def test_structure_short_rows_padding():
    """Rows with fewer candidates than k: exactly |C(p)| entries, then -1."""
    idx, pos = oracle_rows(30, 16, 8)
    check_idx_structure(idx, pos, 8, 16)
    idx[20, 0, 13] = 99  # p = 20: |C| = 13, so slot 13 must be padding
    with pytest.raises(AssertionError):
        check_idx_structure(idx, pos, 8, 16)
