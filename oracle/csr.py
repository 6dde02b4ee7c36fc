"""Union of block masks and per-query-block kv index lists (test infrastructure only).

Source: the NABLA review ("What carries the argument") ORs the adaptive mask with a
sliding-tile mask; the CalibAtt page describes handing the attention kernel a list
of the blocks to visit per query block instead of a dense mask.
"""
import numpy as np


def mask_or(a, b) -> np.ndarray:
    return np.logical_or(np.asarray(a, dtype=bool), np.asarray(b, dtype=bool))


def mask_to_csr(mask):
    """mask bool [R, nb] -> (row_ptr int64 [R+1], col_idx int64 [nnz]).

    Row r's kept key blocks, ascending, are col_idx[row_ptr[r]:row_ptr[r+1]].
    """
    mask = np.asarray(mask, dtype=bool)
    row_ptr = [0]
    cols = []
    for row in mask:
        nz = np.nonzero(row)[0]
        cols.append(nz)
        row_ptr.append(row_ptr[-1] + len(nz))
    col_idx = np.concatenate(cols) if cols else np.zeros(0, dtype=np.int64)
    return np.asarray(row_ptr, dtype=np.int64), col_idx.astype(np.int64)


def longest_first_order(mask):
    """mask bool [R, nb] -> int64 [R]: the rows by kept count, largest first, rows of
    equal count in ascending index order (a longest-processing-time-first work list
    for the per-row lists above)."""
    counts = np.asarray(mask, dtype=bool).sum(axis=1)
    rows = list(range(len(counts)))
    rows.sort(key=lambda r: (-int(counts[r]), r))
    return np.asarray(rows, dtype=np.int64)
