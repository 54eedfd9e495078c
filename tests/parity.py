"""Comparison rules between the GPU path and the oracle (test logic only).

Mask rule: for each (head, block-row) the GPU's kept set must equal the
oracle's, except for blocks whose cumulative boundary lies within 1e-4 of tau
(the oracle's normalised mass ordered before the block, |C_before - tau| <=
1e-4; the exemption of the block-mask tolerance).  Every other difference is
"unexcused", and the tests require none.  There is no tie category: a block
that swapped places with a near-equal block outside the boundary band counts
as unexcused.
"""
import numpy as np

BOUNDARY = 1e-4


def classify_masks(keep_gpu, keep_orc, cbefore, A_orc, tau, valid_rows=None):
    """Return dict(match_rows, rows, diff_blocks, boundary, unexcused, examples)."""
    keep_gpu = np.asarray(keep_gpu).astype(bool)
    keep_orc = np.asarray(keep_orc).astype(bool)
    nb = keep_orc.shape[-1]
    kg = keep_gpu.reshape(-1, nb)
    ko = keep_orc.reshape(-1, nb)
    cb = np.asarray(cbefore).reshape(-1, nb)
    A = np.asarray(A_orc, dtype=np.float64).reshape(-1, nb)
    out = dict(rows=kg.shape[0], match_rows=0, diff_blocks=0, boundary=0, unexcused=0,
               examples=[])
    W = A.sum(axis=1)
    diff = kg != ko
    out["match_rows"] = int((~diff.any(axis=1)).sum())
    for r in np.nonzero(diff.any(axis=1))[0]:
        an = A[r] / W[r]
        for J in np.nonzero(diff[r])[0]:
            out["diff_blocks"] += 1
            if abs(cb[r, J] - tau) <= BOUNDARY:
                out["boundary"] += 1
                continue
            out["unexcused"] += 1
            if len(out["examples"]) < 5:
                out["examples"].append((int(r), int(J), float(cb[r, J]), float(an[J])))
    return out


def mask_from_list(counts, idx, nb):
    """Dense mask from a compacted (counts, ascending indices) list, vectorised."""
    counts = np.asarray(counts)
    idx = np.asarray(idx)
    Hq = counts.shape[0]
    pos = np.arange(nb)[None, None, :]
    valid = pos < counts[:, :, None]
    m = np.zeros((Hq, nb, nb), dtype=np.uint8)
    hh, II, kk = np.nonzero(valid)
    m[hh, II, idx[hh, II, kk]] = 1
    return m


def list_from_mask(mask):
    """Compacted (counts, ascending indices, -1 padded) from a dense mask, vectorised."""
    mask = np.asarray(mask).astype(bool)
    Hq, nb, _ = mask.shape
    counts = mask.sum(axis=2).astype(np.int32)
    # Stable sort of the keys (0 for kept, 1 for dropped) puts the kept block
    # indices first, in ascending order.
    order = np.argsort(~mask, axis=2, kind="stable").astype(np.int32)
    pos = np.arange(nb)[None, None, :]
    idx = np.where(pos < counts[:, :, None], order, -1).astype(np.int32)
    return counts, idx


def list_is_well_formed(counts, idx):
    """Ascending, in range J <= I, non-empty, -1 padded."""
    counts = np.asarray(counts)
    idx = np.asarray(idx)
    Hq, nb = counts.shape
    pos = np.arange(nb)[None, None, :]
    valid = pos < counts[:, :, None]
    if np.any(counts < 1) or np.any(counts > np.arange(1, nb + 1)[None, :]):
        return False
    if np.any(idx[~valid] != -1):
        return False
    v = np.where(valid, idx, 10 ** 9)
    if np.any(v[valid] < 0):
        return False
    if np.any((v <= np.arange(nb)[None, :, None]) != valid):
        return False
    d = np.diff(np.where(valid, idx, np.iinfo(np.int32).max), axis=2)
    return bool(np.all(d[valid[:, :, 1:]] > 0))


def o_errors(o_gpu, o_ref):
    e = np.abs(np.asarray(o_gpu, dtype=np.float64) - np.asarray(o_ref, dtype=np.float64))
    return float(e.max()), float(e.mean())
