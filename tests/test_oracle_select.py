"""Pins of the oracle's Top-tau step E5: hand-worked cases from the
find_blocks definition, brute-force subset enumeration, and the invariants
(tau=1 keeps all, minimal prefix, monotone in tau, one-hot rows)."""
import itertools
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _select_row(a, tau):
    a = np.asarray(a, dtype=np.float64)
    n = a.shape[0]
    keep, cnt, cb = oracle.select(a[None, :], tau, I_of_row=[n - 1])
    return keep[0], int(cnt[0]), cb[0]


def test_hand_worked_find_blocks_cases():
    path = os.path.join(GOLDEN, "find_blocks_hand.txt")
    n = 0
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        tau, scores, kept = [p.strip() for p in line.split("|")]
        a = [float(x) for x in scores.split()]
        want = [int(x) for x in kept.split()]
        keep, cnt, _ = _select_row(a, float(tau))
        assert list(np.nonzero(keep)[0]) == want, line
        assert cnt == len(want)
        n += 1
    assert n >= 10


def test_brute_force_minimum_cardinality():
    rng = np.random.default_rng(0)
    for trial in range(300):
        n = int(rng.integers(1, 11))
        a = rng.dirichlet(np.full(n, 0.3)) * rng.uniform(0.5, 16)
        if trial % 5 == 0:
            a = np.round(a * 8) / 8 + 1 / 64          # force exact ties
        tau = float(np.float32(rng.choice([0.5, 0.8, 0.9, 0.95, rng.uniform(0.05, 0.999)])))
        keep, cnt, _ = _select_row(a, tau)
        W = a.sum()
        best = None
        for r in range(1, n + 1):
            masses = [sum(a[list(s)]) for s in itertools.combinations(range(n), r)]
            if max(masses) >= tau * W * (1 - 1e-12):
                best = r
                break
        assert cnt == best, (a, tau)
        kept = np.nonzero(keep)[0]
        assert a[kept].sum() >= tau * W * (1 - 1e-12)
        # Among all sets of that size, the kept set carries the largest mass.
        top = max(sum(a[list(s)]) for s in itertools.combinations(range(n), cnt))
        assert a[kept].sum() == pytest.approx(top, rel=1e-12)


def test_ties_prefer_smaller_block_index():
    keep, cnt, _ = _select_row([0.25, 0.25, 0.25, 0.25], 0.5)
    assert list(np.nonzero(keep)[0]) == [0, 1]
    keep, cnt, _ = _select_row([0.125, 0.25, 0.25, 0.25], 0.5)   # needs 0.4375
    assert list(np.nonzero(keep)[0]) == [1, 2]


def test_tau_one_keeps_every_causal_block():
    rng = np.random.default_rng(1)
    nb = 9
    A = np.tril(rng.uniform(0, 1, size=(3, nb, nb)))
    A[:, :, 0] = 0.0  # zero-mass blocks are still kept at tau = 1
    keep, cnt, _ = oracle.select(A, 1.0)
    assert np.array_equal(keep, np.broadcast_to(np.tril(np.ones((nb, nb), np.uint8)), keep.shape))
    assert np.array_equal(cnt, np.broadcast_to(np.arange(1, nb + 1), cnt.shape))


def test_kept_set_is_minimal_prefix_and_monotone_in_tau():
    rng = np.random.default_rng(2)
    nb = 12
    A = np.tril(rng.gamma(0.4, size=(4, nb, nb)))
    prev = None
    for tau in (0.3, 0.5, 0.8, 0.9, 0.95, 0.99):
        keep, cnt, cb = oracle.select(A, tau)
        t32 = float(np.float32(tau))
        for h in range(4):
            for I in range(nb):
                a = A[h, I, :I + 1]
                W = a.sum()
                order = sorted(range(I + 1), key=lambda j: (-a[j], j))
                kept = set(np.nonzero(keep[h, I])[0])
                k = cnt[h, I]
                assert kept == set(order[:k])
                assert a[order[:k]].sum() >= t32 * W * (1 - 1e-12)
                if k > 1:
                    assert a[order[:k - 1]].sum() < t32 * W
                # cbefore is the normalised mass ordered ahead of each block
                for pos, j in enumerate(order):
                    assert cb[h, I, j] == pytest.approx(a[order[:pos]].sum() / W, abs=1e-12)
                assert np.all(cb[h, I, I + 1:] == -1)
        if prev is not None:
            assert np.all(keep >= prev)
        prev = keep


def test_one_hot_row_keeps_single_block():
    nb = 6
    A = np.zeros((1, nb, nb))
    for I in range(nb):
        A[0, I, I // 2] = 2.0
    keep, cnt, _ = oracle.select(A, 0.99)
    assert np.all(cnt == 1)
    for I in range(nb):
        assert list(np.nonzero(keep[0, I])[0]) == [I // 2]


def test_invalid_tau_rejected():
    with pytest.raises(ValueError):
        oracle.select(np.ones((1, 2, 2)), 0.0)
    with pytest.raises(ValueError):
        oracle.select(np.ones((1, 2, 2)), float("nan"))


def test_coverage_fixture_matches_rotation():
    # The oracle's rotation (probed in test_oracle_estimate) covers the
    # offsets listed in the hand-derived fixture.
    path = os.path.join(GOLDEN, "rr_coverage_hand.txt")
    rows = 0
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        head, offs, full = [p.strip() for p in line.split("|")]
        Hq, S = [int(x) for x in head.split()]
        want = [int(x) for x in offs.split()]
        covered = sorted(_sampled_offsets(Hq, S))
        assert covered == want
        assert (full == "yes") == (covered == list(range(S)))
        rows += 1
    assert rows == 5


def _sampled_offsets(Hq, S):
    """Offsets of stride 1 whose query token moves some head's scores."""
    L, d = 2 * S, 4
    rng = np.random.default_rng(3)
    from tests.helpers import bf16
    Q = bf16(rng.standard_normal((L, Hq, d)))
    K = bf16(rng.standard_normal((L, 1, d)))
    out = set()
    for h in range(Hq):
        base = oracle.stride_scores(Q, K, S, h, 1)
        for off in range(S):
            Q2 = Q.copy()
            Q2[S + off, h] = bf16(np.full(d, 2.0))
            if not np.array_equal(oracle.stride_scores(Q2, K, S, h, 1), base):
                out.add(off)
    return out
