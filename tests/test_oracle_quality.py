"""Pins for the oracle's selection-quality measurement (oracle.mask_quality).

The RRAttention summary page ("Key points") reports precision and F1 of the
blocks a method selects.  The oracle writes those out from their definitions;
these tests tie it to a hand-worked case, to brute-force set arithmetic, and
to properties the Top-tau rule fixes (the reference selection on the exact
mass keeps at least tau of every row's mass).
"""
import os

import numpy as np
import pytest

import oracle
from tests.helpers import small_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mask_quality_hand.txt")


def _read_hand():
    rows, totals, prf = [], None, None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        parts = [p.strip() for p in line.split("|")]
        if parts[0] == "=":
            totals = [float(x) for x in parts[1].split()]
        elif parts[0] == "%":
            prf = [float(x) for x in parts[1].split()]
        else:
            rows.append((int(parts[0]), [float(x) for x in parts[1].split()],
                         [int(x) for x in parts[2].split()], [int(x) for x in parts[3].split()],
                         [float(x) for x in parts[4].split()]))
    return rows, totals, prf


def test_hand_case():
    rows, totals, prf = _read_hand()
    nb = len(rows)
    mass = np.zeros((1, nb, nb))
    mask = np.zeros((1, nb, nb), dtype=np.uint8)
    ref = np.zeros((1, nb, nb), dtype=np.uint8)
    for I, m, t, r, _ in rows:
        mass[0, I, :len(m)] = m
        mask[0, I, t] = 1
        ref[0, I, r] = 1
    got_rows, got_tot = oracle.mask_quality(mask, ref, mass)
    for I, _, _, _, want in rows:
        assert list(got_rows[0, I]) == want
    assert list(got_tot) == totals
    q = oracle.quality_metrics(got_tot, nb)
    assert [q["precision"], q["recall"], q["f1"]] == pytest.approx(prf, abs=1e-15)


def _random_masks(rng, Hq, nb, p):
    m = (rng.random((Hq, nb, nb)) < p).astype(np.uint8)
    m &= np.tril(np.ones((nb, nb), dtype=np.uint8))[None]
    return m


def test_brute_force_sets():
    rng = np.random.default_rng(7)
    Hq, nb = 3, 9
    t = _random_masks(rng, Hq, nb, 0.5)
    r = _random_masks(rng, Hq, nb, 0.4)
    t[:, :, 0] = 1  # every row keeps something
    mass = rng.random((Hq, nb, nb))
    rows, tot = oracle.mask_quality(t, r, mass)
    kept = ref = both = 0
    for h in range(Hq):
        for I in range(nb):
            st = {J for J in range(I + 1) if t[h, I, J]}
            sr = {J for J in range(I + 1) if r[h, I, J]}
            kept += len(st)
            ref += len(sr)
            both += len(st & sr)
            share = sum(mass[h, I, J] for J in st) / sum(mass[h, I, J] for J in range(I + 1))
            assert rows[h, I, 3] == pytest.approx(share, rel=1e-14)
    assert (tot[0], tot[1], tot[2]) == (kept, ref, both)


def test_identical_disjoint_dense():
    rng = np.random.default_rng(3)
    Hq, nb = 2, 6
    causal = np.tril(np.ones((nb, nb), dtype=np.uint8))[None].repeat(Hq, 0)
    m = _random_masks(rng, Hq, nb, 0.5)
    m[:, :, 0] = 1
    mass = rng.random((Hq, nb, nb))
    _, tot = oracle.mask_quality(m, m, mass)
    q = oracle.quality_metrics(tot, Hq * nb)
    assert q["precision"] == q["recall"] == q["f1"] == 1.0
    _, tot = oracle.mask_quality(m, causal - m, mass)
    assert tot[2] == 0
    rows, tot = oracle.mask_quality(causal, m, mass)
    assert np.allclose(rows[..., 3], 1.0, atol=1e-15) and tot[4] == pytest.approx(1.0)
    assert oracle.quality_metrics(tot, Hq * nb)["recall"] == 1.0


def test_reference_on_exact_mass_keeps_tau():
    """S = 1 block scores are the exact causal block mass; Top-tau on them
    keeps >= tau of every row, and the RR mask is scored against it."""
    w, g = small_workload(L=512, Hq=4, Hkv=2, d=64, B=64, S=8, seed=11)
    q, k = g["q"], g["k"]
    exact = oracle.block_scores(q, k, w.B, 1)
    tau = 0.9
    ref, _, _ = oracle.select(exact, tau)
    rows, tot = oracle.mask_quality(ref, ref, exact)
    assert rows[..., 3].min() >= tau * (1 - 1e-12)
    A = oracle.block_scores(q, k, w.B, w.S)
    rr_mask, _, _ = oracle.select(A, tau)
    rows, tot = oracle.mask_quality(rr_mask, ref, exact)
    qm = oracle.quality_metrics(tot, w.Hq * w.nb)
    assert 0.0 < qm["precision"] <= 1.0 and 0.0 < qm["recall"] <= 1.0
    assert qm["f1"] == pytest.approx(2 * qm["precision"] * qm["recall"] / (qm["precision"] + qm["recall"]))
