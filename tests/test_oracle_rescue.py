"""Pins for the oracle's RBS-style rescue branch (oracle.rescue_scores).

Reading of the RBS-Attention page (abstract and method summary): the rescue
logit of (query block I, key block J) is the largest logit the block's mean
query can reach against any key of block J, bounded through the block's
maximum key radius: sigma * (qc . kc_J + ||qc|| * r_J); the rescue scores
are its softmax over J <= I.  The pins build inputs whose centroids and
radii are known by construction.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.helpers import bf16, small_workload, to_f64


def _known_blocks(rng, L, B, Hq, Hkv, d, radius):
    """Block J holds one key at kc_J + radius_J * e_J, one at
    kc_J - radius_J * e_J (e_J a unit vector) and the rest at kc_J, so its
    centroid is kc_J and its radius (largest distance) exactly radius_J while
    its mean distance is far smaller; every query of block I equals qc_I.
    All values are dyadic, exact in bf16."""
    nb = -(-L // B)
    kc = np.round(rng.standard_normal((nb, Hkv, d)) * 4) / 4
    qc = np.round(rng.standard_normal((nb, Hq, d)) * 4) / 4
    K = np.zeros((L, Hkv, d))
    Q = np.zeros((L, Hq, d))
    for J in range(nb):
        n1 = min(L, (J + 1) * B)
        for g in range(Hkv):
            e = np.zeros(d)
            e[(J * 7 + g) % d] = 1.0
            for n in range(J * B, n1):
                sgn = {0: 1.0, 1: -1.0}.get(n - J * B, 0.0)
                K[n, g] = kc[J, g] + sgn * radius[J, g] * e
        Q[J * B:n1] = qc[J][None]
    return bf16(Q), bf16(K), qc, kc


@pytest.mark.parametrize("zero_radius,L", [(True, 512), (False, 512), (False, 480)])
def test_known_centroids_and_radii(zero_radius, L):
    # L = 480: the last block holds 32 tokens, whose mean and radius alone count.
    rng = np.random.default_rng(3)
    B, Hq, Hkv, d = 64, 4, 2, 16
    nb = -(-L // B)
    radius = np.zeros((nb, Hkv)) if zero_radius else rng.integers(0, 9, (nb, Hkv)) / 4.0
    Q, K, qc, kc = _known_blocks(rng, L, B, Hq, Hkv, d, radius)
    A = oracle.rescue_scores(Q, K, B)
    G = Hq // Hkv
    for h in range(Hq):
        g = h // G
        for I in range(nb):
            u = torch.tensor([(qc[I, h] @ kc[J, g] + np.linalg.norm(qc[I, h]) * radius[J, g]) / np.sqrt(d)
                              for J in range(I + 1)], dtype=torch.float64)
            want = torch.softmax(u, dim=0).numpy()
            np.testing.assert_allclose(A[h, I, :I + 1], want, rtol=1e-12, atol=1e-15)
            assert np.all(A[h, I, I + 1:] == 0)


def test_rows_sum_to_one_and_permutation_invariance():
    w, g = small_workload(L=640, Hq=4, Hkv=2, d=32, B=64, S=8, seed=21)
    A = oracle.rescue_scores(g["q"], g["k"], 64)
    np.testing.assert_allclose(A.sum(axis=-1), 1.0, rtol=1e-12)
    assert A.min() >= 0
    # Reordering keys inside a block or queries inside a block changes nothing.
    rng = np.random.default_rng(1)
    k2, q2 = g["k"].copy(), g["q"].copy()
    for J in range(w.nb):
        p = rng.permutation(64) + J * 64
        k2[J * 64:(J + 1) * 64] = g["k"][p]
        q2[J * 64:(J + 1) * 64] = g["q"][rng.permutation(64) + J * 64]
    np.testing.assert_allclose(oracle.rescue_scores(q2, k2, 64), A, rtol=1e-12, atol=1e-15)


def test_short_last_block_uses_its_tokens_only():
    w, g = small_workload(L=576, Hq=2, Hkv=1, d=16, B=128, S=8, seed=8)   # last block: 64 tokens
    A = oracle.rescue_scores(g["q"], g["k"], 128)
    # Appending tokens after L must not change any score of the full blocks'
    # rows, while the last row sees its 64 tokens only (same as a 64-token block
    # at the end of a longer, B-aligned input whose extra tokens are cut off).
    assert A.shape == (2, 5, 5)
    np.testing.assert_allclose(A.sum(axis=-1), 1.0, rtol=1e-12)
    A_full = oracle.rescue_scores(g["q"][:512], g["k"][:512], 128)
    np.testing.assert_allclose(A[:, :4, :4], A_full, rtol=1e-12, atol=1e-15)


def test_union_of_masks():
    a = np.array([[[1, 0, 0], [0, 1, 0], [1, 0, 1]]], dtype=np.uint8)
    b = np.array([[[1, 0, 0], [1, 0, 0], [0, 1, 0]]], dtype=np.uint8)
    assert oracle.union_masks(a, b).tolist() == [[[1, 0, 0], [1, 1, 0], [1, 1, 1]]]
