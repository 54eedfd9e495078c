"""Pins for the oracle's XAttention estimator (X1 antidiagonal scoring, then
the same stride softmax, block pooling and Top-tau as the round-robin path).

XAttention review page, "importance prediction" and "threshold block
selection" steps 1-2: inside each S x S sub-block of the attention map the
antidiagonal elements (lower-left to upper-right) are summed; a softmax over
the sums gives probabilities that find_blocks thresholds.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.helpers import bf16, small_workload, to_f64


def _dense_logits(q, k, h, G):
    d = q.shape[2]
    return (q[:, h, :] @ k[:, h // G, :].T) / np.sqrt(d)


@pytest.mark.parametrize("S,L", [(4, 64), (8, 128), (2, 40)])
def test_antidiagonal_matches_brute_force(S, L):
    # Read the sums straight off the dense logit matrix: sub-block (i, j) is
    # rows iS..iS+S-1 x cols jS..jS+S-1, its antidiagonal runs from the
    # bottom-left element (iS+S-1, jS) to the top-right one (iS, jS+S-1).
    w, g = small_workload(L=L, Hq=4, Hkv=2, d=16, B=S * 4, S=S, seed=5)
    q, k = to_f64(g["q"]), to_f64(g["k"])
    ns = L // S
    for h in (0, 3):
        logits = _dense_logits(q, k, h, 2)
        for i in (0, ns // 2, ns - 1):
            got = oracle.xattn_stride_scores(g["q"], g["k"], S, h, i)
            want = np.array([sum(logits[i * S + S - 1 - u, j * S + u] for u in range(S))
                             for j in range(i + 1)])
            np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
            main_diag = np.array([sum(logits[i * S + u, j * S + u] for u in range(S))
                                  for j in range(i + 1)])
            assert not np.allclose(got, main_diag)
            mean = oracle.xattn_stride_scores(g["q"], g["k"], S, h, i, average=True)
            np.testing.assert_allclose(mean, want / S, rtol=1e-12, atol=1e-12)


def _exact_block_mass(q, k, B, Hq, Hkv):
    L, _, d = q.shape
    G = Hq // Hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, 0)
    logits = qt @ kt.transpose(1, 2) / np.sqrt(d)
    causal = torch.ones(L, L, dtype=torch.bool).tril()
    P = torch.softmax(logits.masked_fill(~causal, float("-inf")), dim=-1).numpy()
    nb = -(-L // B)
    Pp = np.zeros((Hq, nb * B, nb * B))
    Pp[:, :L, :L] = P
    return Pp.reshape(Hq, nb, B, nb, B).sum(axis=(2, 4))


@pytest.mark.parametrize("L,B,average", [(256, 64, False), (288, 64, False), (256, 64, True)])
def test_stride_one_is_exact_block_mass(L, B, average):
    # With S = 1 each sub-block is one logit: the estimate is exact attention.
    w, g = small_workload(L=L, Hq=4, Hkv=2, d=32, B=B, S=1)
    A = oracle.xattn_block_scores(g["q"], g["k"], B, 1, average=average)
    want = _exact_block_mass(to_f64(g["q"]), to_f64(g["k"]), B, w.Hq, w.Hkv)
    np.testing.assert_allclose(A, want, rtol=1e-10, atol=1e-12)


def test_stride_constant_inputs_scale_round_robin_scores():
    # If every token of a stride carries the same query and the same key, the
    # antidiagonal sum is S times the stride logit, which is the round-robin
    # score (any sampled query, mean key): x = S * s.
    rng = np.random.default_rng(4)
    L, Hq, Hkv, d, S = 96, 4, 2, 16, 4
    ns = L // S
    Qs = rng.standard_normal((ns, Hq, d))
    Ks = rng.standard_normal((ns, Hkv, d))
    Q = bf16(np.repeat(Qs, S, axis=0))
    K = bf16(np.repeat(Ks, S, axis=0))
    for h in range(Hq):
        for i in (0, 7, ns - 1):
            x = oracle.xattn_stride_scores(Q, K, S, h, i)
            s = oracle.stride_scores(Q, K, S, h, i)
            np.testing.assert_allclose(x, S * s, rtol=1e-12, atol=1e-12)
            xm = oracle.xattn_stride_scores(Q, K, S, h, i, average=True)
            np.testing.assert_allclose(xm, s, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("S,B,L,average", [(8, 64, 512, False), (4, 64, 320, False),
                                           (16, 128, 1024, False), (8, 64, 512, True)])
def test_rows_sum_to_strides_and_row_list(S, B, L, average):
    w, g = small_workload(L=L, Hq=4, Hkv=2, d=32, B=B, S=S, seed=9)
    A = oracle.xattn_block_scores(g["q"], g["k"], B, S, average=average)
    c = B // S
    ns = L // S
    for I in range(w.nb):
        cI = min(c, ns - I * c)
        np.testing.assert_allclose(A[:, I, :].sum(axis=-1), cI, rtol=1e-12)
        assert np.all(A[:, I, I + 1:] == 0)
    assert A.min() >= 0
    rows = [(3, w.nb - 1), (0, 0), (2, 1)]
    Ar = oracle.xattn_block_scores(g["q"], g["k"], B, S, rows=rows, average=average)
    for r, (h, I) in enumerate(rows):
        np.testing.assert_array_equal(Ar[r], A[h, I])


def test_differs_from_round_robin_on_generic_inputs():
    w, g = small_workload(L=512, Hq=4, Hkv=2, d=32, B=64, S=8, seed=3)
    A_x = oracle.xattn_block_scores(g["q"], g["k"], 64, 8)
    A_r = oracle.block_scores(g["q"], g["k"], 64, 8)
    assert np.abs(A_x - A_r).max() > 1e-3
