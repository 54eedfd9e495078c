"""Pins of the oracle's estimation steps E1-E4 against facts that do not
re-type the oracle's formulas: exact block attention mass (S=1), a
closed form for constant keys, constructed stride means, probing which query
token each head samples, and the row-sum invariant."""
import numpy as np
import pytest
import torch

import oracle
from tests.helpers import small_workload, to_f64, bf16


def test_pool_keys_recovers_constructed_stride_means():
    # Keys built as (stride mean) + (offsets that cancel inside the stride),
    # with every value exactly representable, so the mean is known exactly.
    rng = np.random.default_rng(0)
    L, Hkv, d, S = 64, 3, 16, 8
    ns = L // S
    means = rng.integers(-8, 8, size=(ns, Hkv, d)).astype(np.float64)
    offs = rng.integers(-4, 5, size=(ns, S // 2, Hkv, d)).astype(np.float64)
    offs = np.concatenate([offs, -offs], axis=1)  # zero sum per stride
    K = (means[:, None] + offs).reshape(L, Hkv, d)
    Kbar = oracle.pool_keys(bf16(K), S)
    assert Kbar.shape == (Hkv, ns, d)
    np.testing.assert_array_equal(Kbar, means.transpose(1, 0, 2))


def test_scores_equal_mean_of_token_logits():
    # Linearity: the score against a pooled key is the average of the S
    # token-level logits of that stride, computed here token by token.
    w, g = small_workload(L=256, Hq=4, Hkv=2, d=32, S=8)
    q, k = to_f64(g["q"]), to_f64(g["k"])
    G = w.Hq // w.Hkv
    for h in range(w.Hq):
        for i in (0, 5, w.L // w.S - 1):
            s = oracle.stride_scores(g["q"], g["k"], w.S, h, i)
            t = i * w.S + h % w.S
            tok = q[t, h] @ k[:, h // G].T / np.sqrt(w.d)       # [L]
            want = tok[: (i + 1) * w.S].reshape(i + 1, w.S).mean(axis=1)
            np.testing.assert_allclose(s, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("Hq,S", [(8, 8), (4, 8), (6, 4), (2, 16)])
def test_each_head_samples_one_token_per_stride(Hq, S):
    # Perturbing one query token changes stride row i of head h only if the
    # token is the one head h samples in stride i: offset h mod S.  The union
    # over heads covers every offset iff Hq >= S.
    L, d = 4 * S, 8
    rng = np.random.default_rng(1)
    Q = bf16(rng.standard_normal((L, Hq, d)))
    K = bf16(rng.standard_normal((L, 1 if Hq % 2 else 2, d)))
    Hkv = K.shape[1]
    i = 2
    covered = set()
    for h in range(Hq):
        base = oracle.stride_scores(Q, K, S, h, i)
        hit = []
        for off in range(S):
            Q2 = Q.copy()
            Q2[i * S + off, h] = bf16(np.full(d, 3.0))
            if not np.array_equal(oracle.stride_scores(Q2, K, S, h, i), base):
                hit.append(off)
        assert hit == [h % S]
        covered.update(hit)
    assert (covered == set(range(S))) == (Hq >= S)


def _exact_block_mass(q, k, B, Hq, Hkv):
    """Dense causal softmax attention probabilities summed over BxB blocks."""
    L, _, d = q.shape
    G = Hq // Hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)                       # [Hq][L][d]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, 0)
    logits = qt @ kt.transpose(1, 2) / np.sqrt(d)
    causal = torch.ones(L, L, dtype=torch.bool).tril()
    P = torch.softmax(logits.masked_fill(~causal, float("-inf")), dim=-1).numpy()
    nb = -(-L // B)
    Pp = np.zeros((Hq, nb * B, nb * B))
    Pp[:, :L, :L] = P
    return Pp.reshape(Hq, nb, B, nb, B).sum(axis=(2, 4))


@pytest.mark.parametrize("L,B", [(256, 64), (288, 64), (64, 64)])
def test_stride_one_gives_exact_block_attention_mass(L, B):
    # With S = 1 every token is sampled and every key is its own stride, so
    # the block scores are the exact causal attention mass per BxB block.
    w, g = small_workload(L=L, Hq=4, Hkv=2, d=32, B=B, S=1)
    A = oracle.block_scores(g["q"], g["k"], B, 1)
    want = _exact_block_mass(to_f64(g["q"]), to_f64(g["k"]), B, w.Hq, w.Hkv)
    np.testing.assert_allclose(A, want, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("B,S,L", [(64, 8, 256), (64, 4, 192), (32, 8, 160)])
def test_constant_keys_closed_form(B, S, L):
    # Equal keys give equal scores, so stride row i spreads 1/(i+1) on each of
    # its i+1 strides.  Hence A[I][J<I] = sum_a c/(Ic+a+1) and
    # A[I][I] = sum_a (a+1)/(Ic+a+1) over the c_I strides a of block I.
    rng = np.random.default_rng(2)
    Hq, Hkv, d = 4, 2, 16
    Q = bf16(rng.standard_normal((L, Hq, d)))
    kvec = bf16(rng.standard_normal((1, Hkv, d)))
    K = np.repeat(kvec, L, axis=0)
    A = oracle.block_scores(Q, K, B, S)
    c, ns, nb = B // S, L // S, -(-L // B)
    want = np.zeros((nb, nb))
    for I in range(nb):
        cI = min(c, ns - I * c)
        for a in range(cI):
            i = I * c + a
            for J in range(I):
                want[I, J] += c / (i + 1)
            want[I, I] += (a + 1) / (i + 1)
    for h in range(Hq):
        np.testing.assert_allclose(A[h], want, rtol=1e-13, atol=1e-15)


def test_block_rows_sum_to_stride_count_and_upper_triangle_is_zero():
    for L in (512, 544):  # 544 = 8.5 blocks of 64: a short last block
        w, g = small_workload(L=L, Hq=4, Hkv=2, d=32, B=64, S=8)
        A = oracle.block_scores(g["q"], g["k"], w.B, w.S)
        c, ns = w.B // w.S, w.L // w.S
        cI = np.array([min(c, ns - I * c) for I in range(w.nb)], dtype=np.float64)
        np.testing.assert_allclose(A.sum(axis=2), np.broadcast_to(cI, (w.Hq, w.nb)), rtol=1e-13)
        assert (A >= 0).all()
        assert np.all(np.triu(A, 1) == 0)


def test_row_list_matches_full_array():
    w, g = small_workload(L=512, Hq=4, Hkv=2, d=32, B=64, S=8)
    A = oracle.block_scores(g["q"], g["k"], w.B, w.S)
    rows = [(3, 7), (0, 0), (2, 4)]
    Ar = oracle.block_scores(g["q"], g["k"], w.B, w.S, rows=rows)
    for r, (h, I) in enumerate(rows):
        np.testing.assert_array_equal(Ar[r], A[h, I])


def test_gqa_query_heads_read_their_own_kv_head():
    # Changing kv-head 1 must change exactly the query heads 2..3 when G = 2.
    w, g = small_workload(L=256, Hq=4, Hkv=2, d=32, B=64, S=8)
    A = oracle.block_scores(g["q"], g["k"], w.B, w.S)
    k2 = g["k"].copy()
    k2[:, 1] = bf16(np.random.default_rng(3).standard_normal((w.L, w.d)))
    A2 = oracle.block_scores(g["q"], k2, w.B, w.S)
    assert np.array_equal(A[:2], A2[:2])
    assert not np.array_equal(A[2:], A2[2:])


def test_thread_count_does_not_change_results():
    w, g = small_workload(L=512, Hq=4, Hkv=2, d=32, B=64, S=8)
    n = oracle.get_threads()
    try:
        oracle.set_threads(1)
        A1 = oracle.block_scores(g["q"], g["k"], w.B, w.S)
        oracle.set_threads(max(2, n))
        A2 = oracle.block_scores(g["q"], g["k"], w.B, w.S)
    finally:
        oracle.set_threads(n)
    assert np.array_equal(A1, A2)


def test_bad_shapes_are_rejected():
    w, g = small_workload(L=256, Hq=4, Hkv=2, d=32, B=64, S=8)
    with pytest.raises(ValueError):
        oracle.block_scores(g["q"], g["k"], 64, 12)  # B % S != 0
    with pytest.raises(ValueError):
        oracle.block_scores(g["q"][:250], g["k"][:250], 64, 8)  # L % S != 0


def test_oracle_regression_fixture():
    # Written by tests/golden/make_oracle_fixtures.py (oracle only).
    import json
    import os
    from rr_workloads import generate, get_config
    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_tiny_1k.json")
    fx = json.load(open(path))
    w = get_config(0)
    g = generate(w)
    A = oracle.block_scores(g["q"], g["k"], w.B, w.S)
    keep, cnt, _ = oracle.select(A, w.tau)
    assert cnt.tolist() == fx["counts"]
    np.testing.assert_allclose(A[0, 7], fx["A_head0_row7"], rtol=1e-12)
    np.testing.assert_allclose(A[5, 3, :4], fx["A_head5_row3"], rtol=1e-12)


def test_batched_stride_scores_equal_single_rows():
    # The batched E2 call forms the pooled keys once and must return exactly
    # the single-row values (same arithmetic, same order).
    w, g = small_workload(kind="llama", L=512, Hq=4, Hkv=2, d=32, B=64, S=8, seed=5)
    rows = [(0, 0), (3, 63), (1, 17), (2, 40), (0, 63)]
    got = oracle.stride_score_rows(g["q"], g["k"], 8, rows)
    for (h, i), s in zip(rows, got):
        assert s.shape == (i + 1,)
        assert np.array_equal(s, oracle.stride_scores(g["q"], g["k"], 8, h, i))
