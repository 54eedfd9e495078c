"""Pins of the oracle's attention step E6 against PyTorch's
scaled_dot_product_attention in float64 on the CPU (GQA through
repeat_interleave, block masks through an explicit boolean mask)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from tests.helpers import small_workload, to_f64


def _sdpa(q, k, v, B, mask=None):
    L, Hq, d = q.shape
    G = Hq // k.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    if mask is None:
        o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    else:
        tb = torch.arange(L) // B
        m = torch.from_numpy(mask.astype(bool))[:, tb][:, :, tb]        # [Hq][L][L]
        m = m & torch.ones(L, L, dtype=torch.bool).tril()
        o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m[None])
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("L,B", [(256, 64), (200, 64), (64, 64)])
def test_dense_mask_equals_causal_sdpa(L, B):
    w, g = small_workload(L=L if L % 8 == 0 else 256, Hq=4, Hkv=2, d=32, B=B, S=8)
    q, k, v = g["q"][:L], g["k"][:L], g["v"][:L]
    nb = -(-L // B)
    mask = np.broadcast_to(np.tril(np.ones((nb, nb), np.uint8)), (4, nb, nb)).copy()
    O = oracle.attention(q, k, v, B, mask)
    want = _sdpa(to_f64(q), to_f64(k), to_f64(v), B)
    np.testing.assert_allclose(O, want, rtol=1e-10, atol=1e-12)


def test_random_block_mask_equals_masked_sdpa():
    w, g = small_workload(L=384, Hq=6, Hkv=3, d=32, B=64, S=8)
    rng = np.random.default_rng(4)
    nb = w.nb
    mask = (rng.uniform(size=(w.Hq, nb, nb)) < 0.5).astype(np.uint8)
    mask = np.tril(mask)
    for h in range(w.Hq):
        for I in range(nb):
            if mask[h, I].sum() == 0:
                mask[h, I, rng.integers(0, I + 1)] = 1
    O = oracle.attention(g["q"], g["k"], g["v"], w.B, mask)
    want = _sdpa(to_f64(g["q"]), to_f64(g["k"]), to_f64(g["v"]), w.B, mask)
    np.testing.assert_allclose(O, want, rtol=1e-10, atol=1e-12)


def test_token_list_matches_full_output():
    w, g = small_workload(L=256, Hq=4, Hkv=2, d=32, B=64, S=8)
    nb = w.nb
    mask = np.tril(np.ones((w.Hq, nb, nb), np.uint8))
    mask[1, 3, 1] = 0
    O = oracle.attention(g["q"], g["k"], g["v"], w.B, mask)
    toks = [(1, 200), (0, 0), (3, 255)]
    Or = oracle.attention(g["q"], g["k"], g["v"], w.B, mask, toks=toks)
    for r, (h, t) in enumerate(toks):
        np.testing.assert_array_equal(Or[r], O[t, h])


def test_off_diagonal_only_row_sees_no_own_block():
    # A block-row that keeps only block 0 attends exactly to the first B keys.
    w, g = small_workload(L=256, Hq=2, Hkv=1, d=32, B=64, S=8)
    nb = w.nb
    mask = np.zeros((2, nb, nb), np.uint8)
    mask[:, :, 0] = 1
    O = oracle.attention(g["q"], g["k"], g["v"], w.B, mask, toks=[(0, 130)])
    q, k, v = to_f64(g["q"]), to_f64(g["k"]), to_f64(g["v"])
    l = q[130, 0] @ k[:64, 0].T / np.sqrt(32)
    p = np.exp(l - l.max())
    p /= p.sum()
    np.testing.assert_allclose(O[0], p @ v[:64, 0], rtol=1e-12, atol=1e-13)


def test_mask_list_round_trip():
    rng = np.random.default_rng(5)
    nb = 7
    mask = np.tril((rng.uniform(size=(3, nb, nb)) < 0.4).astype(np.uint8))
    counts, idx = oracle.list_from_mask(mask)
    assert np.array_equal(oracle.mask_from_list(counts, idx, nb), mask)
    for h in range(3):
        for I in range(nb):
            row = idx[h, I, :counts[h, I]]
            assert np.all(np.diff(row) > 0)
