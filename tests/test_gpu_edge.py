"""GPU edge cases against the oracle: degenerate shapes of the method and
the largest supported block count.

* one block (L = B), one short block (L < B), a single stride (L = S),
  fewer query heads than the stride (Hq < S: the round-robin offsets cover
  only Hq of the S positions), one head, eight query heads per kv-head;
* tau so small that exactly one block (the largest, earliest on ties) is
  kept per row;
* rr_select on rows of equal scores, all-zero rows included;
* rr_select on long rows (nb up to 4096) of dyadic scores drawn from a few
  levels, so most cuts fall inside a run of ties: every sum is exact in
  fp32 and fp64 alike, so the lists must equal the oracle's exactly;
* nb = 4096 (L = 524288 at B = 128), the largest list the selection takes:
  end to end, checked on sampled block-rows and tokens.
Rules as for the other parity tests: masks equal up to blocks within 1e-4 of
the tau boundary, block scores to 1e-5 of the row total, attention outputs
max |err| <= 1e-2 and mean <= 1e-3 (fp32 output).
"""
import numpy as np
import pytest
import torch

import oracle
from tests.helpers import small_workload
from tests.parity import classify_masks, list_is_well_formed, mask_from_list, o_errors

pytestmark = pytest.mark.gpu

BLOCK_SCORE_TOL = 1e-5
O_MAX, O_MEAN = 1e-2, 1e-3


def _rr():
    import long_context_prefill_rr_amd as rr
    rr.load_library()
    return rr


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


DEGENERATE = [
    # (kind, L, Hq, Hkv, d, B, S, tau)
    ("llama", 128, 4, 2, 128, 128, 8, 0.9),    # one block
    ("llama", 64, 4, 2, 128, 128, 8, 0.9),     # one short block
    ("llama", 8, 2, 1, 64, 64, 8, 0.9),        # one stride, one short block
    ("llama", 1024, 2, 1, 64, 128, 8, 0.9),    # Hq < S
    ("llama", 512, 1, 1, 64, 64, 4, 0.9),      # a single head
    ("llama", 1024, 8, 1, 128, 128, 8, 0.9),   # G = 8: four head pairs
    ("llama", 1216, 8, 2, 128, 128, 8, 1e-6),  # tau -> one block per row
]


@pytest.mark.parametrize("case", DEGENERATE, ids=["-".join(map(str, c)) for c in DEGENERATE])
def test_degenerate_shapes_end_to_end(case):
    kind, L, Hq, Hkv, d, B, S, tau = case
    rr = _rr()
    w, g = small_workload(kind=kind, L=L, Hq=Hq, Hkv=Hkv, d=d, B=B, S=S, seed=17)
    w = w.with_params(tau=tau)
    print("case %s" % (case,), flush=True)
    A_orc = oracle.block_scores(g["q"], g["k"], B, S)
    keep_o, cnt_o, cb = oracle.select(A_orc, tau)
    q, k, v = _dev(g["q"]), _dev(g["k"]), _dev(g["v"])
    A = rr.rr_estimate(q, k, B, S)
    O, counts, idx = rr.rr_prefill(q, k, v, B, S, tau, out_dtype=torch.float32)
    torch.cuda.synchronize()
    W = A_orc.sum(axis=2, keepdims=True)
    err = float((np.abs(A.cpu().numpy().astype(np.float64) - A_orc) / W).max())
    assert err <= BLOCK_SCORE_TOL
    counts, idx = counts.cpu().numpy(), idx.cpu().numpy()
    assert list_is_well_formed(counts, idx)
    mask = mask_from_list(counts, idx, w.nb)
    res = classify_masks(mask, keep_o, cb, A_orc, tau)
    print("  |dA|/W %.3g mask %s" % (err, {k_: v_ for k_, v_ in res.items() if k_ != "examples"}),
          flush=True)
    assert res["unexcused"] == 0
    if tau < 1e-3:
        assert np.all(counts == 1)
    O_ref = oracle.attention(g["q"], g["k"], g["v"], B, mask)
    mx, mean = o_errors(O.cpu().numpy(), O_ref)
    print("  O max %.3g mean %.3g" % (mx, mean), flush=True)
    assert mx <= O_MAX and mean <= O_MEAN


def test_select_equal_and_zero_rows():
    rr = _rr()
    nb, B, L = 6, 64, 6 * 64
    A = np.zeros((2, nb, nb), dtype=np.float32)
    for I in range(nb):
        A[1, I, :I + 1] = 0.25          # equal scores: the earliest blocks win
    for tau in (0.3, 0.5, 0.9, 1.0):
        counts, idx = rr.rr_select(torch.from_numpy(A).cuda(), L, B, tau)
        torch.cuda.synchronize()
        keep_o, cnt_o, _ = oracle.select(A.astype(np.float64), tau)
        counts, idx = counts.cpu().numpy(), idx.cpu().numpy()
        assert list_is_well_formed(counts, idx)
        assert np.array_equal(mask_from_list(counts, idx, nb), keep_o.astype(np.uint8))
        assert np.array_equal(counts, cnt_o)


@pytest.mark.parametrize("nb", [64, 1000, 4096])
def test_select_exact_on_dyadic_rows_with_ties(nb):
    """Scores are multiples of 2^-6 no larger than 1 and tau is a multiple of
    2^-4, so row totals, running sums and tau * total are exact in fp32 (at
    most 22 significant bits) and the selection has one right answer."""
    rr = _rr()
    rng = np.random.default_rng(100 + nb)
    levels = np.array([0.0, 1 / 64, 1 / 16, 0.25, 0.5, 1.0], dtype=np.float32)
    Hq = 2
    A = rng.choice(levels, size=(Hq, nb, nb)).astype(np.float32)
    A *= np.tril(np.ones((nb, nb), dtype=np.float32))[None]
    A[1, nb // 3] = 0.0                     # an all-zero row: the first block is kept
    A[0, nb - 1, : nb // 2] = 0.25          # a long run of equal scores at the start of the last row
    A_dev = torch.from_numpy(A).cuda()
    print("select dyadic nb=%d" % nb, flush=True)
    for tau in (0.5, 0.75, 0.875, 0.9375):
        counts, idx = rr.rr_select(A_dev, nb * 64, 64, tau)
        torch.cuda.synchronize()
        counts, idx = counts.cpu().numpy(), idx.cpu().numpy()
        keep_o, cnt_o, _ = oracle.select(A.astype(np.float64), tau)
        assert list_is_well_formed(counts, idx)
        assert np.array_equal(counts, cnt_o), tau
        assert np.array_equal(mask_from_list(counts, idx, nb), keep_o.astype(np.uint8)), tau
        assert counts[1, nb // 3] == 1 and idx[1, nb // 3, 0] == 0


def test_largest_block_count():
    """nb = 4096 (L = 524288, B = 128): the longest Top-tau rows and lists."""
    rr = _rr()
    L, B, S, tau = 524288, 128, 16, 0.9
    w, g = small_workload(kind="llama", L=L, Hq=2, Hkv=1, d=64, B=B, S=S, seed=23)
    assert w.nb == 4096
    q, k, v = _dev(g["q"]), _dev(g["k"]), _dev(g["v"])
    O, counts, idx = rr.rr_prefill(q, k, v, B, S, tau, out_dtype=torch.float32)
    A = rr.rr_estimate(q, k, B, S)
    torch.cuda.synchronize()
    counts, idx = counts.cpu().numpy(), idx.cpu().numpy()
    assert list_is_well_formed(counts, idx)
    rows = [(0, 0), (1, 1), (0, 2047), (1, 4094), (0, 4095), (1, 4095)]
    hs = np.array([h for h, _ in rows])
    Is = np.array([I for _, I in rows], dtype=np.int32)
    A_o = oracle.block_scores(g["q"], g["k"], B, S, rows=rows)
    W = A_o.sum(axis=-1, keepdims=True)
    err = float((np.abs(A.cpu().numpy()[hs, Is].astype(np.float64) - A_o) / W).max())
    keep_o, _, cb = oracle.select(A_o, tau, I_of_row=Is)
    mask = mask_from_list(counts, idx, w.nb)
    res = classify_masks(mask[hs, Is], keep_o, cb, A_o, tau)
    print("  nb=4096 |dA|/W %.3g mask %s kept(h0,4095)=%d" % (
        err, {k_: v_ for k_, v_ in res.items() if k_ != "examples"}, counts[0, 4095]), flush=True)
    assert err <= BLOCK_SCORE_TOL
    assert res["unexcused"] == 0
    toks = []
    for h, I in rows:
        lo = I * B
        toks += [(h, lo), (h, lo + 63), (h, lo + B - 1)]
    O_ref = oracle.attention(g["q"], g["k"], g["v"], B, mask, toks=toks)
    O_np = O.cpu().numpy()
    got = np.stack([O_np[t, h] for h, t in toks])
    mx, mean = o_errors(got, O_ref)
    print("  O on %d tokens: max %.3g mean %.3g" % (len(toks), mx, mean), flush=True)
    assert mx <= O_MAX and mean <= O_MEAN
