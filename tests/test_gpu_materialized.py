"""GPU parity of rr_estimate_materialized: the stride scores it writes to
memory and the block scores it pools from them, against the fp64 oracle.

* Stride scores (E2, in base-2 units): for every sampled row (h, i) and every
  stride j <= i, |s_gpu - log2(e) s_oracle| is within the worst-case bound of
  an fp32 dot product of 3d exact bf16 x bf16 terms (the three pooled-key
  planes) plus the rounding of the fp32 pooled key and of the scaling:
      (3d + 2) 2^-24 log2(e) sum_k |q_k Kbar_k| / sqrt(d) + 3 2^-24 |s|.
  Strides j > i inside the row's block-row are -inf exactly.
* Block scores: |A - A_oracle| / W <= 1e-5 (the bar of rr_estimate), and
  within 1e-6 of rr_estimate's own A (same products, other summation order).
* Masks: rr_select on these block scores against the oracle's Top-tau, with
  the usual boundary excusal.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from rr_workloads import generate, get_config
from tests.helpers import small_workload, to_f64
from tests.parity import classify_masks, mask_from_list

pytestmark = pytest.mark.gpu

LOG2E = 1.0 / math.log(2.0)
U = 2.0 ** -24
BLOCK_SCORE_TOL = 1e-5
SAME_PATH_TOL = 1e-6


def _rr():
    import long_context_prefill_rr_amd as rr
    rr.load_library()
    return rr


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _score_offset(c, I, a, j):
    return c * c * I * (I + 1) // 2 + a * (I + 1) * c + j


def _check_rows(sc_dev, g, w, rows):
    """Compare the stored scores of stride rows (h, i) with the oracle."""
    c, S, d = w.B // w.S, w.S, w.d
    SP = c * c * w.nb * (w.nb + 1) // 2
    q64 = to_f64(g["q"])
    abs_kbar = np.abs(oracle.pool_keys(g["k"], S))   # [Hkv][ns][d]
    wants = oracle.stride_score_rows(g["q"], g["k"], S, rows)
    G = w.Hq // w.Hkv
    # Small buffers come over whole; large ones row by row.
    host = sc_dev.cpu().numpy() if sc_dev.numel() <= (1 << 28) else None
    worst = 0.0
    for n, ((h, i), want) in enumerate(zip(rows, wants)):
        I, a = divmod(i, c)
        span = (I + 1) * c
        base = h * SP + _score_offset(c, I, a, 0)
        src = host[base:base + span] if host is not None else sc_dev[base:base + span].cpu().numpy()
        got = src.astype(np.float64)
        want = want * LOG2E
        qrow = q64[i * S + (h % S), h]
        l1 = (abs_kbar[h // G, :i + 1] @ np.abs(qrow)) / math.sqrt(d)   # sum_k |q_k Kbar_k| / sqrt(d)
        tol = (3 * d + 2) * U * LOG2E * l1 + 3 * U * np.abs(want) + 1e-30
        err = np.abs(got[:i + 1] - want)
        assert np.all(err <= tol), (h, i, float((err / tol).max()))
        worst = max(worst, float((err / tol).max()))
        assert np.all(np.isneginf(got[i + 1:span])), (h, i)
        if n % 4096 == 4095:
            print("  %d / %d rows checked" % (n + 1, len(rows)), flush=True)
    return worst


SMALL = [
    # (kind, L, Hq, Hkv, d, B, S, tau)
    ("llama", 1216, 8, 2, 128, 128, 8, 0.9),   # ragged last block, c = 16
    ("llama", 1024, 8, 2, 128, 128, 16, 0.8),  # c = 8
    ("tiny", 640, 4, 4, 64, 64, 4, 0.9),       # G = 1, ragged, c = 16
    ("video", 2048, 7, 1, 128, 128, 16, 0.95),  # G = 7
    ("llama", 320, 4, 1, 64, 64, 1, 0.9),      # S = 1, c = 64
    ("llama", 512, 4, 2, 64, 64, 2, 0.9),      # c = 32
    ("llama", 512, 4, 2, 128, 128, 1, 0.9),    # c = 128
    ("llama", 1024, 6, 3, 64, 128, 32, 0.5),   # c = 4
]


@pytest.mark.parametrize("case", SMALL, ids=[str(c) for c in SMALL])
def test_materialized_matches_oracle(case):
    rr = _rr()
    kind, L, Hq, Hkv, d, B, S, tau = case
    w, g = small_workload(kind=kind, L=L, Hq=Hq, Hkv=Hkv, d=d, B=B, S=S, seed=13)
    w = w.with_params(tau=tau)
    print("materialized %s" % (case,), flush=True)
    q, k = _dev(g["q"]), _dev(g["k"])
    sc, A = rr.rr_estimate_materialized(q, k, B, S)
    A_fused = rr.rr_estimate(q, k, B, S)
    torch.cuda.synchronize()
    assert sc.numel() == rr.stride_scores_count(L, Hq, Hkv, d, B, S)

    ns = L // S
    rows = [(h, i) for h in range(Hq) for i in range(ns)]
    ratio = _check_rows(sc, g, w, rows)

    A_orc = oracle.block_scores(g["q"], g["k"], B, S)
    A_np = A.cpu().numpy().astype(np.float64)
    W = A_orc.sum(axis=2, keepdims=True)
    err = float((np.abs(A_np - A_orc) / W).max())
    same = float((np.abs(A_np - A_fused.cpu().numpy()) / W).max())
    print("  scores: worst err/bound %.3g; max |dA|/W %.3g; vs rr_estimate %.3g" % (ratio, err, same),
          flush=True)
    assert err <= BLOCK_SCORE_TOL
    assert same <= SAME_PATH_TOL
    assert np.all(np.triu(A_np, 1) == 0)

    counts, idx = rr.rr_select(A, L, B, tau)
    keep_o, _, cb = oracle.select(A_orc, tau)
    res = classify_masks(mask_from_list(counts.cpu().numpy(), idx.cpu().numpy(), w.nb), keep_o, cb,
                         A_orc, tau)
    assert res["unexcused"] == 0, res


def test_materialized_unsupported_stride_count():
    rr = _rr()
    w, g = small_workload(kind="llama", L=512, Hq=4, Hkv=2, d=128, B=64, S=32, seed=3)
    with pytest.raises(rr.RRError):
        rr.rr_estimate_materialized(_dev(g["q"]), _dev(g["k"]), 64, 32)   # B/S = 2


@pytest.mark.parametrize("cfg", [1, 3])
def test_materialized_workload(cfg):
    """8K: every stride row of every head; 128K: stride rows 37 + 64m of
    every head (with the last row), and the block scores and masks of every
    16th block-row.  All of A is compared with rr_estimate's."""
    rr = _rr()
    w = get_config(cfg)
    print("materialized workload %s" % w.name, flush=True)
    g = generate(w)
    q, k = _dev(g["q"]), _dev(g["k"])
    sc, A = rr.rr_estimate_materialized(q, k, w.B, w.S)
    A_fused = rr.rr_estimate(q, k, w.B, w.S)
    torch.cuda.synchronize()
    ns, nb = w.L // w.S, w.nb
    if cfg == 1:
        srows = [(h, i) for h in range(w.Hq) for i in range(ns)]
        brows = None
    else:
        srows = [(h, i) for h in range(w.Hq) for i in list(range(37, ns, 64)) + [ns - 1]]
        Is = sorted(set(list(range(0, nb, 16)) + [nb - 1]))
        brows = [(h, I) for h in range(w.Hq) for I in Is]
    ratio = _check_rows(sc, g, w, srows)
    del sc
    torch.cuda.empty_cache()

    A_np = A.cpu().numpy().astype(np.float64)
    Wf = np.maximum(A_fused.cpu().numpy().astype(np.float64).sum(axis=2, keepdims=True), 1e-30)
    same = float((np.abs(A_np - A_fused.cpu().numpy()) / Wf).max())
    counts, idx = rr.rr_select(A, w.L, w.B, w.tau)
    mask = mask_from_list(counts.cpu().numpy(), idx.cpu().numpy(), nb)
    if brows is None:
        A_orc = oracle.block_scores(g["q"], g["k"], w.B, w.S)
        keep_o, _, cb = oracle.select(A_orc, w.tau)
        A_g, sel = A_np, mask
    else:
        A_orc = oracle.block_scores(g["q"], g["k"], w.B, w.S, rows=brows)
        I_of_row = np.array([I for _, I in brows], dtype=np.int32)
        hs = np.array([h for h, _ in brows])
        keep_o, _, cb = oracle.select(A_orc, w.tau, I_of_row=I_of_row)
        A_g, sel = A_np[hs, I_of_row], mask[hs, I_of_row]
    W = A_orc.sum(axis=-1, keepdims=True)
    err = float((np.abs(A_g - A_orc) / W).max())
    res = classify_masks(sel, keep_o, cb, A_orc, w.tau)
    print("  rows %d: scores worst err/bound %.3g; max |dA|/W %.3g; vs rr_estimate %.3g; masks %s"
          % (len(srows), ratio, err, same, res), flush=True)
    assert err <= BLOCK_SCORE_TOL
    assert same <= SAME_PATH_TOL
    assert res["unexcused"] == 0, res
