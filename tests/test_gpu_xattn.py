"""GPU parity of XAttention's antidiagonal estimate (rr_xattn_estimate)
against the oracle, and of the Top-tau masks selected from it.

Block scores: |A_gpu - A_oracle| / W <= 1e-5 (the antidiagonal sums are
exact bf16 products accumulated in fp32 over S*d terms; a block score is a
sum of probabilities).  Masks: the same rule as the round-robin path
(differences only for blocks whose oracle cumulative boundary is within 1e-4
of tau).
"""
import json

import numpy as np
import pytest
import torch

import oracle
from rr_workloads import generate, get_config
from tests.helpers import small_workload
from tests.parity import classify_masks, list_is_well_formed, mask_from_list

pytestmark = pytest.mark.gpu

BLOCK_SCORE_TOL = 1e-5


def _rr():
    import long_context_prefill_rr_amd as rr
    rr.load_library()
    return rr


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


SMALL = [
    # (kind, L, Hq, Hkv, d, B, S, tau)
    ("llama", 1024, 8, 2, 128, 128, 8, 0.9),
    ("llama", 1216, 8, 2, 128, 128, 8, 0.9),   # ragged: 152 strides, short last block
    ("llama", 2048, 4, 1, 128, 128, 16, 0.9),  # c = 8
    ("llama", 1024, 4, 2, 128, 128, 4, 0.9),   # c = 32
    ("tiny", 640, 4, 4, 64, 64, 4, 0.9),       # d = 64, B = 64, G = 1, ragged
    ("video", 2048, 7, 1, 128, 128, 16, 0.95),  # G = 7
    ("llama", 256, 4, 2, 64, 64, 2, 0.8),      # c = 32 at B = 64, fewer strides than a tile
]


@pytest.mark.parametrize("average", [False, True], ids=["sum", "mean"])
@pytest.mark.parametrize("case", SMALL, ids=["-".join(map(str, c)) for c in SMALL])
def test_xattn_estimate_and_mask_match_oracle(case, average):
    kind, L, Hq, Hkv, d, B, S, tau = case
    rr = _rr()
    w, g = small_workload(kind=kind, L=L, Hq=Hq, Hkv=Hkv, d=d, B=B, S=S, seed=13)
    q, k = _dev(g["q"]), _dev(g["k"])
    A = rr.rr_xattn_estimate(q, k, B, S, average=average)
    counts, idx = rr.rr_select(A, L, B, tau)
    torch.cuda.synchronize()
    A_o = oracle.xattn_block_scores(g["q"], g["k"], B, S, average=average)
    W = A_o.sum(axis=-1, keepdims=True)
    err = float((np.abs(A.cpu().numpy().astype(np.float64) - A_o) / W).max())
    print("  xattn max |dA|/W = %.3g" % err, flush=True)
    assert err <= BLOCK_SCORE_TOL
    keep_o, _, cb = oracle.select(A_o, tau)
    cn, inp = counts.cpu().numpy(), idx.cpu().numpy()
    assert list_is_well_formed(cn, inp)
    res = classify_masks(mask_from_list(cn, inp, w.nb), keep_o, cb, A_o, tau)
    print("  mask %s" % res, flush=True)
    assert res["unexcused"] == 0


def test_xattn_rejects_unsupported_stride():
    rr = _rr()
    w, g = small_workload(L=512, Hq=4, Hkv=2, d=64, B=64, S=1)
    q, k = _dev(g["q"]), _dev(g["k"])
    with pytest.raises(rr.RRError):
        rr.rr_xattn_estimate(q, k, 64, 1)   # B/S = 64: not compiled


def _rows_sample(w, every):
    Is = sorted(set(list(range(0, w.nb, every)) + [w.nb - 1]))
    return [(h, I) for h in range(w.Hq) for I in Is]


@pytest.mark.parametrize("cfg,every,average", [(1, 1, False), (1, 1, True), (3, 64, False),
                                               (3, 64, True), (4, 32, False), (4, 32, True)])
def test_xattn_full_size(cfg, every, average):
    rr = _rr()
    w = get_config(cfg)
    g = generate(w)
    q, k = _dev(g["q"]), _dev(g["k"])
    A = rr.rr_xattn_estimate(q, k, w.B, w.S, average=average)
    counts, idx = rr.rr_select(A, w.L, w.B, w.tau)
    torch.cuda.synchronize()
    rows = _rows_sample(w, every)
    hs = np.array([h for h, _ in rows])
    Is = np.array([I for _, I in rows], dtype=np.int32)
    A_o = oracle.xattn_block_scores(g["q"], g["k"], w.B, w.S, rows=rows, average=average)
    A_g = A.cpu().numpy()[hs, Is].astype(np.float64)
    W = A_o.sum(axis=-1, keepdims=True)
    err = float((np.abs(A_g - A_o) / W).max())
    keep_o, _, cb = oracle.select(A_o, w.tau, I_of_row=Is)
    cn, inp = counts.cpu().numpy(), idx.cpu().numpy()
    assert list_is_well_formed(cn, inp)
    mask = mask_from_list(cn, inp, w.nb)
    res = classify_masks(mask[hs, Is], keep_o, cb, A_o, w.tau)
    density = float(mask.sum()) / (w.Hq * w.nb * (w.nb + 1) / 2)
    print("XATTN " + json.dumps(dict(workload=w.name, average=average, rows_checked=len(rows),
                                     block_score_err=err,
                                     density=density,
                                     mask=dict((k_, v_) for k_, v_ in res.items() if k_ != "examples"))),
          flush=True)
    assert err <= BLOCK_SCORE_TOL
    assert res["unexcused"] == 0
