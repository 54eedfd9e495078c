"""GPU parity of the selection-quality measurement (rr_mask_quality).

* On given masks and block masses the per-row counts (kept, reference, both)
  must equal the oracle's exactly and the kept mass share agree to 1e-6
  (fp32 sums of at most a few thousand terms in [0, 1]).
* End to end (1K and 8K workloads): the round-robin mask and the reference
  mask (Top-tau on the exact block mass, rr_estimate with S = 1) are each
  compared with the oracle's under the usual mask rule, and the quality
  numbers the GPU reports on the oracle's masks equal the oracle's.
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

SHARE_TOL = 1e-6
BLOCK_SCORE_TOL = 1e-5


def _rr():
    import long_context_prefill_rr_amd as rr
    rr.load_library()
    return rr


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _lists(mask):
    c, i = oracle.list_from_mask(mask)
    nb = mask.shape[-1]
    i = np.where(np.arange(nb)[None, None, :] < c[:, :, None], i, -1).astype(np.int32)
    return torch.from_numpy(c).cuda(), torch.from_numpy(i).cuda()


def _compare_rows(rows_gpu, totals_gpu, rows_o, totals_o):
    rg = rows_gpu.cpu().numpy().astype(np.float64)
    assert np.array_equal(rg[..., :3], rows_o[..., :3])
    assert np.abs(rg[..., 3] - rows_o[..., 3]).max() <= SHARE_TOL
    tg = totals_gpu.cpu().numpy()
    assert list(tg[:3]) == list(totals_o[:3])
    assert abs(tg[3] - totals_o[3]) <= SHARE_TOL * rows_o.shape[0] * rows_o.shape[1]
    assert abs(tg[4] - totals_o[4]) <= SHARE_TOL


@pytest.mark.parametrize("Hq,nb,p,seed", [(3, 9, 0.5, 1), (4, 70, 0.3, 2), (2, 300, 0.6, 3)])
def test_rows_match_oracle_on_random_masks(Hq, nb, p, seed):
    rr = _rr()
    rng = np.random.default_rng(seed)
    tri = np.tril(np.ones((nb, nb), dtype=np.uint8))[None]
    t = (rng.random((Hq, nb, nb)) < p).astype(np.uint8) & tri
    r = (rng.random((Hq, nb, nb)) < p).astype(np.uint8) & tri
    t[:, :, 0] = 1
    r[:, np.arange(nb), np.arange(nb)] = 1
    mass = (rng.random((Hq, nb, nb)) * tri).astype(np.float32)
    ct, it = _lists(t)
    cr, ir = _lists(r)
    B = 64
    rows, totals = rr.rr_mask_quality(ct, it, cr, ir, torch.from_numpy(mass).cuda(), nb * B - 5, B)
    torch.cuda.synchronize()
    rows_o, totals_o = oracle.mask_quality(t, r, mass.astype(np.float64))
    _compare_rows(rows, totals, rows_o, totals_o)


def test_ignores_out_of_range_and_repeated_entries():
    rr = _rr()
    nb, B = 5, 64
    counts = torch.tensor([[1, 2, 3, 3, 4]], dtype=torch.int32).cuda()
    idx = torch.full((1, nb, nb), -1, dtype=torch.int32)
    idx[0, 0, :1] = torch.tensor([0])
    idx[0, 1, :2] = torch.tensor([1, 1])          # repeated
    idx[0, 2, :3] = torch.tensor([0, 4, 2])       # 4 > I: ignored
    idx[0, 3, :3] = torch.tensor([-1, 3, 0])      # -1: ignored
    idx[0, 4, :4] = torch.tensor([0, 1, 2, 4])
    idx = idx.cuda()
    mass = torch.tril(torch.ones(1, nb, nb)).cuda()
    rows, totals = rr.rr_mask_quality(counts, idx, counts, idx, mass, nb * B, B)
    torch.cuda.synchronize()
    got = rows.cpu().numpy()
    assert list(got[0, :, 0]) == [1, 1, 2, 2, 4]
    assert np.allclose(got[0, :, 3], [1.0, 0.5, 2 / 3, 0.5, 0.8])


@pytest.mark.parametrize("cfg", [0, 1])
def test_selection_quality_end_to_end(cfg):
    rr = _rr()
    w = get_config(cfg)
    g = generate(w)
    q, k = _dev(g["q"]), _dev(g["k"])
    A_rr = rr.rr_estimate(q, k, w.B, w.S)
    exact = rr.rr_estimate(q, k, w.B, 1)
    c_rr, i_rr = rr.rr_select(A_rr, w.L, w.B, w.tau)
    c_ref, i_ref = rr.rr_select(exact, w.L, w.B, w.tau)
    _, totals = rr.rr_mask_quality(c_rr, i_rr, c_ref, i_ref, exact, w.L, w.B)
    torch.cuda.synchronize()
    nrows = w.Hq * w.nb
    gpu_q = rr.quality_summary(totals.cpu().numpy(), nrows)

    A_o = oracle.block_scores(g["q"], g["k"], w.B, w.S)
    ex_o = oracle.block_scores(g["q"], g["k"], w.B, 1)
    keep_rr, _, cb_rr = oracle.select(A_o, w.tau)
    keep_ref, _, cb_ref = oracle.select(ex_o, w.tau)
    W = ex_o.sum(axis=-1, keepdims=True)
    ex_err = float((np.abs(exact.cpu().numpy() - ex_o) / W).max())
    assert ex_err <= BLOCK_SCORE_TOL
    for (c, i), keep, cb, A in (((c_rr, i_rr), keep_rr, cb_rr, A_o),
                                ((c_ref, i_ref), keep_ref, cb_ref, ex_o)):
        cn, inp = c.cpu().numpy(), i.cpu().numpy()
        assert list_is_well_formed(cn, inp)
        res = classify_masks(mask_from_list(cn, inp, w.nb), keep, cb, A, w.tau)
        assert res["unexcused"] == 0, res

    rows_o, totals_o = oracle.mask_quality(keep_rr, keep_ref, ex_o)
    orc_q = oracle.quality_metrics(totals_o, nrows)
    ct, it = _lists(keep_rr)
    cr, ir = _lists(keep_ref)
    rows_g, totals_g = rr.rr_mask_quality(ct, it, cr, ir, torch.from_numpy(ex_o.astype(np.float32)).cuda(),
                                          w.L, w.B)
    torch.cuda.synchronize()
    _compare_rows(rows_g, totals_g, rows_o, totals_o)
    print("QUALITY " + json.dumps(dict(workload=w.name, gpu=gpu_q, oracle=orc_q, exact_mass_err=ex_err)),
          flush=True)
