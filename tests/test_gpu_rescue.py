"""GPU parity of the RBS-style rescue branch (rr_rescue_estimate) and of the
mask union (rr_merge_masks) against the oracle.

* Rescue scores: max |A_gpu - A_oracle| <= RESCUE_TOL per entry (rows are
  probabilities summing to 1; centroids, radii and logits are fp32 on the
  GPU, so a logit u of size |u| carries ~|u| * 2^-22 of error and a
  probability p about p * that).
* Rescue masks: rr_select on the GPU scores against oracle Top-tau on the
  oracle scores, with the usual 1e-4 boundary rule.
* Union: bit-exact against the oracle's OR of the same two lists.
* End to end: attention under the union of the oracle's round-robin and
  rescue masks within max 1e-2 / mean 1e-3 of the oracle.
"""
import json

import numpy as np
import pytest
import torch

import oracle
from rr_workloads import generate, get_config
from tests.helpers import small_workload
from tests.parity import classify_masks, list_is_well_formed, mask_from_list, o_errors

pytestmark = pytest.mark.gpu

RESCUE_TOL = 1e-5
O_MAX, O_MEAN = 1e-2, 1e-3


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


CASES = [
    # (kind, L, Hq, Hkv, d, B, S, tau, tau_rescue)
    ("llama", 1024, 8, 2, 128, 128, 8, 0.9, 0.5),
    ("llama", 1216, 8, 2, 128, 128, 8, 0.9, 0.8),   # short last block
    ("tiny", 640, 4, 4, 64, 64, 4, 0.9, 0.5),       # d = 64, B = 64, G = 1
    ("video", 2048, 7, 1, 128, 128, 16, 0.9, 0.3),  # G = 7
]


@pytest.mark.parametrize("case", CASES, ids=["-".join(map(str, c)) for c in CASES])
def test_rescue_branch_matches_oracle(case):
    kind, L, Hq, Hkv, d, B, S, tau, tau_r = case
    rr = _rr()
    w, g = small_workload(kind=kind, L=L, Hq=Hq, Hkv=Hkv, d=d, B=B, S=S, seed=29)
    q, k, v = _dev(g["q"]), _dev(g["k"]), _dev(g["v"])
    Ar = rr.rr_rescue_estimate(q, k, B)
    cr, ir = rr.rr_select(Ar, L, B, tau_r)
    A = rr.rr_estimate(q, k, B, S)
    c0, i0 = rr.rr_select(A, L, B, tau)
    cu, iu = rr.rr_merge_masks(c0, i0, cr, ir, L, B)
    torch.cuda.synchronize()
    Ar_o = oracle.rescue_scores(g["q"], g["k"], B)
    err = float(np.abs(Ar.cpu().numpy().astype(np.float64) - Ar_o).max())
    print("  rescue max |dA| = %.3g" % err, flush=True)
    assert err <= RESCUE_TOL
    keep_r, _, cb_r = oracle.select(Ar_o, tau_r)
    crn, irn = cr.cpu().numpy(), ir.cpu().numpy()
    assert list_is_well_formed(crn, irn)
    res = classify_masks(mask_from_list(crn, irn, w.nb), keep_r, cb_r, Ar_o, tau_r)
    print("  rescue mask %s" % {k_: v_ for k_, v_ in res.items() if k_ != "examples"}, flush=True)
    assert res["unexcused"] == 0
    # The union the GPU formed from its own two lists is exactly their OR.
    m0 = mask_from_list(c0.cpu().numpy(), i0.cpu().numpy(), w.nb)
    cun, iun = cu.cpu().numpy(), iu.cpu().numpy()
    assert list_is_well_formed(cun, iun)
    assert np.array_equal(mask_from_list(cun, iun, w.nb), oracle.union_masks(m0, mask_from_list(crn, irn, w.nb)))
    # Attention under the oracle's union mask.
    A_o = oracle.block_scores(g["q"], g["k"], B, S)
    keep_0, _, _ = oracle.select(A_o, tau)
    union_o = oracle.union_masks(keep_0, keep_r)
    cuo, iuo = _lists(union_o)
    O = rr.rr_sparse_attn(q, k, v, B, cuo, iuo, out_dtype=torch.float32)
    torch.cuda.synchronize()
    O_ref = oracle.attention(g["q"], g["k"], g["v"], B, union_o)
    mx, mean = o_errors(O.cpu().numpy(), O_ref)
    print("  density rr %.3f rescue %.3f union %.3f; O max %.3g mean %.3g" % (
        keep_0.mean(), keep_r.mean(), union_o.mean(), mx, mean), flush=True)
    assert mx <= O_MAX and mean <= O_MEAN


@pytest.mark.parametrize("Hq,nb,seed", [(3, 9, 1), (2, 300, 2), (1, 4096, 3)])
def test_merge_is_exact_union(Hq, nb, seed):
    rr = _rr()
    rng = np.random.default_rng(seed)
    tri = np.tril(np.ones((nb, nb), dtype=np.uint8))[None]
    a = (rng.random((Hq, nb, nb)) < 0.3).astype(np.uint8) & tri
    b = (rng.random((Hq, nb, nb)) < 0.1).astype(np.uint8) & tri
    a[:, np.arange(nb), np.arange(nb)] = 1   # non-empty rows, as rr_select returns
    ca, ia = _lists(a)
    cb, ib = _lists(b)
    cu, iu = rr.rr_merge_masks(ca, ia, cb, ib, nb * 64, 64)
    torch.cuda.synchronize()
    cun, iun = cu.cpu().numpy(), iu.cpu().numpy()
    assert list_is_well_formed(cun, iun)
    assert np.array_equal(mask_from_list(cun, iun, nb), oracle.union_masks(a, b))


def test_merge_of_empty_lists_is_empty():
    rr = _rr()
    nb = 5
    c = torch.zeros((2, nb), dtype=torch.int32).cuda()
    i = torch.full((2, nb, nb), -1, dtype=torch.int32).cuda()
    cu, iu = rr.rr_merge_masks(c, i, c, i, nb * 64, 64)
    torch.cuda.synchronize()
    assert int(cu.abs().sum()) == 0 and bool((iu == -1).all())


@pytest.mark.parametrize("cfg", [3, 4])
def test_rescue_at_full_size(cfg):
    """128K and 64K-video workloads: every rescue score against the oracle."""
    rr = _rr()
    w = get_config(cfg)
    g = generate(w)
    q, k = _dev(g["q"]), _dev(g["k"])
    Ar = rr.rr_rescue_estimate(q, k, w.B)
    torch.cuda.synchronize()
    Ar_o = oracle.rescue_scores(g["q"], g["k"], w.B)   # whole array: cheap (block level)
    err = float(np.abs(Ar.cpu().numpy().astype(np.float64) - Ar_o).max())
    print("RESCUE " + json.dumps(dict(workload=w.name, max_abs_err=err)), flush=True)
    assert err <= RESCUE_TOL
