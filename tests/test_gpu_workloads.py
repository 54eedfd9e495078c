"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (rr_prefill on the default stream, bf16 inputs, one layer).

* Block masks: every (head, block-row) at 1K, 8K, 32K and 64K; at 128K the
  oracle scores a deterministic sample (every 16th block-row of every head,
  plus the last).  Rule: equal except for blocks whose oracle cumulative
  boundary is within 1e-4 of tau.
* Block scores: |A_gpu - A_oracle| / W on the same rows.
* Attention: rr_sparse_attn under the oracle's mask (GPU mask outside the
  sampled rows at 128K), compared with the oracle on sampled tokens of the
  sampled rows: max |err| <= 1e-2, mean |err| <= 1e-3 (fp32 output).
Each case prints one JSON line with its counts and errors.
"""
import json

import numpy as np
import pytest
import torch

import oracle
from rr_workloads import generate, get_config
from tests.parity import classify_masks, list_is_well_formed, mask_from_list, o_errors

pytestmark = pytest.mark.gpu

BLOCK_SCORE_TOL = 1e-5
O_MAX, O_MEAN = 1e-2, 1e-3

_inputs = {}


def _gen(cfg):
    if cfg not in _inputs:
        _inputs.clear()
        _inputs[cfg] = generate(get_config(cfg))
    return _inputs[cfg]


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _rows_for(w):
    if w.L <= 65536:
        return None  # every row
    Is = sorted(set(list(range(0, w.nb, 16)) + [w.nb - 1]))
    return [(h, I) for h in range(w.Hq) for I in Is]


def _token_sample(w, rows, per_row=3):
    rng = np.random.default_rng(1234 + w.index)
    toks = []
    for h, I in rows:
        lo, hi = I * w.B, min(w.L, (I + 1) * w.B)
        for t in sorted(set([lo, hi - 1] + list(rng.integers(lo, hi, size=per_row - 2)))):
            toks.append((h, int(t)))
    return toks


POINTS = [(0, None, None), (1, None, None), (2, None, None), (3, None, None), (4, None, None)]
POINTS += [(2, S, tau) for S in (8, 16) for tau in (0.8, 0.9, 0.95) if (S, tau) != (8, 0.9)]


@pytest.mark.parametrize("cfg,S,tau", POINTS, ids=["cfg%d%s" % (c, "" if S is None else "-S%d-tau%g" % (S, t))
                                                    for c, S, t in POINTS])
def test_workload_parity(cfg, S, tau):
    import long_context_prefill_rr_amd as rr
    w = get_config(cfg)
    if S is not None:
        w = w.with_params(S=S, tau=tau)
    print("workload %s L=%d S=%d tau=%g" % (w.name, w.L, w.S, w.tau), flush=True)
    g = _gen(cfg)
    q, k, v = _dev(g["q"]), _dev(g["k"]), _dev(g["v"])
    nb = w.nb

    O, counts, idx = rr.rr_prefill(q, k, v, w.B, w.S, w.tau, out_dtype=torch.float32)
    A_gpu = rr.rr_estimate(q, k, w.B, w.S)
    torch.cuda.synchronize()
    counts_np, idx_np = counts.cpu().numpy(), idx.cpu().numpy()
    assert list_is_well_formed(counts_np, idx_np)
    mask_gpu = mask_from_list(counts_np, idx_np, nb)

    rows = _rows_for(w)
    if rows is None:
        A_orc = oracle.block_scores(g["q"], g["k"], w.B, w.S)
        keep_o, _, cb = oracle.select(A_orc, w.tau)
        A_g = A_gpu.cpu().numpy().astype(np.float64)
        sel_gpu = mask_gpu
        rows_all = [(h, I) for h in range(w.Hq) for I in range(nb)]
        mask_o = keep_o
    else:
        A_orc = oracle.block_scores(g["q"], g["k"], w.B, w.S, rows=rows)
        I_of_row = np.array([I for _, I in rows], dtype=np.int32)
        keep_o, _, cb = oracle.select(A_orc, w.tau, I_of_row=I_of_row)
        hs = np.array([h for h, _ in rows])
        A_g = A_gpu.cpu().numpy()[hs, I_of_row].astype(np.float64)
        sel_gpu = mask_gpu[hs, I_of_row]
        rows_all = rows
        mask_o = mask_gpu.copy()
        mask_o[hs, I_of_row] = keep_o

    W = A_orc.sum(axis=-1, keepdims=True)
    a_err = float((np.abs(A_g - A_orc) / W).max())
    res = classify_masks(sel_gpu, keep_o, cb, A_orc, w.tau)

    # Attention under the oracle's mask, on sampled tokens.
    c_o, i_o = oracle.list_from_mask(mask_o)
    i_o = np.where(np.arange(nb)[None, None, :] < c_o[:, :, None], i_o, -1).astype(np.int32)
    O_om = rr.rr_sparse_attn(q, k, v, w.B, torch.from_numpy(c_o).cuda(), torch.from_numpy(i_o).cuda(),
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    step = max(1, len(rows_all) // 96)
    toks = _token_sample(w, rows_all[::step])
    O_ref = oracle.attention(g["q"], g["k"], g["v"], w.B, mask_o, toks=toks)
    O_om_np = O_om.cpu().numpy()
    got = np.stack([O_om_np[t, h] for h, t in toks])
    o_max, o_mean = o_errors(got, O_ref)
    # The GPU's own end-to-end output under its own mask (information).
    O_np = O.cpu().numpy()
    O_ref_g = oracle.attention(g["q"], g["k"], g["v"], w.B, mask_gpu, toks=toks)
    e2e_max, e2e_mean = o_errors(np.stack([O_np[t, h] for h, t in toks]), O_ref_g)

    out = dict(workload=w.name, L=w.L, S=w.S, tau=w.tau, rows_checked=len(rows_all),
               density=float(mask_gpu.sum()) / (w.Hq * nb * (nb + 1) / 2),
               mask=dict((k_, v_) for k_, v_ in res.items() if k_ != "examples"),
               mask_examples=res["examples"], block_score_err=a_err, tokens_checked=len(toks),
               o_max_err=o_max, o_mean_err=o_mean, e2e_o_max_err=e2e_max, e2e_o_mean_err=e2e_mean)
    print("PARITY " + json.dumps(out), flush=True)
    assert a_err <= BLOCK_SCORE_TOL
    assert res["unexcused"] == 0
    assert o_max <= O_MAX and o_mean <= O_MEAN
