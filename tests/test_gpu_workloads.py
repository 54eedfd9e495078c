"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (bf16 inputs, one layer, the default stream).

* Block masks: every (head, block-row) of every workload, the 128K one
  included, against the oracle's E1-E5.  Rule: equal except for blocks
  whose oracle cumulative boundary is within 1e-4 of tau.
* Block scores: |A_gpu - A_oracle| / W on every row.
* Attention: rr_sparse_attn under the oracle's mask (fp32 output), against
  the oracle's E6: every (token, head) at 1K and 8K; at 32K, 64K and 128K
  every token of a deterministic sample of whole block-rows spread over all
  heads and block-rows (the first and the last block-row included).  Bar:
  max |err| <= 1e-2, mean |err| <= 1e-3.  rr_prefill's own output under its
  own mask is held to the same bar on the same tokens.
* The benchmark's own call (rr_prefill with bf16 output): its kept lists
  equal the fp32 call's and its output equals the fp32 output rounded to
  bf16, bit for bit, on every element.
Each case prints one JSON line with its counts and errors.
"""
import json

import numpy as np
import pytest
import torch

import oracle
from rr_workloads import generate, get_config
from tests.parity import (classify_masks, list_from_mask, list_is_well_formed, mask_from_list,
                          o_errors)

pytestmark = pytest.mark.gpu

BLOCK_SCORE_TOL = 1e-5
O_MAX, O_MEAN = 1e-2, 1e-3
FULL_O_MAX_L = 8192       # every (token, head) compared up to this length
SAMPLED_ROWS = 128        # whole block-rows compared above it

_inputs = {}


def _gen(cfg):
    if cfg not in _inputs:
        _inputs.clear()
        _inputs[cfg] = generate(get_config(cfg))
    return _inputs[cfg]


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _row_sample(w):
    """Whole block-rows for the attention comparison above FULL_O_MAX_L:
    SAMPLED_ROWS (head, block-row) pairs spread over every head and over the
    block-rows by a fixed stride, plus block-row 0 and the last block-row of
    head 0 and of the last head."""
    rows = set()
    for r in range(SAMPLED_ROWS):
        rows.add((r % w.Hq, (r * 37 + 11) % w.nb))
    rows.update({(0, 0), (0, w.nb - 1), (w.Hq - 1, 0), (w.Hq - 1, w.nb - 1)})
    return sorted(rows)


def _tokens(w, rows):
    toks = []
    for h, I in rows:
        for t in range(I * w.B, min(w.L, (I + 1) * w.B)):
            toks.append((h, t))
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
    # The benchmark's configuration: the same call with bf16 output.  The
    # kept lists must repeat exactly, and O must be the fp32 output rounded
    # to bf16 (round to nearest even): the two kernels differ only in the
    # final store.
    Ob, counts_b, idx_b = rr.rr_prefill(q, k, v, w.B, w.S, w.tau, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    bf16_lists_equal = bool(torch.equal(counts_b, counts) and torch.equal(idx_b, idx))
    bf16_out_equal = bool(torch.equal(Ob, O.to(torch.bfloat16)))
    del Ob, counts_b, idx_b
    A_gpu = rr.rr_estimate(q, k, w.B, w.S)
    torch.cuda.synchronize()
    counts_np, idx_np = counts.cpu().numpy(), idx.cpu().numpy()
    assert list_is_well_formed(counts_np, idx_np)
    mask_gpu = mask_from_list(counts_np, idx_np, nb)
    A_g = A_gpu.cpu().numpy().astype(np.float64)
    del A_gpu

    # E1-E5 on every row.
    print("  oracle estimate + select on all %d rows" % (w.Hq * nb), flush=True)
    A_orc = oracle.block_scores(g["q"], g["k"], w.B, w.S)
    keep_o, _, cb = oracle.select(A_orc, w.tau)
    W = A_orc.sum(axis=-1, keepdims=True)
    a_err = float((np.abs(A_g - A_orc) / W).max())
    del A_g
    res = classify_masks(mask_gpu, keep_o, cb, A_orc, w.tau)
    del cb, A_orc, W

    # Attention under the oracle's mask, and the end-to-end output.
    c_o, i_o = list_from_mask(keep_o)
    O_om = rr.rr_sparse_attn(q, k, v, w.B, torch.from_numpy(c_o).cuda(), torch.from_numpy(i_o).cuda(),
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    O_om_np, O_np = O_om.cpu().numpy(), O.cpu().numpy()
    del O_om, O
    if w.L <= FULL_O_MAX_L:
        print("  oracle attention on every (token, head)", flush=True)
        O_ref = oracle.attention(g["q"], g["k"], g["v"], w.B, keep_o)
        o_max, o_mean = o_errors(O_om_np, O_ref)
        O_ref_g = oracle.attention(g["q"], g["k"], g["v"], w.B, mask_gpu)
        e2e_max, e2e_mean = o_errors(O_np, O_ref_g)
        n_rows_o, n_tok = w.Hq * nb, w.L * w.Hq
    else:
        rows_o = _row_sample(w)
        toks = _tokens(w, rows_o)
        print("  oracle attention on %d whole block-rows (%d tokens)" % (len(rows_o), len(toks)),
              flush=True)
        tt = np.array([t for _, t in toks])
        hh = np.array([h for h, _ in toks])
        O_ref = oracle.attention(g["q"], g["k"], g["v"], w.B, keep_o, toks=toks)
        o_max, o_mean = o_errors(O_om_np[tt, hh], O_ref)
        O_ref_g = oracle.attention(g["q"], g["k"], g["v"], w.B, mask_gpu, toks=toks)
        e2e_max, e2e_mean = o_errors(O_np[tt, hh], O_ref_g)
        n_rows_o, n_tok = len(rows_o), len(toks)

    out = dict(workload=w.name, L=w.L, S=w.S, tau=w.tau, rows_checked=w.Hq * nb,
               density=float(mask_gpu.sum()) / (w.Hq * nb * (nb + 1) / 2),
               mask=dict((k_, v_) for k_, v_ in res.items() if k_ != "examples"),
               mask_examples=res["examples"], block_score_err=a_err,
               o_block_rows_checked=n_rows_o, o_tokens_checked=n_tok,
               o_max_err=o_max, o_mean_err=o_mean, e2e_o_max_err=e2e_max, e2e_o_mean_err=e2e_mean,
               bf16_call_lists_equal=bf16_lists_equal, bf16_call_out_equal_rounded_f32=bf16_out_equal)
    print("PARITY " + json.dumps(out), flush=True)
    assert a_err <= BLOCK_SCORE_TOL
    assert res["unexcused"] == 0
    assert o_max <= O_MAX and o_mean <= O_MEAN
    assert e2e_max <= O_MAX and e2e_mean <= O_MEAN
    assert bf16_lists_equal and bf16_out_equal
