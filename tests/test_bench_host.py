"""Host-side logic of bench.py (no GPU): the single-GPU guard, the
kept-block FLOP count, and the source check of the committed traffic
summaries."""
import importlib.util
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one MI355X" in r.stderr and r.stdout == ""


def test_kept_block_flops_counts_causal_pairs():
    b = _bench()
    L, B, d = 320, 128, 64           # nb = 3, last block holds 64 queries
    counts = torch.tensor([[1, 2, 2]], dtype=torch.int32)
    idx = torch.tensor([[[0, -1, -1], [0, 1, -1], [0, 2, -1]]], dtype=torch.int32)
    flops, kept, diag = b.kept_block_flops(counts, idx, L, B, d)
    # block 0: diagonal, 128*129/2 pairs; block 1: one full block + diagonal;
    # block 2 (64 rows): one full block (64*128) + diagonal 64*65/2.
    pairs = 128 * 129 / 2 + (128 * 128 + 128 * 129 / 2) + (64 * 128 + 64 * 65 / 2)
    assert flops == pytest.approx(4.0 * d * pairs)
    assert (kept, diag) == (5, 3)


def test_traffic_summary_requires_matching_source(tmp_path):
    import hashlib
    b = _bench()
    src = open(os.path.join(b.CSRC, "rr_attn.hip"), "rb").read()
    good = hashlib.sha256(src).hexdigest()
    path = tmp_path / "t_{}.md"
    # a per-kernel summary: one source hash
    (tmp_path / "t_wl.md").write_text("- source_sha256: `0000`\n- traffic_bytes_per_launch: 123\n")
    spec = ([str(path)], ["rr_attn.hip"], "attn")
    assert b.measured_traffic("wl", spec, "traffic_bytes_per_launch") is None      # stale hash
    (tmp_path / "t_wl.md").write_text("- source_sha256: `%s`\n- traffic_bytes_per_launch: 123\n" % good)
    assert b.measured_traffic("wl", spec, "traffic_bytes_per_launch") == 123.0
    assert b.measured_traffic("wl", spec, "other_field") is None
    assert b.measured_traffic(None, spec, "traffic_bytes_per_launch") is None       # non-default S / tau
    # an all-kernel summary: per-kind hashes, and a field prefix for the materialised figures
    (tmp_path / "t_wl.md").write_text("- attn_source_sha256: `%s`\n- est_source_sha256: `0000`\n"
                                      "- traffic_bytes_per_step: 7\n- materialized_traffic_bytes_per_step: 9\n"
                                      % good)
    assert b.measured_traffic("wl", ([str(path)], ["rr_attn.hip"], "attn"), "traffic_bytes_per_step") == 7.0
    assert b.measured_traffic("wl", ([str(path)], ["rr_attn.hip"], "attn", "materialized_"),
                              "traffic_bytes_per_step") == 9.0
    assert b.measured_traffic("wl", ([str(path)], ["rr_attn.hip"], "est"), "traffic_bytes_per_step") is None
    # committed summaries
    assert b.measured_traffic("no-such-workload", b.ATTN_TRAFFIC, "traffic_bytes_per_launch") is None
    got = b.measured_traffic("llama8b-128k", b.ATTN_TRAFFIC, "traffic_bytes_per_launch")
    assert got is None or got > 1e9
