"""The seeded input generator (rr_workloads): determinism, bf16 rounding,
RoPE, and the placement of the scaled sink / vertical keys (CPU only)."""
import numpy as np
import pytest
import torch

from rr_workloads import get_config, generate, f32_to_bf16_bits, bf16_bits_to_f32
from rr_workloads.gen import _rope


def _small(kind="llama", **kw):
    base = {"tiny": 0, "llama": 1, "video": 4}[kind]
    p = dict(L=1024, Hq=4, Hkv=2, d=32, seed=3)
    p.update(kw)
    w = get_config(base).with_params(**p)
    if kind == "llama":
        w = w.with_params(n_vertical=min(w.n_vertical, 16))
    if kind == "video":
        w = w.with_params(frame_len=64)
    return w


@pytest.mark.parametrize("kind", ["tiny", "llama", "video"])
def test_same_seed_same_inputs_other_seed_other_inputs(kind):
    w = _small(kind)
    a, b = generate(w), generate(w)
    for key in ("q", "k", "v"):
        assert np.array_equal(a[key], b[key])
    c = generate(w.with_params(seed=w.seed + 1))
    assert not np.array_equal(a["q"], c["q"])
    assert not np.array_equal(a["k"], c["k"])


def test_chunked_draws_do_not_depend_on_length():
    # Noise is drawn in 4096-token chunks: a longer sequence starts with the
    # shorter one's queries (queries do not depend on the vertical positions).
    short = generate(_small("tiny", L=4096))
    long = generate(_small("tiny", L=8192))
    assert np.array_equal(long["q"][:4096], short["q"])
    assert np.array_equal(long["k"][:4096], short["k"])


def test_bf16_rounding_is_round_to_nearest_even():
    one = np.float32(1.0).view(np.uint32)
    hand = {
        0x3F800000: 0x3F80,          # 1.0
        0x3F808000: 0x3F80,          # halfway, even below
        0x3F818000: 0x3F82,          # halfway, even above
        0x3F808001: 0x3F81,          # just above halfway
        0x3F807FFF: 0x3F80,          # just below halfway
        0xBF818000: 0xBF82,          # negative, halfway
        0x7F7FFFFF: 0x7F80,          # largest float rounds to inf
        0x7F800000: 0x7F80,          # inf
    }
    x = np.array(list(hand.keys()), dtype=np.uint32).view(np.float32)
    got = f32_to_bf16_bits(x)
    assert [int(g) for g in got] == list(hand.values())
    assert one == 0x3F800000
    # Against torch's float32 -> bfloat16 conversion on random values.
    rng = np.random.default_rng(0)
    r = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    want = torch.from_numpy(r).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(r), want)
    # Widening is exact.
    assert np.array_equal(bf16_bits_to_f32(want), torch.from_numpy(want.view(np.int16)).view(torch.bfloat16)
                          .to(torch.float32).numpy())


def test_rope_rotates_pairs_by_the_stated_angles():
    d, base = 32, 10000.0
    rng = np.random.default_rng(1)
    x = rng.standard_normal((40, 3, d)).astype(np.float32)
    t0 = 17
    y = _rope(x, t0, base).astype(np.float64)
    x = x.astype(np.float64)
    half = d // 2
    # Norm of every (f, f + d/2) pair is preserved.
    nx = x[..., :half] ** 2 + x[..., half:] ** 2
    ny = y[..., :half] ** 2 + y[..., half:] ** 2
    assert np.allclose(nx, ny, rtol=1e-5)
    # Rotation angle of pair f at token t0 + n is (t0 + n) * base^(-2f/d).
    ang_x = np.arctan2(x[..., half:], x[..., :half])
    ang_y = np.arctan2(y[..., half:], y[..., :half])
    want = (np.arange(t0, t0 + 40)[:, None] * base ** (-2.0 * np.arange(half) / d))[:, None, :]
    diff = np.angle(np.exp(1j * (ang_y - ang_x - want)))
    assert np.abs(diff).max() < 1e-4
    # Dot products depend only on the position difference.
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, d)).astype(np.float32)
    d1 = float((_rope(q, 100, base) * _rope(k, 90, base)).sum())
    d2 = float((_rope(q, 510, base) * _rope(k, 500, base)).sum())
    assert abs(d1 - d2) < 1e-4 * (abs(d1) + 1)


def test_sink_and_vertical_keys_are_scaled_by_exactly_four():
    w = _small("llama", L=2048, Hkv=2, Hq=4)
    g4 = generate(w)
    g1 = generate(w.with_params(key_scale=1.0))
    assert np.array_equal(g4["sinks"], np.arange(w.n_sinks))
    vert = g4["verticals"]
    assert vert.shape == (w.Hkv, w.n_vertical)
    for g in range(w.Hkv):
        assert len(set(vert[g].tolist())) == w.n_vertical
        assert vert[g].min() >= w.n_sinks and vert[g].max() < w.L
    k4, k1 = bf16_bits_to_f32(g4["k"]), bf16_bits_to_f32(g1["k"])
    scaled = np.zeros((w.L, w.Hkv), dtype=bool)
    scaled[g4["sinks"], :] = True
    for g in range(w.Hkv):
        scaled[vert[g], g] = True
    # A power-of-two scale commutes with bf16 rounding: exactly 4x there,
    # identical elsewhere; queries and values untouched.
    assert np.array_equal(k4[scaled], 4.0 * k1[scaled])
    assert np.array_equal(k4[~scaled], k1[~scaled])
    assert np.array_equal(g4["q"], g1["q"]) and np.array_equal(g4["v"], g1["v"])


def test_video_keys_share_frame_and_slot_vectors():
    # Without noise and with RoPE switched off by a huge base (all angles but
    # the first pair's vanish), K[t] = F_{t // frame} + P_{t % frame}: tokens
    # of one frame differ only by their slot vectors.
    w = _small("video", L=256, noise_std=0.0, rope_base=1e300)
    g = generate(w)
    k = bf16_bits_to_f32(g["k"]).astype(np.float64)[..., 1:16]   # pairs 1..15 (unrotated halves)
    f = w.frame_len
    # (K[t] - K[t + f]) is the same for every slot t of frame 0 vs frame 1: F_0 - F_1.
    dif = k[0:f] - k[f:2 * f]
    assert np.abs(dif - dif[0:1]).max() < 0.1
    # and K[t] - K[t'] for two slots is the same in every frame: P_s - P_s'.
    ds = k[0::f] - k[1::f]
    assert np.abs(ds - ds[0:1]).max() < 0.1
