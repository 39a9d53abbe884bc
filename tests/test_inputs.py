"""Seeded input generator: determinism, rounding, moments, skew recipe (CPU)."""
import math

import numpy as np
import torch

import seeded_inputs as si


def test_deterministic_and_row_addressable():
    c = si.CONFIGS["main_n8192"].replace(seqlen_kv=512, seqlen_q=512)
    a = si.host_view_rows(c, "k")
    b = si.host_view_rows(c, "k")
    np.testing.assert_array_equal(a, b)
    rows = np.array([5, 0, 511, 17])
    np.testing.assert_array_equal(si.host_view_rows(c, "k", rows), a[rows])


def test_bf16_is_round_to_nearest_even_of_fp32():
    """The bf16 value is the library's RNE conversion of the fp32 value of the same element."""
    c32 = si.CONFIGS["main_n8192"].replace(seqlen_kv=256, seqlen_q=256, dtype=si.F32)
    c16 = c32.replace(dtype=si.BF16)
    f = si.host_view_rows(c32, "v")
    h = si.host_view_rows(c16, "v")
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(h, ref)


def test_moments_of_irwin_hall_normal():
    x = si.normals_f64(123, 1, 0, 200000)
    assert abs(x.mean()) < 0.01
    assert abs(x.var() - 1.0) < 0.01
    assert np.abs(x).max() < 6.0
    # fourth moment of Irwin-Hall(12)-6 is 3 - 1.2/12 = 2.9
    assert abs(np.mean(x ** 4) - 2.9) < 0.05


def test_skew_recipe():
    c = si.CONFIGS["skewed_n131072"]
    hot = si.hot_block_list(c)
    assert hot[0] == 0 and len(set(hot.tolist())) == 65 and hot.max() < c.num_blocks
    sh = si.skew_shift(c)
    assert math.isclose(float(np.linalg.norm(sh)), 3 * c.scale, rel_tol=1e-12)
    f = si.q_idx_boost_flags(c, np.arange(100000))
    assert 0.48 < f.mean() < 0.52
    # boosted K_idx rows carry the shift: mean projection on u is ~3 sigma
    u = sh / np.linalg.norm(sh)
    rows = np.arange(0, 128)  # block 0 is always hot
    kv = si.as_f32(c, si.host_view_rows(c, "k_idx", rows)).astype(np.float64)
    assert abs(float((kv @ u).mean()) - 3 * c.scale) < 0.3
