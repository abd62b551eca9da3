"""The seeded input generators: encodings, shapes, distributions (no GPU)."""
import numpy as np

from moe_inputs import (LAYER_CONFIGS, bf16_bits_from_f32, make_layer_inputs,
                        zipf_target_shares)


def test_bf16_encoder_round_to_nearest_even():
    # exactly representable values survive; halfway cases go to even
    vals = np.array([1.0, -2.5, 0.0, 3.140625], dtype=np.float32)
    assert np.array_equal(bf16_bits_from_f32(vals), [0x3F80, 0xC020, 0x0000, 0x4049])
    u = np.array([0x3F808000, 0x3F818000, 0x3F808001, 0x3F807FFF], dtype=np.uint32)
    got = bf16_bits_from_f32(u.view(np.float32))
    assert np.array_equal(got, [0x3F80, 0x3F82, 0x3F81, 0x3F80])


def test_shapes_and_ranges():
    inp = make_layer_inputs(T=5, E=4, k=2, seed=1, H=64, I=32)
    assert inp["x"].shape == (5, 64) and inp["x"].dtype == np.uint16
    assert inp["Wr"].shape == (4, 64) and inp["Wr"].dtype == np.float32
    assert inp["w13_codes"].shape == (4, 64, 32) and inp["w13_scales"].shape == (4, 64, 2)
    assert inp["w2_codes"].shape == (4, 64, 16) and inp["w2_scales"].shape == (4, 64, 1)
    assert inp["b13"].shape == (4, 64) and inp["b2"].shape == (4, 64)
    for key in ("w13_scales", "w2_scales"):
        assert inp[key].min() >= 119 and inp[key].max() <= 122


def test_seeded_and_distinct():
    a = make_layer_inputs(T=3, E=4, k=2, seed=7, H=64, I=32)
    b = make_layer_inputs(T=3, E=4, k=2, seed=7, H=64, I=32)
    c = make_layer_inputs(T=3, E=4, k=2, seed=8, H=64, I=32)
    for key in a:
        assert np.array_equal(a[key], b[key])
    assert not np.array_equal(a["x"], c["x"])


def test_code_nibbles_uniform():
    inp = make_layer_inputs(T=1, E=2, k=1, seed=2, H=256, I=256)
    c = inp["w13_codes"].ravel()
    for nib in (c & 15, c >> 4):
        hist = np.bincount(nib, minlength=16) / nib.size
        assert np.all(np.abs(hist - 1 / 16) < 0.01)


def test_zipf_shares_capped_and_normalised():
    for E, s in ((128, 1.1), (128, 1.3), (32, 2.0)):
        sh = zipf_target_shares(E, 4, s)
        assert np.isclose(sh.sum(), 1.0) and sh.max() <= 0.25 + 1e-12
        assert np.all(np.diff(sh) <= 1e-15)


def test_config_table():
    assert [c.T for c in LAYER_CONFIGS] == [16, 64, 4096, 8192, 16384]
    assert [c.E for c in LAYER_CONFIGS] == [32, 32, 32, 128, 128]
    assert all(c.k == 4 for c in LAYER_CONFIGS)
