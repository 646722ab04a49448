"""Pins of the oracle's MXFP8 projections (oracle/mxfp8.py) to facts outside it: torch's
float8_e4m3fn dtype (an independent E4M3 codec with round-to-nearest-even), a brute-force
nearest-value search over the 254 finite E4M3 values, the shared-exponent rule's closed
forms, exact integer products and the algebra of the LoRA merge."""
import numpy as np
import pytest
import torch

from oracle import mxfp8 as mx


def grid() -> np.ndarray:
    """All finite E4M3 values with their codes, from torch's codec."""
    codes = np.arange(256, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    ok = np.isfinite(vals)
    return codes[ok], vals[ok]


def test_decode_matches_torch_codec():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(mx.e4m3_decode(codes), want)
    # spot values from the format definition
    assert mx.e4m3_decode([0x7E])[0] == 448.0 and mx.e4m3_decode([0x38])[0] == 1.0
    assert mx.e4m3_decode([0x01])[0] == 2.0 ** -9 and mx.e4m3_decode([0x08])[0] == 2.0 ** -6
    assert mx.e4m3_decode([0xB8])[0] == -1.0 and np.isnan(mx.e4m3_decode([0xFF])[0])


def test_round_matches_torch_cast_in_range():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200_000) * np.exp2(rng.integers(-14, 9, 200_000))
    x = np.concatenate([x[np.abs(x) < 448], [0.0, -0.0, 2.0 ** -10, -2.0 ** -10, 3 * 2.0 ** -11]])
    # torch's cast starts from float32: compare on float32-representable inputs
    x = x.astype(np.float32).astype(np.float64)
    t = torch.from_numpy(x).float().to(torch.float8_e4m3fn)
    np.testing.assert_array_equal(mx.e4m3_round(x), t.double().numpy())
    np.testing.assert_array_equal(mx.e4m3_encode(mx.e4m3_round(x)), t.view(torch.uint8).numpy())


def test_round_is_nearest_with_ties_to_even_by_brute_force():
    codes, vals = grid()
    rng = np.random.default_rng(1)
    # random points plus every midpoint between neighbouring grid values
    pos = np.unique(vals[vals >= 0])
    mids = (pos[1:] + pos[:-1]) / 2
    x = np.concatenate([rng.uniform(-448, 448, 3000), rng.uniform(-0.05, 0.05, 3000), mids, -mids])
    got = mx.e4m3_round(x)
    for xi, gi in zip(x, got):
        dist = np.abs(vals - xi)
        best = vals[dist == dist.min()]
        if best.size == 1:
            assert gi == best[0], xi
        else:  # a tie: the candidate with an even code (mantissa bit 0 clear)
            even = [v for v in best if (mx.e4m3_encode(np.array([v]))[0] & 1) == 0]
            assert gi in even, (xi, best)


def test_saturation():
    x = np.array([448.0, 449.0, 463.99, 464.0, 479.0, 511.0, -500.0])
    np.testing.assert_array_equal(mx.e4m3_round(x), [448, 448, 448, 448, 448, 448, -448])


def test_shared_exponent_closed_forms():
    # amax in [2^e, 2^(e+1)) gives e - 8
    for e in range(-20, 20):
        for f in (1.0, 1.5, 1.999):
            assert mx.mx_shared_exponent(f * 2.0 ** e) == e - 8
    assert mx.mx_shared_exponent(0.0) == -127
    assert mx.mx_shared_exponent(2.0 ** -140) == -127  # clamped
    assert mx.mx_shared_exponent(2.0 ** 200) == 127


def test_block_max_lands_in_top_binade():
    """The largest element of a block becomes a value in [256, 448]; a block whose
    largest element is 448 * 2^s keeps the scale 2^s and that element exactly."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 128)) * np.exp2(rng.integers(-30, 30, (64, 1)))
    codes, scales = mx.mx_quantize(x)
    vals = mx.e4m3_decode(codes).reshape(64, 4, 32)
    top = np.abs(vals).max(axis=2)
    assert np.all((top >= 256) & (top <= 448))
    y = np.zeros((1, 32))
    y[0, 5] = -448 * 2.0 ** -3
    y[0, 6] = 1.0 * 2.0 ** -3
    c, s = mx.mx_quantize(y)
    assert s[0, 0] == 127 - 3 and mx.e4m3_decode(c[0, 5]) == -448 and mx.e4m3_decode(c[0, 6]) == 1


def test_zero_block_and_sign_of_zero():
    x = np.zeros((2, 64))
    x[1, 33] = -1e-30  # rounds to -0 next to a large element
    x[1, 40] = 1.0
    c, s = mx.mx_quantize(x)
    assert s[0].tolist() == [0, 0] and not c[0].any()
    assert c[1, 33] == 0x80 and s[1, 1] == 127 - 8


def test_quantisation_error_bound():
    """Elements not saturated and above the subnormal range keep a relative error of at
    most 2^-4 (3 mantissa bits, round to nearest)."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((32, 256)) * np.exp2(rng.integers(-8, 8, (32, 256)))
    c, s = mx.mx_quantize(x)
    back = mx.mx_dequantize(c, s)
    scale = np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=1)
    normal = (np.abs(x) / scale >= 2.0 ** -6) & (np.abs(x) / scale <= 448)
    assert normal.mean() > 0.5
    assert np.all(np.abs(back - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal])
    sat = np.abs(x) / scale > 448
    assert np.all(np.abs(back[sat]) == 448 * scale[sat])


def test_grid_values_round_trip_exactly():
    """Values that are E4M3 values times the block's own scale come back unchanged."""
    codes, vals = grid()
    rng = np.random.default_rng(4)
    blocks = rng.choice(vals, size=(16, 4, 32))
    blocks[:, :, 0] = 448.0  # fixes each block's scale at 2^0 ...
    e = rng.integers(-40, 40, (16, 4, 1))
    x = (blocks * np.exp2(e)).reshape(16, 128)  # ... then 2^e
    c, s = mx.mx_quantize(x)
    np.testing.assert_array_equal(mx.mx_dequantize(c, s), x)
    np.testing.assert_array_equal(s.astype(np.int64) - 127, e[:, :, 0])


def test_linear_equals_integer_product():
    """Codes whose values are small integers and scales 2^0: the product equals the
    integer matmul computed with Python integers."""
    rng = np.random.default_rng(5)
    ints = np.arange(-16, 17)
    a = rng.choice(ints, (7, 96))
    w = rng.choice(ints, (11, 96))
    ac, wc = mx.e4m3_encode(a.astype(float)), mx.e4m3_encode(w.astype(float))
    ones_a = np.full((7, 3), 127, np.uint8)
    ones_w = np.full((11, 3), 127, np.uint8)
    bias = rng.integers(-5, 5, 11).astype(float)
    got = mx.mx_linear(ac, ones_a, wc, ones_w, bias)
    want = [[sum(int(a[i, k]) * int(w[j, k]) for k in range(96)) + int(bias[j]) for j in range(11)]
            for i in range(7)]
    np.testing.assert_array_equal(got, np.array(want, dtype=float))


def test_block_scale_acts_on_its_block_only():
    rng = np.random.default_rng(6)
    a, w = rng.standard_normal((5, 128)), rng.standard_normal((9, 128))
    ac, as_ = mx.mx_quantize(a)
    wc, ws = mx.mx_quantize(w)
    base = mx.mx_linear(ac, as_, wc, ws)
    as2 = as_.copy()
    as2[3, 2] += 1  # doubles block 2 (elements 64..95) of row 3
    diff = mx.mx_linear(ac, as2, wc, ws) - base
    blk = mx.mx_dequantize(ac, as_)[3, 64:96] @ mx.mx_dequantize(wc, ws)[:, 64:96].T
    np.testing.assert_allclose(diff[3], blk, rtol=1e-12, atol=1e-12)
    assert not np.delete(diff, 3, axis=0).any()


def test_lora_merge_algebra():
    rng = np.random.default_rng(7)
    w = rng.standard_normal((12, 40))
    b, a = rng.standard_normal((12, 4)), rng.standard_normal((4, 40))
    x = rng.standard_normal((3, 40))
    merged = mx.lora_merge(w, b, a, 0.25)
    # x W'^T = x W^T + s (x A^T) B^T
    np.testing.assert_allclose(x @ merged.T, x @ w.T + 0.25 * (x @ a.T) @ b.T, rtol=1e-12, atol=1e-12)
    # rank one: row i of B = e_i adds s * A's row to row i only
    b1 = np.zeros((12, 1))
    b1[5, 0] = 1.0
    m1 = mx.lora_merge(w, b1, a[:1], 2.0)
    np.testing.assert_array_equal(np.delete(m1, 5, axis=0), np.delete(w, 5, axis=0))
    np.testing.assert_allclose(m1[5], w[5] + 2.0 * a[0], rtol=1e-15)


def test_input_projections_split_and_order():
    """Five equal column blocks in weight-row order; with a zero LoRA scale the merge is
    the identity."""
    rng = np.random.default_rng(8)
    x, w = rng.standard_normal((6, 64)), rng.standard_normal((5 * 32, 64))
    outs = mx.input_projections(x, w, lora_b=rng.standard_normal((160, 2)),
                                lora_a=rng.standard_normal((2, 64)), lora_scale=0.0)
    assert len(outs) == 5 and all(o.shape == (6, 32) for o in outs)
    xc, xs = mx.mx_quantize(x)
    for i, o in enumerate(outs):
        wc, ws = mx.mx_quantize(w[32 * i:32 * (i + 1)])
        np.testing.assert_array_equal(o, mx.mx_linear(xc, xs, wc, ws))


@pytest.mark.parametrize("k", [31, 33, 48])
def test_rejects_ragged_rows(k):
    with pytest.raises(ValueError):
        mx.mx_quantize(np.ones((2, k)))


# ---- planted mistakes: each must make at least one pin above fail -----------------------
PINS = [test_decode_matches_torch_codec, test_round_matches_torch_cast_in_range,
        test_round_is_nearest_with_ties_to_even_by_brute_force, test_saturation,
        test_shared_exponent_closed_forms, test_block_max_lands_in_top_binade,
        test_zero_block_and_sign_of_zero, test_quantisation_error_bound,
        test_grid_values_round_trip_exactly, test_linear_equals_integer_product,
        test_block_scale_acts_on_its_block_only, test_lora_merge_algebra,
        test_input_projections_split_and_order]

_o = dict(round=mx.e4m3_round, decode=mx.e4m3_decode, quant=mx.mx_quantize, deq=mx.mx_dequantize,
          linear=mx.mx_linear, merge=mx.lora_merge, shexp=mx.mx_shared_exponent)


def _round_half_away(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    q = np.exp2(np.maximum(ex - 1, -6).astype(np.float64) - 3)
    return np.copysign(np.minimum(np.floor(a / q + 0.5) * q, 448.0), x)


def _round_no_saturation(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    q = np.exp2(np.maximum(ex - 1, -6).astype(np.float64) - 3)
    return np.copysign(np.round(a / q) * q, x)


def _decode_subnormal_as_normal(c):
    c = np.asarray(c, dtype=np.int64)
    v = _o["decode"](c)
    e = (c >> 3) & 0xF
    alt = np.where(c & 0x80, -1.0, 1.0) * (1 + (c & 7) / 8.0) * 2.0 ** -7
    return np.where((e == 0) & ((c & 0x7F) != 0), alt, v)


def _linear_no_bias(a, sa, w, sw, bias=None):
    return _o["linear"](a, sa, w, sw, None)


def _linear_w_scales_of_a(a, sa, w, sw, bias=None):
    return _o["linear"](a, sa, w, np.full_like(sw, 127), bias)


MUTANTS = {
    "scale_exponent_off_by_one": ("EMAX_E4M3", 7),
    "round_half_away": ("e4m3_round", _round_half_away),
    "no_saturation": ("e4m3_round", _round_no_saturation),
    "subnormals_decoded_as_normals": ("e4m3_decode", _decode_subnormal_as_normal),
    "blocks_of_16": ("MX_BLOCK", 16),
    "bias_dropped": ("mx_linear", _linear_no_bias),
    "weight_scales_ignored": ("mx_linear", _linear_w_scales_of_a),
    "lora_sign_flipped": ("lora_merge", lambda w, b, a, s: _o["merge"](w, b, a, -s)),
    "scale_bias_128": ("SCALE_BIAS", 128),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, value = MUTANTS[name]
    monkeypatch.setattr(mx, attr, value)
    failed = []
    for pin in PINS:
        try:
            pin()
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"no pin catches {name}"
