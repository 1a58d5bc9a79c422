"""Pins of the oracle's NVFP4 quantiser: page-stated shapes and scale
direction, exact-arithmetic re-derivation of scales and codes, invariants."""
import os

import numpy as np

from oracle import formats, quant, moe

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [l.split() for l in f if l.strip() and not l.startswith("#")]


def _data(rows, cols, seed=0, outliers=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    if outliers:
        pos = rng.choice(x.size, max(1, x.size // 1000), replace=False)
        x.reshape(-1)[pos] *= 20
    x[0, :16] = 0.0                       # an all-zero block
    x[1, 16:32] *= np.float32(1e-6)       # a block whose scale is subnormal or zero
    return x


def test_packed_shapes_match_page_table():
    rng = np.random.default_rng(3)
    for name, lr, lc, pr, pc, mb in _rows("shared_expert_shapes.txt"):
        lr, lc, pr, pc, mb = int(lr), int(lc), int(pr), int(pc), int(mb)
        # quantise a thin slice of the real width; the packed width follows
        w = (rng.standard_normal((4, lc)) * 0.02).astype(np.float32)
        c, s, _ = moe.quantize_weight(w)
        assert c.shape == (4, pc) and s.shape == (4, lc // 16)
        assert round(lr * pc / 1e6) == mb


def test_scale_direction_page_example_saturates_without_nan():
    (stored, mult), = _rows("scale_direction.txt")
    gs = np.float32(float(stored))
    assert round(1.0 / float(gs), 1) == float(mult)
    # Activations far larger than 6*448*gs can encode: the quantiser divides by
    # gs (the multiplier is 1/gs) and saturates at scale 448 / code +-6.
    x = (np.random.default_rng(4).standard_normal((8, 64)) * 50).astype(np.float32)
    c, s = quant.quantize(x, gs)
    deq = quant.dequantize(c, s, gs)
    assert np.isfinite(deq).all()
    assert (s <= 0x7E).all() and (s == 0x7E).any()
    assert np.abs(deq).max() <= 6 * 448 * float(gs) * (1 + 1e-6)
    codes = quant.unpack_codes(c)
    assert ((codes & 7) == 7).any()


def test_global_scale_definition():
    assert quant.global_scale(2688.0) == np.float32(1.0)
    assert quant.global_scale(0.0) == np.float32(1.0)
    a = np.float32(3.7)
    assert quant.global_scale(a) == np.float32(a / np.float32(2688.0))


def test_nibble_order_and_block_layout():
    # one row of 32: block 0 holds 6,-0.5,1,0,... (scale 1 with gs = 1), block 1 zero
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, :4] = [6.0, -0.5, 1.0, 0.0]
    c, s = quant.quantize(x, np.float32(1.0))
    # bamax 6 -> s = 6/6 = 1 -> E4M3 0x38; codes 7, 0x9, 2, 0
    assert s.tolist() == [[0x38, 0x00]]
    assert c[0, 0] == (7 | (0x9 << 4)) and c[0, 1] == 2
    assert (c[0, 8:] == 0).all()


def test_scales_and_codes_follow_exact_arithmetic():
    """Re-derive every scale and code in float64 with exhaustive nearest
    search; disagreements are allowed only where the float64 value sits within
    a float32 rounding of a tie."""
    x = _data(64, 512, seed=5)
    gs = quant.global_scale(quant.amax(x) * np.float32(0.7))    # some saturation too
    c, s = quant.quantize(x, gs)
    xb = x.astype(np.float64).reshape(64, 32, 16)
    s64 = np.abs(xb).max(axis=2) / (6.0 * float(gs))
    vals = formats.E4M3_POS_VALUES
    d = np.abs(np.minimum(s64, 448.0)[..., None] - vals)
    near = np.argmin(d, axis=-1)
    second = np.sort(d, axis=-1)[..., 1]
    tie_zone = np.abs(d.min(axis=-1) - second) <= 4e-7 * np.maximum(s64, 1e-30)
    assert ((near == s) | tie_zone).all()
    sf = formats.e4m3_decode(s)
    with np.errstate(invalid="ignore", divide="ignore"):
        v64 = np.where(sf[..., None] > 0, xb / (sf[..., None] * float(gs)), 0.0)
    mags = formats.E2M1_MAGNITUDE
    dv = np.abs(np.abs(v64)[..., None] - mags)
    nearv = np.argmin(dv, axis=-1)
    tie_v = np.abs(np.sort(dv, axis=-1)[..., 0] - np.sort(dv, axis=-1)[..., 1]) <= 1e-6 * np.abs(v64)
    codes = quant.unpack_codes(c).reshape(64, 32, 16)
    assert (((codes & 7) == nearv) | tie_v).all()
    nz = sf[..., None].repeat(16, -1) > 0
    assert (((codes >> 3) == np.signbit(xb)) | ~nz).all()


def test_idempotent_on_normal_unsaturated_blocks():
    x = _data(128, 256, seed=6)
    gs = quant.global_scale(quant.amax(x))
    c, s = quant.quantize(x, gs)
    d = quant.dequantize(c, s, gs).astype(np.float32)
    c2, s2 = quant.quantize(d, gs)
    sf = formats.e4m3_decode(s)
    normal = (sf >= 2.0 ** -6) & (s < 0x7E)
    cb = quant.unpack_codes(c).reshape(128, 16, 16)
    cb2 = quant.unpack_codes(c2).reshape(128, 16, 16)
    assert np.array_equal(s[normal], s2[normal])
    assert np.array_equal(cb[normal], cb2[normal])
    # every such block contains a +-6 code
    assert ((cb[normal] & 7) == 7).any(axis=-1).all()


def test_error_bound_per_element():
    x = _data(64, 1024, seed=7)
    gs = quant.global_scale(quant.amax(x))
    c, s = quant.quantize(x, gs)
    d = quant.dequantize(c, s, gs)
    sf = np.repeat(formats.e4m3_decode(s), 16, axis=1)
    bound = np.where(sf > 0, float(gs) * sf, np.abs(x).astype(np.float64))
    assert (np.abs(x - d) <= bound * (1 + 1e-6) + 1e-30).all()
    assert (s <= 0x7E).all()


def test_zero_block_gives_zero_codes_and_scale():
    x = _data(4, 64, seed=8)
    c, s = quant.quantize(x, quant.global_scale(quant.amax(x)))
    assert s[0, 0] == 0 and (c[0, :8] == 0).all()


def test_reciprocal_overflow_keeps_zero_codes_and_saturates_the_rest():
    """A global scale so small that 1/(sf*gs) overflows float32: each step is
    still one float32 operation, so a non-zero element times inf saturates to
    6 (index 7) with its sign, and a zero element (either sign) keeps the
    magnitude code of zero instead of the NaN that 0 * inf would give."""
    gs = np.float32(1e-40)                                  # a float32 subnormal
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 1], x[0, 2], x[0, 3] = np.float32(5e-39), np.float32(-1e-39), np.float32(-0.0)
    x[0, 16:] = np.linspace(-1, 1, 16, dtype=np.float32)   # an ordinary block
    c, s = quant.quantize(x, gs)
    sf = formats.e4m3_decode(s[0, 0])
    with np.errstate(over="ignore"):
        assert sf > 0 and not np.isfinite(np.float32(1.0) / np.float32(np.float32(sf) * gs))
    codes = np.empty(32, dtype=np.uint8)
    codes[0::2], codes[1::2] = c[0] & 0xF, c[0] >> 4
    assert codes[0] == 0 and codes[1] == 0x7 and codes[2] == 0xF and codes[3] == 0x8
    assert (codes[4:16] == 0).all()
    assert s[0, 1] == 0x7E and (codes[16:] & 7).max() == 7   # 1/(448*gs) is finite


def test_brute_force_tiny_block_reconstruction_is_nearest_grid_point():
    """For unsaturated normal blocks, every element decodes to the grid point
    of {+-e2m1 * sf * gs} nearest to it (ties either way)."""
    rng = np.random.default_rng(9)
    for _ in range(200):
        x = (rng.standard_normal((1, 16)) * rng.uniform(0.01, 10)).astype(np.float32)
        gs = np.float32(rng.uniform(0.0005, 0.01))
        c, s = quant.quantize(x, gs)
        sf = formats.e4m3_decode(s)[0, 0]
        if not (2.0 ** -6 <= sf < 448):
            continue
        grid = np.concatenate([-formats.E2M1_MAGNITUDE, formats.E2M1_MAGNITUDE]) * sf * float(gs)
        d = quant.dequantize(c, s, gs)[0]
        for xi, di in zip(x[0].astype(np.float64), d):
            best = np.abs(grid - xi).min()
            assert abs(di - xi) <= best * (1 + 1e-6) + 1e-12


def _f32_div(a, b):
    """IEEE float32 a / b of float32 operands, via float64: the float64
    quotient rounded once to float32 is the correctly rounded float32
    quotient (53 >= 2 * 24 + 2 bits, so the double rounding is innocuous)."""
    return (np.asarray(a, np.float32).astype(np.float64) / np.asarray(b, np.float32).astype(np.float64)).astype(
        np.float32)


def _f32_mul(a, b):
    """IEEE float32 a * b of float32 operands: the float64 product is exact
    (48 significant bits), so one rounding to float32 is the float32 product."""
    return (np.asarray(a, np.float32).astype(np.float64) * np.asarray(b, np.float32).astype(np.float64)).astype(
        np.float32)


def _pre_rounding_cases():
    """Blocks of every kind: normal scales, subnormal scales, saturated
    scales (block amax far above what 448 * 6 * gs can encode), all-zero."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((16, 256)).astype(np.float32)
    x[0, :16] = 0.0                                   # all-zero block
    x[1, :] *= np.float32(3e-5)                       # subnormal block scales
    x[2, 16:32] *= np.float32(1e-9)                   # scale rounds to zero: flushed
    x[3, :] *= np.float32(400.0)                      # saturated scales (448)
    gs = quant.global_scale(np.float32(4.0))          # amax 4 -> most blocks normal
    return x, gs


def test_pre_rounding_values_follow_the_quantisation_steps():
    """pre_rounding_values re-derived with float64 arithmetic and one rounding
    per step (a different route to the same IEEE float32 results):
    s = bamax / (6 gs), r = 1 / (sf gs), v = x r, v = 0 in flushed blocks."""
    x, gs = _pre_rounding_cases()
    s, v = quant.pre_rounding_values(x, gs)
    xb = x.reshape(16, 16, 16)
    bamax = np.abs(xb).max(axis=2)
    d = _f32_mul(np.float32(6.0), gs)
    s_ref = _f32_div(bamax, d)
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32))
    sf = formats.e4m3_decode(formats.e4m3_encode_nonneg(s_ref)).astype(np.float32)
    with np.errstate(divide="ignore"):
        r = np.where(sf > 0, _f32_div(np.float32(1.0), _f32_mul(sf, gs)), np.float32(0.0)).astype(np.float32)
    v_ref = _f32_mul(xb, r[:, :, None]).reshape(16, 256)
    assert np.array_equal(np.abs(v), np.abs(v_ref))
    # the cases really are there: zero, subnormal, flushed, saturated, normal
    assert (s == 0).any() and (sf == 0).sum() >= 2
    assert ((sf > 0) & (sf < 2.0 ** -6)).any()
    assert (s > 448).any()
    assert ((sf >= 2.0 ** -6) & (sf < 448)).any()
    # in unsaturated normal blocks the largest element sits within one E4M3
    # rounding (at most 1/16 relative) of 6
    normal = (sf >= 2.0 ** -6) & (s <= 448)
    vmax = np.abs(v.reshape(16, 16, 16)).max(axis=2)
    assert (np.abs(vmax[normal] - 6.0) <= 6.0 / 15.0).all()


def test_quantize_is_the_encoding_of_pre_rounding_values():
    """quantize(x, gs) equals, bit for bit, the E4M3 encoding of the block
    values s and the sign plus E2M1 encoding of the element values v that
    pre_rounding_values reports, on normal, subnormal, saturated and zero
    blocks: the audit of rounding flips reads the numbers the encoders saw."""
    x, gs = _pre_rounding_cases()
    c, sc = quant.quantize(x, gs)
    s, v = quant.pre_rounding_values(x, gs)
    assert np.array_equal(sc, formats.e4m3_encode_nonneg(s))
    sf = np.repeat(formats.e4m3_decode(sc), 16, axis=1)
    codes = quant.unpack_codes(c)
    want = formats.e2m1_magnitude_index(np.abs(v)) | (np.signbit(x).astype(np.uint8) << 3)
    want = np.where(sf > 0, want, 0).astype(np.uint8)
    assert np.array_equal(codes, want)
    # saturated blocks: scale code 0x7E (448) and some element at code 6
    sat = s > 448
    assert (sc[sat] == 0x7E).all()
    assert ((codes.reshape(16, 16, 16)[sat] & 7) == 7).any(axis=-1).all()
