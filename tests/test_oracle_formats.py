"""Pins of the oracle's number formats against published tables, torch's own
casts (independent library routines) and brute force."""
import os

import numpy as np
import pytest
import torch

from oracle import formats, expf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [l.split() for l in f if l.strip() and not l.startswith("#")]


def test_e2m1_table_matches_published_values():
    rows = _rows("e2m1_values.txt")
    codes = np.array([int(r[0]) for r in rows], dtype=np.uint8)
    vals = np.array([float(r[1]) for r in rows])
    got = formats.e2m1_decode(codes)
    assert np.array_equal(got, vals)
    assert np.array_equal(np.signbit(got), np.signbit(vals))   # 0x8 is -0.0


def _brute_e2m1_index(a):
    """Nearest magnitude by exhaustive distance, ties to the even index."""
    mags = formats.E2M1_MAGNITUDE
    d = np.abs(a[:, None] - mags[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among candidates prefer an even index
    even = cand & (np.arange(8)[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
    return pick.astype(np.uint8)


def test_e2m1_encode_brute_force_all_bf16():
    # all finite non-negative bf16 values up to 2**20 (beyond that float64
    # distances to the eight magnitudes can no longer be told apart, and the
    # answer is saturation, checked separately)
    bits = np.arange(0, 0x4980, dtype=np.uint32)
    a = (bits << 16).view(np.float32).astype(np.float64)
    assert a.max() < 2.0 ** 20
    assert np.array_equal(formats.e2m1_magnitude_index(a), _brute_e2m1_index(a))
    big = ((np.arange(0x4980, 0x7F80, dtype=np.uint32)) << 16).view(np.float32)
    assert (formats.e2m1_magnitude_index(big.astype(np.float64)) == 7).all()


def test_e2m1_encode_brute_force_around_midpoints():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    pts = []
    for m in mids:
        f = np.float32(m)
        for d in range(-3, 4):
            pts.append(np.nextafter(f, np.float32(np.inf if d > 0 else -np.inf)) if d else f)
            x = f
            for _ in range(abs(d)):
                x = np.nextafter(x, np.float32(np.inf if d > 0 else -np.inf))
            pts.append(x)
    a = np.array(pts, dtype=np.float32).astype(np.float64)
    assert np.array_equal(formats.e2m1_magnitude_index(a), _brute_e2m1_index(a))
    # ties go to the even code: 0.25->0, 0.75->1.0, 1.25->1.0, 1.75->2, 2.5->2, 3.5->4, 5->4
    idx = formats.e2m1_magnitude_index(np.array(mids))
    assert formats.E2M1_MAGNITUDE[idx].tolist() == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    assert formats.e2m1_magnitude_index(np.array([6.0, 7.0, 1e30])).tolist() == [7, 7, 7]


def test_e4m3_landmarks_match_published_values():
    for code, val in _rows("e4m3_landmarks.txt"):
        c = int(code, 16)
        assert formats.e4m3_decode(np.array([c], dtype=np.uint8))[0] == float(val)
        assert formats.e4m3_encode_nonneg(np.array([float(val)]))[0] == c
    assert np.isnan(formats.e4m3_decode(np.array([0x7F, 0xFF], dtype=np.uint8))).all()


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = formats.e4m3_decode(codes)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_e4m3_encode_matches_torch_cast_after_clamp():
    # torch's cast is round-to-nearest-even but not saturating (470 -> NaN),
    # so the reference clamps to 448 first.
    rng = np.random.default_rng(0)
    vals = formats.E4M3_POS_VALUES
    mids = (vals[:-1] + vals[1:]) / 2
    s = np.concatenate([
        vals, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
        rng.uniform(0, 500, 20000), np.exp2(rng.uniform(-14, 9, 20000)),
        [0.0, 1e-30, 447.9, 448.0, 463.9, 464.0, 465.0, 1e6],
    ]).astype(np.float32)
    got = formats.e4m3_encode_nonneg(s)
    ref = torch.from_numpy(np.minimum(s, 448.0)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(10000) * 1e-38).astype(np.float32),     # subnormal range
        (rng.standard_normal(10000) * 1e30).astype(np.float32),
        # exact ties: bf16 value + half an ulp
        ((rng.integers(0x3F80, 0x4780, 10000).astype(np.uint32) << 16) | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38], dtype=np.float32),
    ])
    got = formats.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_exp_spec_within_two_ulp_of_float64():
    x = np.concatenate([np.linspace(-80, 88, 400001),
                        np.random.default_rng(2).uniform(-2, 2, 200000)]).astype(np.float32)
    y = expf.exp_spec(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert (np.abs(y - ref) / ulp).max() <= 2.0


def test_exp_spec_special_values():
    x = np.array([0.0, -0.0, 88.5, 1000.0, -80.5, -1e30, 1.0], dtype=np.float32)
    y = expf.exp_spec(x)
    assert y[0] == 1.0 and y[1] == 1.0
    assert np.isinf(y[2]) and np.isinf(y[3])
    assert y[4] == 0.0 and y[5] == 0.0
    assert abs(float(y[6]) - np.e) <= np.spacing(np.float32(np.e))
