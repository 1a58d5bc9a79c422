"""Pins of the explained-flip audit the end-to-end tests apply to the
re-quantised intermediate: a GPU code or scale may differ from the oracle's
only where the oracle's own pre-rounding value sits at a rounding midpoint.
The audit must accept such flips and reject any other."""
import numpy as np
import pytest

from _helpers import audit_code_flips
from oracle import formats, quant

F32 = np.float32


def _block_at(v_target, gs=F32(1.0)):
    """One 16-element block whose element 0 is the block max (v = 6 with an
    exact scale of 1) and element 1 has pre-rounding value v_target."""
    x = np.zeros((1, 16), F32)
    x[0, 0] = F32(6.0)                      # bamax 6, s = 6 / 6 = 1: scale exactly 1
    x[0, 1] = F32(v_target)
    x[0, 2:] = F32(0.3)
    return x, F32(gs)


def _flip_code(codes, elem, new_mag):
    c = quant.unpack_codes(codes)
    c[0, elem] = (c[0, elem] & 8) | new_mag
    packed = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    return packed


def test_audit_accepts_code_flip_at_a_midpoint():
    # v = 2.5 (1 + 2^-20): nearest is 3 (index 5); a summation-order
    # difference can put the GPU's value just below 2.5, giving 2 (index 4)
    x, gs = _block_at(2.5 * (1 + 2.0 ** -20))
    c, s = quant.quantize(x, gs)
    pre_s, pre_v = quant.pre_rounding_values(x, gs)
    assert quant.unpack_codes(c)[0, 1] == 5
    flipped = _flip_code(c, 1, 4)
    n_s, n_c = audit_code_flips(flipped, s, c, s, pre_s, pre_v)
    assert (n_s, n_c) == (0, 1)


def test_audit_rejects_code_flip_away_from_midpoints():
    x, gs = _block_at(2.8)                  # nearest 3, far from the 2.5 / 3.5 midpoints
    c, s = quant.quantize(x, gs)
    pre_s, pre_v = quant.pre_rounding_values(x, gs)
    flipped = _flip_code(c, 1, 4)
    with pytest.raises(AssertionError, match="unexplained code flips"):
        audit_code_flips(flipped, s, c, s, pre_s, pre_v)


def test_audit_accepts_scale_flip_at_a_midpoint_and_the_codes_it_moves():
    # block amax chosen so that s sits on the midpoint of E4M3 values 1 and
    # 1.125 (to within 2^-20 relative): a neighbouring scale is explained, and
    # so are all codes of that block
    gs = F32(1.0)
    s_mid = 1.0625 * (1 + 2.0 ** -20)
    x = np.full((1, 16), F32(0.7), F32)
    x[0, 0] = F32(6.0 * s_mid)
    c, s = quant.quantize(x, gs)
    pre_s, pre_v = quant.pre_rounding_values(x, gs)
    other = np.array([[s[0, 0] - 1]], np.uint8)      # the other neighbour of the midpoint
    assert formats.e4m3_decode(other)[0, 0] in (1.0, 1.125)
    # under the other scale some codes move too: they are explained by the
    # block's scale flip
    orig = int(quant.unpack_codes(c)[0, 3] & 7)
    c_other = _flip_code(c, 3, (orig + 1) % 8)
    n_s, n_c = audit_code_flips(c_other, other, c, s, pre_s, pre_v)
    assert n_s == 1 and n_c >= 1


def test_audit_rejects_scale_flip_away_from_midpoints():
    gs = F32(1.0)
    x = np.full((1, 16), F32(0.7), F32)
    x[0, 0] = F32(6.0 * 1.03)                        # s = 1.03: nearest 1, far from 1.0625
    c, s = quant.quantize(x, gs)
    pre_s, pre_v = quant.pre_rounding_values(x, gs)
    with pytest.raises(AssertionError, match="unexplained block-scale flips"):
        audit_code_flips(c, s + 1, c, s, pre_s, pre_v)


def test_audit_rejects_flip_when_oracle_value_has_the_wrong_global_scale():
    # the audit is only as good as the pre-rounding values it reads: values
    # computed with a different global scale (a plausible mistake) no longer
    # explain the midpoint flip
    x, gs = _block_at(2.5 * (1 + 2.0 ** -20))
    c, s = quant.quantize(x, gs)
    flipped = _flip_code(c, 1, 4)
    bad_s, bad_v = quant.pre_rounding_values(x, F32(gs * F32(1.01)))
    with pytest.raises(AssertionError):
        audit_code_flips(flipped, s, c, s, bad_s, bad_v)
