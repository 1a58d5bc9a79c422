"""Shared helpers of the GPU parity tests: seeded data, host copies and the
comparison rules (bit-exact for codes, scales, indices; the float32
summation bound and the cosine / max-abs gate for GEMM outputs)."""
import sys

import numpy as np
import torch

from oracle import formats, quant

F32 = np.float32


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_np(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.to(torch.float32).numpy()
    return t.numpy()


def bf16_tensor(x_np, device):
    """float32 array holding bf16 values -> bf16 tensor on device."""
    return torch.from_numpy(np.ascontiguousarray(x_np, dtype=np.float32)).to(torch.bfloat16).to(device)


def oracle_nvfp4(x_np, gs=None):
    x_np = np.asarray(x_np, dtype=np.float32)
    if gs is None:
        gs = quant.global_scale(quant.amax(x_np))
    c, s = quant.quantize(x_np, gs)
    return c, s, F32(gs)


def exact_gemm_rows(a_codes, a_scales, w_codes, w_scales):
    """float64 product of block-scaled values (exact up to float64 summation)
    and the matching sum of magnitudes used by the float32 error bound."""
    A = quant.dequantize_blocks(a_codes, a_scales)
    W = quant.dequantize_blocks(w_codes, w_scales)
    return A @ W.T, np.abs(A) @ np.abs(W).T


def check_gemm(got, exact, absum, alpha, K, out_bf16, what=""):
    """got: GPU output (float values); exact: float64 dot products before the
    global scales; absum: sum |a||w|; alpha: float64 per element (broadcast).

    float32 outputs: every element within the float32 summation bound
    gamma_K * sum|a w| of the exact value, max-abs error <= 2e-2 * RMS and
    cosine >= 0.999.
    bf16 outputs: every element equals the exact value rounded to bf16, or
    sits one bf16 ulp away where the exact value is within the float32 bound
    of the rounding midpoint (the two sides rounded slightly different float32
    sums); cosine >= 0.999; and the max-abs gate on the value before the
    output rounding: |got - exact| <= 2e-2 * RMS + one bf16 ulp of the
    element (the bf16 rounding of the output is part of its definition, and
    one ulp covers it and a midpoint flip)."""
    ref = exact * alpha
    gamma = K * 2.0 ** -24 / (1 - K * 2.0 ** -24)
    fbound = gamma * absum * np.abs(alpha) + 2 * np.abs(ref) * 2.0 ** -24 + 1e-37
    g64 = got.astype(np.float64)
    rms = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    if not out_bf16:
        err = np.abs(g64 - ref)
        bad = err > fbound
        assert not bad.any(), "%s: %d elements outside the float32 bound, worst %g vs %g" % (
            what, bad.sum(), err[bad].max(), fbound[bad][np.argmax(err[bad])])
        if ref.size and rms > 0:
            assert err.max() <= 2e-2 * rms, what
    else:
        ref_b = formats.bf16_round(ref.astype(np.float32)).astype(np.float64)
        diff = g64 != ref_b
        if diff.any():
            mid = (g64[diff] + ref_b[diff]) / 2
            ulp_ok = np.abs(g64[diff] - ref_b[diff]) <= np.spacing(
                np.abs(ref_b[diff]).astype(np.float32)).astype(np.float64) * 2 ** 16 * 1.0001
            near_mid = np.abs(ref[diff] - mid) <= fbound[diff]
            assert (ulp_ok & near_mid).all(), "%s: %d unexplained bf16 differences" % (
                what, (~(ulp_ok & near_mid)).sum())
        err = np.abs(g64 - ref)
        if ref.size and rms > 0:
            ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64) * 2 ** 16
            assert (err <= 2e-2 * rms + ulp).all(), "%s: max-abs gate" % what
            err = np.maximum(err - ulp, 0.0)
    if ref.size and rms > 0:
        cos = float((g64 * ref).sum() / np.sqrt((g64 ** 2).sum() * (ref ** 2).sum()))
        assert cos >= 0.999, (what, cos)
        return err.max() / rms
    return 0.0


def layer_gate(got, ref, what=""):
    """The gate on FP32-accumulated layer outputs: max-abs error <= 2e-2 *
    RMS(ref) and cosine >= 0.999, both always applied.  Returns (cosine,
    max-abs / RMS)."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(r ** 2))
    rel = float(np.abs(g - r).max() / rms) if rms > 0 else 0.0
    c = cosine(g, r) if rms > 0 else 1.0
    assert rel <= 2e-2, "%s: max-abs error %.3g x RMS" % (what, rel)
    assert c >= 0.999, "%s: cosine %.7f" % (what, c)
    return c, rel


def cosine(a, b):
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    return float((a * b).sum() / np.sqrt((a * a).sum() * (b * b).sum()))


def audit_code_flips(gpu_codes, gpu_scales, ora_codes, ora_scales, pre_s, pre_v, rel=1e-4):
    """Every code or block scale where the GPU and the oracle disagree must sit
    at a rounding boundary of the oracle's own pre-rounding value: the block
    scale s within `rel` of an E4M3 midpoint, or the element v within `rel` of
    an E2M1 midpoint (or in a block whose scale flipped).  Returns the number
    of flipped scales and codes."""
    e4 = formats.E4M3_POS_VALUES
    e4_mid = (e4[:-1] + e4[1:]) / 2
    e2_mid = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    s_diff = gpu_scales != ora_scales
    if s_diff.any():
        s = pre_s[s_diff].astype(np.float64)
        near = np.min(np.abs(s[:, None] - e4_mid[None, :]) / np.maximum(s[:, None], 1e-30), axis=1) <= rel
        assert near.all(), "unexplained block-scale flips: %d" % (~near).sum()
    gc = quant.unpack_codes(gpu_codes)
    oc = quant.unpack_codes(ora_codes)
    c_diff = gc != oc
    blk_flip = np.repeat(s_diff, 16, axis=1)
    c_check = c_diff & ~blk_flip
    if c_check.any():
        v = np.abs(pre_v[c_check].astype(np.float64))
        near = np.min(np.abs(v[:, None] - e2_mid[None, :]) / np.maximum(v[:, None], 1e-30), axis=1) <= rel
        assert near.all(), "unexplained code flips: %d" % (~near).sum()
    return int(s_diff.sum()), int(c_diff.sum())
