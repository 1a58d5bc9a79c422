"""Pins of SiLU(gate)*up and the weighted combine."""
import numpy as np

from oracle import formats, moe


def test_silu_special_values_and_float64_agreement():
    I = 4096
    rng = np.random.default_rng(0)
    g = np.concatenate([rng.standard_normal(I - 8) * 4, [0.0, -0.0, 20.0, 30.0, 89.0, -89.0, -200.0, 1e-30]])
    u = np.ones(I)
    gu = np.concatenate([g, u]).astype(np.float32)[None, :]
    h = moe.silu_mul(gu)[0].astype(np.float64)
    g32 = gu[0, :I].astype(np.float64)
    ref = g32 / (1.0 + np.exp(-g32))
    assert h[I - 8] == 0.0
    assert h[I - 6] == 20.0 and h[I - 5] == 30.0 and h[I - 4] == 89.0
    assert h[I - 2] == 0.0 and np.signbit(h[I - 2])        # exp overflows: -0.0
    # exp(-g) is +Inf by convention once -g > 88, so silu(g) is -0.0 there
    # where the true value is below 2e-36 in magnitude
    dom = g32 >= -88.0
    ok = np.abs(h - ref) <= 4 * np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64) + 1e-37
    assert ok[dom].all()
    assert (np.abs(ref[~dom]) < 2e-36).all() and (h[~dom] == 0).all()


def test_silu_mul_is_product_with_up():
    rng = np.random.default_rng(1)
    gu = rng.standard_normal((3, 64)).astype(np.float32)
    h = moe.silu_mul(gu)
    gu1 = gu.copy(); gu1[:, 32:] = 1.0
    s = moe.silu_mul(gu1)
    assert np.array_equal(h, (s * gu[:, 32:]).astype(np.float32))


def test_combine_identity_for_k1_w1():
    y = formats.bf16_round(np.random.default_rng(2).standard_normal((10, 24)).astype(np.float32))
    inv = np.random.default_rng(3).permutation(10).reshape(10, 1).astype(np.int32)
    w = np.ones((10, 1), dtype=np.float32)
    out = moe.combine(y, inv, w)
    assert np.array_equal(out, y[inv[:, 0]])


def test_combine_scaling_by_two_is_exact_and_sum_is_close_to_float64():
    rng = np.random.default_rng(4)
    T, k, H = 12, 6, 40
    y = formats.bf16_round(rng.standard_normal((T * k, H)).astype(np.float32))
    inv = rng.permutation(T * k).reshape(T, k).astype(np.int32)
    w = rng.uniform(0, 1, (T, k)).astype(np.float32)
    out = moe.combine(y, inv, w)
    out2 = moe.combine(y, inv, (w * 2).astype(np.float32))
    assert np.array_equal(out2, (out.astype(np.float64) * 2).astype(np.float32))
    ref = np.einsum("tj,tjh->th", w.astype(np.float64), y[inv].astype(np.float64))
    # before the bf16 rounding the float32 sum is within k ulps of float64
    assert np.allclose(out, ref, rtol=2.0 ** -8, atol=np.abs(ref).max() * 2.0 ** -8)


def test_combine_residual_is_one_more_float32_addition_before_rounding():
    """With a residual, out = bf16(fp32(acc + r)) where acc is the slot sum:
    re-derived here with float64 arithmetic rounded to float32 after every
    operation (the float32 result of a float32 op), then rounded to bf16."""
    rng = np.random.default_rng(5)
    T, k, H = 9, 6, 64
    y = formats.bf16_round(rng.standard_normal((T * k, H)).astype(np.float32))
    inv = rng.permutation(T * k).reshape(T, k).astype(np.int32)
    w = rng.uniform(0, 1, (T, k)).astype(np.float32)
    r = formats.bf16_round((rng.standard_normal((T, H)) * 3).astype(np.float32))
    out = moe.combine(y, inv, w, residual=r)
    acc = (w[:, :1].astype(np.float64) * y[inv[:, 0]]).astype(np.float32)
    for j in range(1, k):
        p = (w[:, j:j + 1].astype(np.float64) * y[inv[:, j]]).astype(np.float32)
        acc = (acc.astype(np.float64) + p).astype(np.float32)
    acc = (acc.astype(np.float64) + r).astype(np.float32)
    assert np.array_equal(out, formats.bf16_round(acc))
    # the residual is added before the single bf16 rounding, not after it
    late = formats.bf16_round((moe.combine(y, inv, w).astype(np.float64) + r).astype(np.float32))
    assert not np.array_equal(out, late)


def test_combine_residual_special_cases():
    rng = np.random.default_rng(6)
    T, k, H = 7, 2, 32
    y = formats.bf16_round(rng.standard_normal((T * k, H)).astype(np.float32))
    inv = rng.permutation(T * k).reshape(T, k).astype(np.int32)
    w = rng.uniform(0, 1, (T, k)).astype(np.float32)
    # a zero residual changes nothing
    assert np.array_equal(moe.combine(y, inv, w, residual=np.zeros((T, H), np.float32)), moe.combine(y, inv, w))
    # zero routing weights: the output is the residual itself (bf16 values)
    r = formats.bf16_round(rng.standard_normal((T, H)).astype(np.float32))
    assert np.array_equal(moe.combine(y, inv, np.zeros_like(w), residual=r), r)
    # a residual of minus the routed sum cancels exactly when that sum is a bf16 value
    s = moe.combine(y, inv, w)
    inv1 = np.arange(T, dtype=np.int32).reshape(T, 1)
    assert (moe.combine(s, inv1, np.ones((T, 1), np.float32), residual=-s) == 0).all()
