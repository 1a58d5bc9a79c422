"""Pins of the oracle's grouped NVFP4 GEMM: exact integer arithmetic, a
library matmul within the float32 summation bound, the one-group identity,
group and segment structure."""
import numpy as np

from oracle import formats, quant, moe


def _nvfp4(rows, cols, seed, std=1.0):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, cols)) * std).astype(np.float32)
    gs = quant.global_scale(quant.amax(x))
    c, s = quant.quantize(x, gs)
    return c, s, gs


def _int_values(codes, scales):
    """Dequantised values as exact integers times 2**-10: e2m1 = V/2 with V an
    integer, E4M3 = S * 2**-9 with S an integer."""
    cd = quant.unpack_codes(codes).astype(np.int64)
    V = np.array([0, 1, 2, 3, 4, 6, 8, 12], dtype=np.int64)[cd & 7]
    V = np.where(cd & 8, -V, V)
    S = np.rint(formats.e4m3_decode(scales) * 512).astype(np.int64)
    rows, cols = V.shape
    return (V.reshape(rows, -1, 16) * S[:, :, None]).reshape(rows, cols)


def test_one_group_equals_exact_integer_gemm():
    M, N, K = 24, 40, 256
    a = _nvfp4(M, K, 1)
    w = _nvfp4(N, K, 2, std=0.02)
    out = moe.grouped_gemm(a[0], a[1], a[2], w[0][None], w[1][None], np.array([[w[2]]]),
                           [0, N], [0, M])
    ai = _int_values(a[0], a[1])
    wi = _int_values(w[0], w[1])
    exact = ai @ wi.T                                   # int64, exact (< 2**63)
    alpha = np.float32(a[2] * w[2])
    ref = (exact.astype(np.float64) * 2.0 ** -20 * float(alpha)).astype(np.float32)
    assert np.array_equal(out, ref)


def test_one_group_equals_library_matmul_within_fp32_bound():
    M, N, K = 33, 70, 1024
    a = _nvfp4(M, K, 3)
    w = _nvfp4(N, K, 4, std=0.02)
    out = moe.grouped_gemm(a[0], a[1], a[2], w[0][None], w[1][None], np.array([[w[2]]]),
                           [0, N], [0, M]).astype(np.float64)
    A = quant.dequantize(a[0], a[1], a[2]).astype(np.float32)
    W = quant.dequantize(w[0], w[1], w[2]).astype(np.float32)
    lib = (A @ W.T).astype(np.float64)                   # float32 BLAS
    gamma = K * 2.0 ** -24 / (1 - K * 2.0 ** -24)
    bound = gamma * (np.abs(A).astype(np.float64) @ np.abs(W).astype(np.float64).T) \
        + 2 * np.spacing(np.abs(lib).astype(np.float32)).astype(np.float64)
    assert (np.abs(out - lib) <= bound).all()


def test_grouped_rows_equal_per_row_single_group_and_empty_groups():
    G, N, K = 5, 48, 128
    counts = [3, 0, 7, 0, 2]
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(off[-1])
    a = _nvfp4(M + 4, K, 5)
    row_index = np.random.default_rng(6).permutation(M + 4)[:M].astype(np.int32)
    ws = [_nvfp4(N, K, 10 + g, std=0.02) for g in range(G)]
    wc = np.stack([w[0] for w in ws]); wsc = np.stack([w[1] for w in ws])
    wgs = np.array([[w[2], w[2] * np.float32(2)] for w in ws], dtype=np.float32)
    out = moe.grouped_gemm(a[0], a[1], a[2], wc, wsc, wgs, [0, 20, N], off, a_row_index=row_index)
    for g in range(G):
        for m in range(off[g], off[g + 1]):
            r = row_index[m]
            single = moe.grouped_gemm(a[0][r:r + 1], a[1][r:r + 1], a[2], wc[g:g + 1], wsc[g:g + 1],
                                      wgs[g:g + 1], [0, 20, N], [0, 1])
            assert np.array_equal(out[m], single[0])
    # segment 1 uses twice the weight scale: exactly twice segment-0 scaling
    g = 2
    one = moe.grouped_gemm(a[0], a[1], a[2], wc, wsc, np.repeat(wgs[:, :1], 2, 1), [0, 20, N], off,
                           a_row_index=row_index)
    rows = slice(off[g], off[g + 1])
    assert np.array_equal(out[rows, :20], one[rows, :20])
    assert np.array_equal(out[rows, 20:], (one[rows, 20:].astype(np.float64) * 2).astype(np.float32))


def test_group_order_does_not_change_rows():
    G, N, K = 3, 32, 64
    off = np.array([0, 2, 5, 9], dtype=np.int32)
    a = _nvfp4(9, K, 7)
    ws = [_nvfp4(N, K, 20 + g, std=0.02) for g in range(G)]
    wc = np.stack([w[0] for w in ws]); wsc = np.stack([w[1] for w in ws])
    wgs = np.array([[w[2]] for w in ws], dtype=np.float32)
    out = moe.grouped_gemm(a[0], a[1], a[2], wc, wsc, wgs, [0, N], off)
    perm = [2, 0, 1]
    counts = np.diff(off)[perm]
    off2 = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows2 = np.concatenate([np.arange(off[g], off[g + 1]) for g in perm])
    out2 = moe.grouped_gemm(a[0][rows2], a[1][rows2], a[2], wc[perm], wsc[perm], wgs[perm], [0, N], off2)
    assert np.array_equal(out2, out[rows2])


def test_bf16_output_is_rounded_f32_output():
    a = _nvfp4(8, 64, 8)
    w = _nvfp4(16, 64, 9, std=0.02)
    args = (a[0], a[1], a[2], w[0][None], w[1][None], np.array([[w[2]]]), [0, 16], [0, 8])
    f = moe.grouped_gemm(*args)
    b = moe.grouped_gemm(*args, out_dtype="bf16")
    assert np.array_equal(b, formats.bf16_round(f))


def test_f32_mode_within_summation_bound_of_exact_mode():
    """The float32 dequantise-then-matmul mode agrees with the exact mode to
    the float32 summation bound gamma_K * sum |a w| * alpha (plus the two
    roundings of the alpha product), and is not bitwise the same (it really
    sums in float32)."""
    G, N, K = 3, 96, 2048
    off = np.array([0, 5, 5, 17], dtype=np.int32)
    # block magnitudes spread over e^-9 .. 1, so that products of very
    # different sizes meet in the float32 sums and those sums round
    rng = np.random.default_rng(31)
    xa = (rng.standard_normal((17, K)) * np.exp(rng.uniform(-9, 0, (17, K // 16))).repeat(16, 1)).astype(np.float32)
    gsa = quant.global_scale(quant.amax(xa))
    a = quant.quantize(xa, gsa) + (gsa,)
    ws = [_nvfp4(N, K, 40 + g, std=0.02) for g in range(G)]
    wc = np.stack([w[0] for w in ws]); wsc = np.stack([w[1] for w in ws])
    wgs = np.array([[w[2], w[2] * np.float32(1.5)] for w in ws], dtype=np.float32)
    args = (a[0], a[1], a[2], wc, wsc, wgs, [0, 40, N], off)
    ex = moe.grouped_gemm(*args).astype(np.float64)
    f = moe.grouped_gemm(*args, mode="f32").astype(np.float64)
    A = quant.dequantize_blocks(a[0], a[1])
    gamma = K * 2.0 ** -24 / (1 - K * 2.0 ** -24)
    for g in range(G):
        r = slice(off[g], off[g + 1])
        if off[g + 1] == off[g]:
            continue
        W = quant.dequantize_blocks(wc[g], wsc[g])
        absum = np.abs(A[r]) @ np.abs(W).T
        alpha = np.concatenate([np.full(40, float(np.float32(a[2] * wgs[g, 0]))),
                                np.full(N - 40, float(np.float32(a[2] * wgs[g, 1])))])
        bound = gamma * absum * alpha + 3 * np.spacing(np.abs(ex[r]).astype(np.float32)).astype(np.float64)
        assert (np.abs(f[r] - ex[r]) <= bound).all()
    assert not np.array_equal(f, ex)


def test_f32_mode_equals_float32_library_matmul_bitwise():
    """The f32 mode is a float32 matmul of the dequantised operands followed
    by one float32 multiply by alpha: re-computed with torch's float32 CPU
    matmul (a second library) it agrees to the last bit only where both
    libraries sum in the same order, so compare within one float32 ulp of
    the sum magnitude per K-block instead."""
    import torch
    M, N, K = 12, 64, 1024
    a = _nvfp4(M, K, 51)
    w = _nvfp4(N, K, 52, std=0.02)
    f = moe.grouped_gemm(a[0], a[1], a[2], w[0][None], w[1][None], np.array([[w[2]]]), [0, N], [0, M], mode="f32")
    A = torch.from_numpy(quant.dequantize_blocks(a[0], a[1]).astype(np.float32))
    W = torch.from_numpy(quant.dequantize_blocks(w[0], w[1]).astype(np.float32))
    t = (A @ W.T).numpy() * np.float32(a[2] * w[2])
    absum = (np.abs(A.numpy()).astype(np.float64) @ np.abs(W.numpy()).astype(np.float64).T) * float(
        np.float32(a[2] * w[2]))
    gamma = K * 2.0 ** -24 / (1 - K * 2.0 ** -24)
    assert (np.abs(f.astype(np.float64) - t.astype(np.float64)) <= 2 * gamma * absum + 1e-30).all()


def test_layer_in_f32_mode_tracks_exact_mode():
    """The whole tiny layer with float32 GEMMs: routing, permutation and the
    layer input codes are the same; the output agrees with the exact-mode
    layer to cosine 1 - 1e-6 (differences come only from float32 sums and
    the re-quantisation flips they may cause)."""
    from oracle import formats
    rng = np.random.default_rng(60)
    T, H, I, E, k = 16, 256, 128, 8, 2
    x = formats.bf16_round(rng.standard_normal((T, H)).astype(np.float32))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    w1 = [_nvfp4(2 * I, H, 70 + e, std=0.02) for e in range(E)]
    w2 = [_nvfp4(H, I, 90 + e, std=0.02) for e in range(E)]
    W1 = (np.stack([w[0] for w in w1]), np.stack([w[1] for w in w1]),
          np.array([[w[2], w[2]] for w in w1], np.float32))
    W2 = (np.stack([w[0] for w in w2]), np.stack([w[1] for w in w2]), np.array([[w[2]] for w in w2], np.float32))
    gs_x = quant.global_scale(quant.amax(x))
    ex, st = moe.moe_layer(x, logits, k, W1, W2, gs_x, np.float32(0.002), return_stages=True)
    f, sf = moe.moe_layer(x, logits, k, W1, W2, gs_x, np.float32(0.002), return_stages=True, gemm_mode="f32")
    for key in ("ids", "offsets", "sorted_ids", "inv"):
        assert np.array_equal(st[key], sf[key])
    a, b = ex.astype(np.float64).ravel(), f.astype(np.float64).ravel()
    assert (a * b).sum() / np.sqrt((a * a).sum() * (b * b).sum()) >= 1 - 1e-6
