"""Pins of the FP8 weight-only projection oracle (oracle/fp8.py) against
a library cast, closed forms, invariants and exact integer arithmetic."""
import numpy as np
import torch

from oracle import formats, fp8

F32 = np.float32


def _w(N, K, seed, scale=0.02):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((N, K)) * scale).astype(np.float32)
    w[3, 5] = 0.0
    w[4, 7] = -0.0
    return w


def test_codes_match_torch_e4m3_cast_of_the_scaled_weights():
    # torch's float8_e4m3fn cast is round-to-nearest-even but not saturating,
    # hence the clamp to +-448 first
    w = _w(200, 300, 1)
    w[0, :128] *= 1000.0                  # one block with a different range
    codes, s = fp8.quantize_weight(w)
    q = torch.from_numpy(w) / torch.from_numpy(np.repeat(np.repeat(s, 128, 0), 128, 1)[:200, :300])
    ref = q.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


def test_block_scales_and_saturation_invariants():
    w = _w(256, 384, 2)
    w[128:, 128:256] = 0.0                 # an all-zero block
    codes, s = fp8.quantize_weight(w)
    assert s.shape == (2, 3) and s[1, 1] == 1.0
    for i in range(2):
        for j in range(3):
            blk = codes[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            if (i, j) == (1, 1):
                assert np.all((blk & 0x7F) == 0)
                continue
            # amax / (amax / 448) rounds to 448: every block holds a +-448 code
            assert np.any((blk & 0x7F) == 0x7E)
            assert s[i, j] == F32(F32(np.abs(w[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]).max()) / F32(448))
    # no NaN codes, sign bits follow the weights (including -0)
    assert not np.any((codes & 0x7F) == 0x7F)
    assert codes[4, 7] == 0x80 and codes[3, 5] == 0x00


def test_dequantised_error_within_half_an_e4m3_step():
    w = _w(130, 260, 3)
    codes, s = fp8.quantize_weight(w)
    v = fp8.dequantize_weight(codes, s)
    full = np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)[:130, :260]
    q = np.abs(w.astype(np.float64) / full)
    # spacing of the E4M3 grid around q: 2^(e-3) for normal q, 2^-9 below 2^-6
    e = np.floor(np.log2(np.maximum(q, 2.0 ** -6)))
    step = np.exp2(e - 3)
    assert np.all(np.abs(np.abs(v) / full - q) <= step / 2 * (1 + 1e-6) + 1e-300)


def test_gemm_exact_on_small_integers():
    # integer activations and weights whose blocks have power-of-two scales:
    # every product and sum is an exact small number
    rng = np.random.default_rng(4)
    M, N, K = 9, 140, 256
    x = rng.integers(-8, 9, (M, K)).astype(np.float64)
    mag = rng.integers(0, 8, (N, K))                    # 0..7 are exact E4M3 values
    codes = formats.e4m3_encode_nonneg(mag.astype(np.float64)) | (rng.integers(0, 2, (N, K)) << 7).astype(np.uint8)
    s = np.array([[1.0, 0.5], [4.0, 2.0]], np.float32)
    vals = formats.e4m3_decode(codes)
    full = np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)[:N, :K]
    expect = x @ (vals * full).T
    got = fp8.weight_gemm(x, codes, s)
    assert np.array_equal(got, expect.astype(np.float32))


def test_gemm_blocks_scale_linearly_and_match_a_library_matmul():
    rng = np.random.default_rng(5)
    M, N, K = 7, 130, 384
    x = formats.bf16_round(rng.standard_normal((M, K)).astype(np.float32))
    codes, s = fp8.quantize_weight(_w(N, K, 6))
    base = fp8.weight_gemm(x, codes, s).astype(np.float64)
    # the result is the sum over k-blocks of (block scale) x (block dot
    # product of bf16 x and E4M3 values), rounded once: scaling the scales of
    # k-block j by 2^j scales that block's term by 2^j
    s2 = s.copy()
    s2[:, 1] *= 2.0
    s2[:, 2] *= 4.0
    x64 = x.astype(np.float64)
    vals = formats.e4m3_decode(codes)
    srow = np.repeat(s.astype(np.float64), 128, axis=0)[:N]          # [N, KB]
    parts = [(x64[:, j * 128:(j + 1) * 128] @ vals[:, j * 128:(j + 1) * 128].T) * srow[:, j][None, :]
             for j in range(3)]
    got = fp8.weight_gemm(x, codes, s2).astype(np.float64)
    for res, exact in ((got, parts[0] + 2 * parts[1] + 4 * parts[2]), (base, sum(parts))):
        assert np.all(np.abs(res - exact) <= 2.0 ** -24 * np.abs(exact) + 1e-300)
    # a float32 library matmul of the dequantised weights lies within the
    # float32 summation bound of the float64 result
    w32 = fp8.dequantize_weight(codes, s).astype(np.float32)
    lib = torch.from_numpy(x.astype(np.float32)) @ torch.from_numpy(w32).T
    bound = K * 2.0 ** -24 * (np.abs(x).astype(np.float64) @ np.abs(w32.astype(np.float64)).T)
    assert np.all(np.abs(lib.numpy().astype(np.float64) - base) <= bound + 1e-30)
