"""FP8 (E4M3) weight-only projection: block-scaled E4M3 weights times bf16
activations.  TEST INFRASTRUCTURE ONLY (see the package docstring).

The model's attention output path has `wo_a` as an FP8 weight-only einsum
with no input scale, followed by `wo_b`, an ordinary projection (page
"Current Bug: vLLM produces empty/garbage output", revision e8b289e, section
"Phase 2: CuTeDSL Attention Kernel"; "CURRENT_BUG.md - DeepSeek-V4 Blackwell
NVFP4", section "Architecture Notes").  The pages give neither the FP8 scale
granularity nor the einsum's index structure.  Readings taken here:

* weights are E4M3 (FN) codes with one float32 dequantisation scale per block
  of 128 x 128 weights: value(n, k) = e4m3(code[n, k]) * s[n // 128, k // 128];
* a block's scale is amax / 448 in float32 (1 for an all-zero block), and the
  code of a weight w is the sign bit of w plus the E4M3 magnitude nearest to
  |w / s| (float32 division; ties to even; saturating at 448);
* activations stay bf16 (weight-only: no input scale);
* wo_a is the dense projection of all heads' outputs, [T, 128 * 512] ->
  [T, o_lora_rank = 1024] (config table of e8b289e).
"""
import numpy as np

from . import formats

BLOCK = 128
E4M3_MAX = np.float32(448.0)


def _blocks(n):
    return -(-n // BLOCK)


def block_scales(w):
    """w [N, K] float32 -> s [ceil(N/128), ceil(K/128)] float32."""
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    s = np.empty((_blocks(N), _blocks(K)), np.float32)
    for i in range(s.shape[0]):
        for j in range(s.shape[1]):
            a = np.float32(np.abs(w[i * BLOCK:(i + 1) * BLOCK, j * BLOCK:(j + 1) * BLOCK]).max())
            s[i, j] = np.float32(a / E4M3_MAX) if a > 0 else np.float32(1.0)
    return s


def _expand(s, N, K):
    return np.repeat(np.repeat(s, BLOCK, axis=0), BLOCK, axis=1)[:N, :K]


def quantize_weight(w):
    """w [N, K] float32 -> (codes uint8 [N, K], scales float32 [NB, KB])."""
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    s = block_scales(w)
    q = (w / _expand(s, N, K)).astype(np.float32)          # one float32 division per weight
    mag = formats.e4m3_encode_nonneg(np.abs(q).astype(np.float64))
    sign = np.signbit(w).astype(np.uint8) << 7
    return (mag | sign).astype(np.uint8), s


def dequantize_weight(codes, scales):
    """Exact weight values (float64)."""
    N, K = codes.shape
    return formats.e4m3_decode(codes) * _expand(np.asarray(scales, np.float64), N, K)


def weight_gemm(x, codes, scales, out_dtype="f32"):
    """out[m, n] = sum_k x[m, k] * value(n, k) with x the bf16 activations (as
    float values) and value the dequantised weights: the products are exact
    in float64 (8 + 4 + 24 significant bits), the sum is float64, and the
    result is rounded once to float32 (or, for out_dtype "bf16", float32 then
    bf16)."""
    x = np.asarray(x, dtype=np.float64)
    out = (x @ dequantize_weight(codes, scales).T).astype(np.float32)
    if out_dtype == "bf16":
        out = formats.bf16_round(out)
    return out
