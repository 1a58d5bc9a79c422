"""NVFP4 quantisation and dequantisation, step by step.

Test infrastructure (see the package docstring); not part of the product path.

Format.  A row-major tensor of C columns (C a multiple of 16) is stored as
* codes  uint8 [rows, C/2]: E2M1 codes, element 2i in the low nibble of byte i,
  element 2i+1 in the high nibble;
* scales uint8 [rows, C/16]: one E4M3 code per 16 consecutive elements of a
  row, row-major, no swizzle;
* gs     float32: one global scale per tensor, in the dequantisation
  direction: element value = gs * scale(block) * e2m1(code).

The global scale.  gs = fp32(amax / 2688), 2688 = 6 * 448 being the largest
magnitude a block can encode before the global factor; amax = 0 gives 1.0.
The pages show what goes wrong when the two directions of this scale are
mixed up: on "Current Bug: vLLM produces empty/garbage output" (revision
a51edd2, section "What the quant method does") a stored scale of 0.00025141
used as an inverse becomes a multiplier of 3977.6 and the activations
overflow to NaN.  Here gs is always a multiplier on dequantisation, and
quantisation divides by it, saturating instead of overflowing.

Quantisation of one block x[0..15] (every step one IEEE float32 operation):
  bamax = max |x_i|                      (exact)
  d     = 6 * gs
  s     = bamax / d
  sq    = E4M3(s)                        (nearest-even, saturate to 448)
  sf    = value(sq)
  if sf == 0: all 16 codes are 0x0 (the block is flushed)
  else:       r = 1 / (sf * gs);  v_i = x_i * r;
              code_i = sign(x_i) << 3 | E2M1 magnitude index of |v_i|
The sign bit of a code is the sign bit of x_i (so -0.1 under a coarse
scale gives code 0x8, the negative zero).  A zero x_i has magnitude index 0
also where sf * gs is so small that r overflows to inf (a subnormal gs):
there the float32 product 0 * inf would be a NaN, and zero stays zero.
"""
import numpy as np

from .formats import e2m1_decode, e2m1_magnitude_index, e4m3_decode, e4m3_encode_nonneg

F32 = np.float32
BLOCK = 16
E2M1_MAX = 6.0
E4M3_MAX = 448.0


def global_scale(amax):
    """gs = fp32(amax / 2688) in the dequantisation direction; 0 -> 1.0."""
    amax = F32(amax)
    if amax == 0:
        return F32(1.0)
    return F32(amax / F32(E2M1_MAX * E4M3_MAX))


def amax(x):
    """Largest magnitude of a float array, as float32."""
    x = np.asarray(x, dtype=np.float32)
    return F32(np.max(np.abs(x))) if x.size else F32(0.0)


def quantize(x, gs, chunk_rows=4096):
    """x float32 [rows, C] -> (codes uint8 [rows, C/2], scales uint8 [rows, C/16])."""
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] % BLOCK:
        raise ValueError("quantize needs a 2-D array whose columns are a multiple of 16")
    if not np.all(np.isfinite(x)):
        raise ValueError("quantize needs finite input")
    rows, cols = x.shape
    codes = np.empty((rows, cols // 2), dtype=np.uint8)
    scales = np.empty((rows, cols // BLOCK), dtype=np.uint8)
    gs = F32(gs)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        c, s = _quantize_rows(x[r0:r1], gs)
        codes[r0:r1] = c
        scales[r0:r1] = s
    return codes, scales


def _quantize_rows(x, gs):
    rows, cols = x.shape
    xb = x.reshape(rows, cols // BLOCK, BLOCK)
    bamax = np.max(np.abs(xb), axis=2)                    # float32, exact
    d = F32(F32(E2M1_MAX) * gs)
    with np.errstate(over="ignore"):                       # saturates below
        s = (bamax / d).astype(F32)
    sq = e4m3_encode_nonneg(s)
    sf = e4m3_decode(sq).astype(F32)                      # exact in float32
    with np.errstate(divide="ignore", over="ignore"):
        denom = (sf * gs).astype(F32)
        r = (F32(1.0) / denom).astype(F32)
    r = np.where(sf == 0, F32(0.0), r).astype(F32)
    with np.errstate(invalid="ignore"):
        v = (xb * r[:, :, None]).astype(F32)
    # zero encodes as zero, also in a block whose 1/(sf*gs) overflowed to inf
    # (where the float32 product 0 * inf would be a NaN)
    v = np.where(xb == 0, F32(0.0), v).astype(F32)
    mag = e2m1_magnitude_index(np.abs(v))
    sign = np.signbit(xb).astype(np.uint8) << 3
    code = (mag | sign).astype(np.uint8)
    code = np.where((sf == 0)[:, :, None], np.uint8(0), code).astype(np.uint8)
    code = code.reshape(rows, cols)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, sq


def unpack_codes(codes):
    """uint8 [rows, C/2] -> uint8 [rows, C] of 4-bit codes (low nibble first)."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = codes & 0x0F
    out[:, 1::2] = codes >> 4
    return out


def dequantize_blocks(codes, scales):
    """Block-scaled values without the global factor: e2m1(code) * scale,
    float64 [rows, C].  The product is exact (at most 6 significant bits)."""
    vals = e2m1_decode(unpack_codes(codes))
    sf = e4m3_decode(scales)
    rows, cols = vals.shape
    return (vals.reshape(rows, cols // BLOCK, BLOCK) * sf[:, :, None]).reshape(rows, cols)


def dequantize(codes, scales, gs):
    """Element values gs * e2m1 * scale, float64 [rows, C]."""
    return dequantize_blocks(codes, scales) * np.float64(F32(gs))


def pre_rounding_values(x, gs):
    """The float32 numbers the encoders round, for audits of rounding flips:
    (s per block [rows, C/16], v per element [rows, C]); v is 0 in flushed
    blocks."""
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    xb = x.reshape(rows, cols // BLOCK, BLOCK)
    gs = F32(gs)
    bamax = np.max(np.abs(xb), axis=2)
    s = (bamax / F32(F32(E2M1_MAX) * gs)).astype(F32)
    sf = e4m3_decode(e4m3_encode_nonneg(s)).astype(F32)
    with np.errstate(divide="ignore"):
        r = (F32(1.0) / (sf * gs).astype(F32)).astype(F32)
    r = np.where(sf == 0, F32(0.0), r).astype(F32)
    with np.errstate(invalid="ignore"):
        v = (xb * r[:, :, None]).astype(F32)
    v = np.where(xb == 0, F32(0.0), v).astype(F32).reshape(rows, cols)
    return s, v
