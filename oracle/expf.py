"""float32 exponential for SiLU and the routing softmax.

Test infrastructure (see the package docstring); not part of the product path.

Both the oracle and the GPU library must make the same float32 decisions
(quantised codes downstream of SiLU, routing weights), so the exponential is
specified as a fixed sequence of IEEE float32 operations rather than "whatever
the platform's exp returns".  The method is the classical one (Cody & Waite,
"Software Manual for the Elementary Functions", 1980):

1. n = rint(x * log2(e)), ties to even;
2. r = (x - n*L_hi) - n*L_lo, with L_hi = 355/512 (nine significant bits, so
   n*L_hi is exact for |n| < 2**15) and L_lo = ln 2 - L_hi rounded to float32;
3. p = sum_{j=0..8} r**j / j!, evaluated by Horner's rule, coefficients 1/j!
   rounded to float32;
4. exp(x) = p * 2**n (exact scaling).

Each arithmetic step is a separate float32 operation (no fused multiply-add).
Domain conventions: x > 88 gives +Inf, x < -80 gives 0, so every finite
non-zero result is a normal float32 (no subnormal or flush-to-zero question
arises on either side).  Accuracy against float64 exp is pinned in the tests.
"""
import math

import numpy as np

F32 = np.float32
LOG2E = F32(1.0 / math.log(2.0))
LN2_HI = F32(355.0 / 512.0)
LN2_LO = F32(math.log(2.0) - 355.0 / 512.0)
TAYLOR = [F32(1.0 / math.factorial(j)) for j in range(9)]   # 1/0! .. 1/8!
X_OVERFLOW = F32(88.0)
X_UNDERFLOW = F32(-80.0)


def exp_spec(x):
    """Elementwise exp of a float32 array, one IEEE float32 op per step."""
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        n = np.rint(x * LOG2E).astype(np.float32)
        r = (x - n * LN2_HI).astype(np.float32)
        r = (r - n * LN2_LO).astype(np.float32)
        p = TAYLOR[8]
        for j in range(7, -1, -1):
            p = (p * r).astype(np.float32)
            p = (p + TAYLOR[j]).astype(np.float32)
        ni = np.clip(n, -200, 200).astype(np.int32)
        y = np.ldexp(p, ni).astype(np.float32)
    y = np.where(x > X_OVERFLOW, F32(np.inf), y)
    y = np.where(x < X_UNDERFLOW, F32(0.0), y)
    return y.astype(np.float32)
