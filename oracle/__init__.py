"""CPU oracle for the NVFP4 mixture-of-experts expert pipeline.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.  It shares no code, table or constant generator with
the HIP library under ``block_scaled_fp4_03_amd/csrc``; the two meet only at the
seeded input generator, which holds none of the method's arithmetic.

What it computes is written from definitions, in numpy, slowly and plainly:

* ``formats``  - the E2M1 element format, the E4M3 scale format and bf16
  rounding, each from its bit-level definition.
* ``expf``     - the float32 exponential used by SiLU and the routing softmax
  (Cody-Waite reduction plus a Taylor polynomial), one IEEE operation at a time.
* ``quant``    - NVFP4 quantisation (16-element blocks, E4M3 block scale, FP32
  global scale in the dequantisation direction) and dequantisation.
* ``fp8``      - the FP8 weight-only projection of the attention output path
  (E4M3 weights with one float32 scale per 128 x 128 block, bf16 inputs).
* ``moe``      - top-k routing, the stable group-by-expert permutation, the
  grouped GEMM of two NVFP4 operands, SiLU(gate)*up with re-quantisation, the
  weighted combine, and the three compositions: the routed MoE layer, the
  shared expert (one group, no routing) and the MLA projections.

Sources.  The pipeline is the one planned on the page "Current Bug: vLLM
produces empty/garbage output" (revision e8b289e, section "Revised Plan: Our
Own NVFP4 Kernels", Phase 1): a first GEMM over the stacked gate and up
weights, SiLU, re-quantisation of the intermediate, a second GEMM over the
down weight; the shared expert is that same pipeline with a single group.  The epilogue factor alpha = input global scale x weight global scale
is on the revision a51edd2 of that page, section "What the quant method does".
The expert count and top-6 routing are on "CURRENT_BUG.md - DeepSeek-V4
Blackwell NVFP4", section "Architecture Notes".  The NVFP4 format itself
(E2M1 values two per byte, one E4M3 scale per 16 elements, one FP32 global
scale per tensor) is the public NVFP4 definition; the pages use but never
define it.

Parity status.  Every function here is pinned by ``tests/test_oracle_*.py``
against tables, library routines, closed forms, invariants or brute force.
The absolute end-to-end values at the full-size workloads have no printed
worked example on the pages: they are pinned only through the pinned parts
(parity unpinned in the sense that no external number states them).
"""
from . import formats, expf, quant, moe, fp8  # noqa: F401
