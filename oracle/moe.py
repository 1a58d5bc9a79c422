"""The MoE expert pipeline, one plain step at a time.

Test infrastructure (see the package docstring); not part of the product path.

Steps and their sources (pages named by title and revision):
* routing: top-k of the router logits, k = 6 of 384 experts in the full model
  ("CURRENT_BUG.md - DeepSeek-V4 Blackwell NVFP4", section "Architecture
  Notes"); the routed path has routing, top-k and a scatter, which the shared
  expert lacks ("Current Bug: vLLM produces empty/garbage output" @e8b289e,
  section "Phase 1: CuTeDSL Shared Expert Kernel").
* permutation: the tokens of each expert are gathered into one contiguous
  group of rows (the grouped GEMM runs over groups; same section).
* L1: grouped GEMM against the stacked gate_up weight, gate rows first, with
  a global scale of its own for gate and for up (the dual-global-scale pattern
  of section "Phase 2: CuTeDSL Attention Kernel", where the fused q_a+kv weight
  carries two weight global scales, the same pattern as gate and up in the MoE).
* SiLU(gate) * up, then re-quantisation of the intermediate to NVFP4 with one
  activation global scale.
* L2: grouped GEMM against the down weight.
* combine: the weighted sum of each token's k expert outputs back in token
  order, in bf16 at the end (the page keeps BF16 for the final scatter,
  section "Phase 3: Clean up").
* GEMM epilogue: output = alpha * sum_k A*W with alpha = activation global
  scale x weight global scale (@a51edd2, section "What the quant method
  does").

Readings where the pages are silent (each listed in the design notes):
* top-k selection compares the raw float32 logits; equal logits go to the
  lower expert id; weights are the softmax over the k selected logits,
  exp(l_j - l_0) / sum, sum taken in slot order, exp being ``expf.exp_spec``.
* permutation is expert-major and, inside an expert, by flat index t*k + j.
* the GEMM is computed exactly (float64 products of exactly-dequantised
  values, float64 sums whose error is far below float32 resolution), scaled
  by alpha in float64 and rounded once to float32, then to bf16 if asked.
* SiLU is g / (1 + exp(-g)) and the product with up stays float32; no bf16
  rounding happens before the re-quantisation.
* combine: acc = w_0*y_0, then acc = acc + w_j*y_j for j = 1..k-1, each a
  separate float32 operation, then one rounding to bf16.
* shared experts folded into the routed layer: a shared expert is an MoE of
  one expert without routing ("Current Bug: vLLM produces empty/garbage
  output" @e8b289e, section "Phase 1: CuTeDSL Shared Expert Kernel"); folded
  in, it is one more expert (id E, E+1, ...) that every token visits, in the
  slots after its k routed ones, with weight 1, so the combine adds its
  output after the routed ones.
"""
import numpy as np

from .expf import exp_spec
from .formats import bf16_round
from .quant import dequantize_blocks, quantize, global_scale, amax

F32 = np.float32


# --- routing and permutation -----------------------------------------------

def route_topk(logits, k):
    """logits float32 [T, E] -> (ids int32 [T, k], weights float32 [T, k]).

    Slot 0 holds the largest logit; equal logits are ordered by expert id."""
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        # stable sort of the negated logits keeps equal logits in id order
        order = np.argsort(-logits[t], kind="stable")
        ids[t] = order[:k]
    sel = np.take_along_axis(logits, ids, axis=1)
    diff = (sel - sel[:, :1]).astype(F32)          # l_j - l_0 <= 0
    e = exp_spec(diff)
    total = e[:, 0].copy()
    for j in range(1, k):
        total = (total + e[:, j]).astype(F32)
    w = (e / total[:, None]).astype(F32)
    return ids, w


def append_shared(ids, w, E, n_shared):
    """Routed (ids, w) [T, k] -> [T, k + n_shared]: slot k + s holds the
    always-on shared expert E + s with weight 1."""
    T = ids.shape[0]
    sid = np.broadcast_to(np.arange(E, E + n_shared, dtype=np.int32), (T, n_shared))
    return (np.concatenate([ids, sid], axis=1).astype(np.int32),
            np.concatenate([w, np.ones((T, n_shared), dtype=F32)], axis=1).astype(F32))


def permute(ids, E):
    """ids int32 [T, k] -> (offsets int32 [E+1], sorted_token_ids int32 [T*k],
    inv int32 [T, k]) with rows grouped by expert, ascending flat index within
    an expert; sorted_token_ids[p] is the token of row p, inv[t, j] the row
    that holds (t, j)."""
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(flat, kind="stable")        # flat indices, expert-major
    sorted_token_ids = (order // k).astype(np.int32)
    inv = np.empty(T * k, dtype=np.int32)
    inv[order] = np.arange(T * k, dtype=np.int32)
    return offsets.astype(np.int32), sorted_token_ids, inv.reshape(T, k)


# --- grouped GEMM -----------------------------------------------------------

def grouped_gemm(a_codes, a_scales, a_gs, w_codes, w_scales, w_gs, n_seg,
                 group_offsets, a_row_index=None, out_dtype="f32", mode="exact"):
    """out[m, n] = alpha(g, seg(n)) * sum_k A[m, k] * W[g, n, k] for rows m of
    group g, A and W dequantised without their global scales,
    alpha = fp32(a_gs * w_gs[g, seg]).

    mode "exact" (the reference): float64 products of the exactly
    dequantised values (exact: each is an integer multiple of 2**-20 below
    2**43 of those units) and float64 sums, which stay exact while partial
    sums are below 2**53 units and otherwise err by less than
    K * 2**-53 * sum |a w|, far below float32 resolution; alpha applied in
    float64, one rounding to float32.
    mode "f32": dequantise to float32 (exact: at most five significant bits)
    and multiply with a float32 library matmul, then alpha in float32 (two
    roundings): the plain dequantise-then-matmul reference, accurate to the
    float32 summation bound gamma_K * sum |a w| of the exact result.

    a_codes/a_scales: NVFP4 [Ma, K]; a_row_index (optional) [M]: logical row m
    reads stored row a_row_index[m]; w_codes/w_scales: [G, N, K/2], [G, N, K/16];
    w_gs float32 [G, S]; n_seg: S+1 column boundaries, n_seg[0] = 0,
    n_seg[S] = N; group_offsets [G+1], non-decreasing, last = M.
    Returns float32 [M, N] (bf16 values stored in float32 if out_dtype="bf16").
    """
    w_codes = np.asarray(w_codes)
    G, N, K2 = w_codes.shape
    K = K2 * 2
    off = np.asarray(group_offsets, dtype=np.int64)
    M = int(off[-1])
    w_gs = np.asarray(w_gs, dtype=F32).reshape(G, -1)
    n_seg = list(n_seg)
    if n_seg[0] != 0 or n_seg[-1] != N or len(n_seg) != w_gs.shape[1] + 1:
        raise ValueError("bad n_seg")
    if mode not in ("exact", "f32"):
        raise ValueError("mode must be 'exact' or 'f32'")
    A = dequantize_blocks(a_codes, a_scales)
    if a_row_index is not None:
        A = A[np.asarray(a_row_index, dtype=np.int64)]
    if A.shape != (M, K):
        raise ValueError("A has shape %s, expected %s" % (A.shape, (M, K)))
    if mode == "f32":
        A = A.astype(F32)                                       # exact
    out = np.zeros((M, N), dtype=F32)
    for g in range(G):
        r0, r1 = int(off[g]), int(off[g + 1])
        if r1 == r0:
            continue
        W = dequantize_blocks(w_codes[g], w_scales[g])          # [N, K] float64
        if mode == "f32":
            acc = A[r0:r1] @ W.astype(F32).T                    # float32 matmul
        else:
            acc = A[r0:r1] @ W.T                                # float64
        for s in range(len(n_seg) - 1):
            c0, c1 = n_seg[s], n_seg[s + 1]
            alpha = F32(F32(a_gs) * w_gs[g, s])
            if mode == "f32":
                out[r0:r1, c0:c1] = (acc[:, c0:c1] * alpha).astype(F32)
            else:
                out[r0:r1, c0:c1] = (acc[:, c0:c1] * np.float64(alpha)).astype(F32)
    if out_dtype == "bf16":
        out = bf16_round(out)
    elif out_dtype != "f32":
        raise ValueError("out_dtype must be 'f32' or 'bf16'")
    return out


# --- SiLU(gate) * up and re-quantisation -----------------------------------

def silu_mul(gate_up):
    """gate_up float32 [M, 2I] (gate columns first) -> h float32 [M, I]."""
    gu = np.asarray(gate_up, dtype=F32)
    I = gu.shape[1] // 2
    g = gu[:, :I]
    u = gu[:, I:]
    e = exp_spec(-g)
    with np.errstate(over="ignore"):
        den = (F32(1.0) + e).astype(F32)
    silu = (g / den).astype(F32)
    return (silu * u).astype(F32)


def silu_mul_requant(gate_up, gs_h):
    """gate_up float32 [M, 2I] -> NVFP4 (codes [M, I/2], scales [M, I/16])."""
    return quantize(silu_mul(gate_up), gs_h)


# --- combine -----------------------------------------------------------------

def combine(y, inv, w, residual=None):
    """y float32 [T*k, H] (bf16 values), inv int32 [T, k], w float32 [T, k]
    -> out float32 [T, H] holding bf16 values.

    With residual (float32 [T, H] holding bf16 values), it is added after
    the last slot, as one more float32 addition before the single rounding
    to bf16: out = bf16(((w_0 y_0 + w_1 y_1) + ...) + residual)."""
    y = np.asarray(y, dtype=F32)
    inv = np.asarray(inv, dtype=np.int64)
    w = np.asarray(w, dtype=F32)
    T, k = inv.shape
    acc = (w[:, 0:1] * y[inv[:, 0]]).astype(F32)
    for j in range(1, k):
        acc = (acc + (w[:, j:j + 1] * y[inv[:, j]]).astype(F32)).astype(F32)
    if residual is not None:
        residual = np.asarray(residual, dtype=F32)
        if residual.shape != acc.shape:
            raise ValueError("residual must be [T, H]")
        acc = (acc + residual).astype(F32)
    return bf16_round(acc)


# --- compositions --------------------------------------------------------------

def moe_layer(x, logits, k, w1, w2, gs_x, gs_h, return_stages=False, n_shared=0, gemm_mode="exact",
              residual=None):
    """The routed MoE layer.

    x float32 [T, H] (bf16 values); logits float32 [T, E];
    w1 = (codes [E, 2I, H/2], scales [E, 2I, H/16], gs [E, 2]) gate rows first;
    w2 = (codes [E, H, I/2], scales [E, H, I/16], gs [E, 1]).
    With n_shared, w1 and w2 hold E + n_shared experts, the last n_shared
    being shared experts folded in (see append_shared).  gemm_mode selects
    the GEMM arithmetic (see grouped_gemm); residual (optional [T, H] bf16
    values) is added by the combine.
    Returns out float32 [T, H] holding bf16 values (and the stages if asked).
    """
    T, H = x.shape
    E = logits.shape[1]
    I2 = w1[0].shape[1]
    I = I2 // 2
    if w1[0].shape[0] != E + n_shared or w2[0].shape[0] != E + n_shared:
        raise ValueError("weights must hold E + n_shared experts")
    xq = quantize(x, gs_x)
    ids, wts = route_topk(logits, k)
    if n_shared:
        ids, wts = append_shared(ids, wts, E, n_shared)
    offsets, sorted_ids, inv = permute(ids, E + n_shared)
    gu = grouped_gemm(xq[0], xq[1], gs_x, w1[0], w1[1], w1[2], [0, I, I2],
                      offsets, a_row_index=sorted_ids, out_dtype="f32", mode=gemm_mode)
    h = silu_mul(gu)
    hq = quantize(h, gs_h)
    y = grouped_gemm(hq[0], hq[1], gs_h, w2[0], w2[1], w2[2], [0, H],
                     offsets, out_dtype="bf16", mode=gemm_mode)
    out = combine(y, inv, wts, residual)
    if return_stages:
        return out, dict(xq=xq, ids=ids, w=wts, offsets=offsets,
                         sorted_ids=sorted_ids, inv=inv, gate_up=gu, h=h, hq=hq, y=y)
    return out


def shared_expert(x, w1, w2, gs_x, gs_h, return_stages=False):
    """The shared expert: the same pipeline with one group and no routing.
    w1 = (codes [1, 2I, H/2], scales, gs [1, 2]); w2 = (codes [1, H, I/2],
    scales, gs [1, 1]).  Returns y float32 [T, H] holding bf16 values."""
    T, H = x.shape
    I2 = w1[0].shape[1]
    I = I2 // 2
    off = [0, T]
    xq = quantize(x, gs_x)
    gu = grouped_gemm(xq[0], xq[1], gs_x, w1[0], w1[1], w1[2], [0, I, I2], off)
    h = silu_mul(gu)
    hq = quantize(h, gs_h)
    y = grouped_gemm(hq[0], hq[1], gs_h, w2[0], w2[1], w2[2], [0, H], off, out_dtype="bf16")
    if return_stages:
        return y, dict(xq=xq, gate_up=gu, h=h, hq=hq)
    return y


def mla_projections(x1, x2, w_qakv, w_qb, gs_x1, gs_x2, n_qa):
    """The MLA projections as one-group NVFP4 GEMMs.

    x1 float32 [T, 7168] -> [T, n_qa + n_kv] through the fused q_a+kv weight
    whose two row segments carry their own global scales (w_qakv gs [1, 2]);
    x2 float32 [T, 1536] -> [T, N_qb] through q_b (gs [1, 1]).  Both outputs
    bf16 values in float32."""
    T = x1.shape[0]
    off = [0, T]
    N1 = w_qakv[0].shape[1]
    N2 = w_qb[0].shape[1]
    x1q = quantize(x1, gs_x1)
    x2q = quantize(x2, gs_x2)
    o1 = grouped_gemm(x1q[0], x1q[1], gs_x1, w_qakv[0], w_qakv[1], w_qakv[2],
                      [0, n_qa, N1], off, out_dtype="bf16")
    o2 = grouped_gemm(x2q[0], x2q[1], gs_x2, w_qb[0], w_qb[1], w_qb[2],
                      [0, N2], off, out_dtype="bf16")
    return o1, o2


def quantize_weight(w):
    """float32 [N, K] weight -> (codes, scales, gs) with gs from its own amax."""
    gs = global_scale(amax(w))
    c, s = quantize(w, gs)
    return c, s, gs
