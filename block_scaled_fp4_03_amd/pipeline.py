"""Compositions of the C-ABI ops into the three workloads of the path.

* routed MoE layer: quantise x -> route + permute -> L1 grouped GEMM over the
  stacked gate_up weights (gate and up with their own global scales) ->
  SiLU(gate)*up re-quantised -> L2 grouped GEMM over the down weights (bf16
  out) -> weighted combine (bf16);
* shared expert: the same with one group and no routing or combine, or
  folded into the routed layer as an always-on extra group;
* MLA projections: one-group GEMMs, the fused q_a+kv weight with two global
  scales, then q_b.
Every step is one call into libnvfp4moe.so; torch only provides the buffers
and the stream.  Weight preparation (drawing seeded weights and quantising
them with the library's own quantiser) lives here too.
"""
from dataclasses import dataclass

import torch

from . import ops, workloads


@dataclass
class NVFP4Weights:
    """A stack of G NVFP4 matrices [G, N, K] with per-(group, segment) scales.

    `tiled`, when set, is the same weights rearranged by prepare_weights; the
    GEMM then streams it instead of the row-major codes and scales (which may
    be dropped to save memory: `codes`/`scales` then keep only their shape)."""
    codes: torch.Tensor      # uint8 [G, N, K/2]
    scales: torch.Tensor     # uint8 [G, N, K/16]
    gs: torch.Tensor         # float32 [G, S]
    n_seg: tuple             # S+1 column boundaries
    tiled: torch.Tensor = None

    @property
    def nbytes(self):
        return self.codes.numel() + self.scales.numel()

    def prepare(self, drop_rows=False):
        """Build the tiled copy (K must be a multiple of 256)."""
        K = self.codes.shape[2] * 2
        if K % 256 == 0:
            self.tiled = ops.prepare_weights(self.codes, self.scales)
            if drop_rows:
                # keep only the shapes (tensors without storage)
                self.codes = torch.empty(self.codes.shape, dtype=torch.uint8, device="meta")
                self.scales = torch.empty(self.scales.shape, dtype=torch.uint8, device="meta")
        return self

    def groups(self, g0, g1):
        """Groups [g0, g1) as a view (no copy): the tiled layout stores the
        groups one after another, so a range of groups is one slice of it."""
        G, N, K2 = self.codes.shape
        if not 0 <= g0 < g1 <= G:
            raise ValueError("groups [%d, %d) outside [0, %d)" % (g0, g1, G))
        tiled = None
        if self.tiled is not None:
            per = ops.prepared_weight_bytes(1, N, 2 * K2)
            tiled = self.tiled[g0 * per:g1 * per]
        return NVFP4Weights(self.codes[g0:g1], self.scales[g0:g1], self.gs[g0:g1], self.n_seg, tiled)

    def reads_dq(self, M, a_rows):
        """Whether a GEMM of M rows (A stored in a_rows rows) reads A's f16 form."""
        G, _, K2 = self.codes.shape
        return ops.gemm_reads_dq(G, M, 2 * K2, a_rows, self.tiled is not None)

    def gemm(self, a_codes, a_scales, a_gs, group_offsets, M, **kw):
        return ops.grouped_gemm(a_codes, a_scales, a_gs, self.codes, self.scales, self.gs, self.n_seg,
                                group_offsets, M, w_tiled=self.tiled, **kw)

    def can_fuse_silu(self):
        """Whether this stacked gate_up stack runs the GEMM with the SiLU
        re-quantisation in its epilogue (tiled layout, I % 32 == 0)."""
        G, N, K2 = self.codes.shape
        return self.tiled is not None and len(self.n_seg) == 3 and N == 2 * self.n_seg[1] and \
            self.n_seg[1] % 32 == 0 and (2 * K2) % 256 == 0

    def fuse_by_default(self, M, a_rows):
        """Whether a first GEMM of M rows runs SiLU-requant in its epilogue by
        default: wherever the fused launch applies (it measures faster on the
        weight-streaming and the matrix-core kernels, and where K is split the
        reduction re-quantises directly; no float32 gate_up either way)."""
        return self.can_fuse_silu()

    def gemm_silu_requant(self, a_codes, a_scales, a_gs, group_offsets, M, gs_h, **kw):
        G, N, K2 = self.codes.shape
        return ops.grouped_gemm_silu_requant(a_codes, a_scales, a_gs, self.tiled, self.gs, group_offsets, M,
                                             N // 2, 2 * K2, gs_h, **kw)

    def can_fuse_silu_f32(self, M):
        """Whether a first GEMM of M rows can write SiLU(gate)*up in float32
        with its maxima (the dynamic-scale route): the fused epilogue without
        a split K."""
        G, N, K2 = self.codes.shape
        return self.can_fuse_silu() and ops.gemm_workspace_size(G, M, N, 2 * K2, True) == 0

    def gemm_silu_f32(self, a_codes, a_scales, a_gs, group_offsets, M, **kw):
        G, N, K2 = self.codes.shape
        return ops.grouped_gemm_silu_f32(a_codes, a_scales, a_gs, self.tiled, self.gs, group_offsets, M, N // 2,
                                         2 * K2, **kw)


def quantize_stack(mats, n_seg, device):
    """Quantise float32 matrices (each [N, K], one global scale per column
    segment, computed by the library from the segment's amax) into one stack."""
    G = len(mats)
    N, K = mats[0].shape
    S = len(n_seg) - 1
    codes = torch.empty(G, N, K // 2, dtype=torch.uint8, device=device)
    scales = torch.empty(G, N, K // 16, dtype=torch.uint8, device=device)
    gs = torch.empty(G, S, dtype=torch.float32, device=device)
    for g, m in enumerate(mats):
        m = m.to(device=device, dtype=torch.float32).contiguous()
        for s in range(S):
            r0, r1 = n_seg[s], n_seg[s + 1]
            ops.global_scale(m[r0:r1].reshape(1, -1), out=gs[g, s:s + 1])
            ops.quantize(m[r0:r1], gs[g, s:s + 1], codes=codes[g, r0:r1], scales=scales[g, r0:r1])
    return NVFP4Weights(codes, scales, gs, tuple(n_seg)).prepare()


def moe_weights(wl, device, seed=0, experts=None, tiled=True, drop_rows=False, n_shared=0):
    """(W1, W2) of a routed workload: W1 stacked gate_up [E, 2I, H] with
    segments (gate, up), W2 down [E, H, I].  Drawn expert by expert on
    `device` and quantised there; with `tiled`, also rearranged for the GEMM
    (and with `drop_rows` the row-major copies are released).  With
    n_shared, the stacks hold E + n_shared groups: the shared experts are
    groups E, E+1, ... (drawn as experts E, E+1, ... of the same seed)."""
    E = (wl.E if experts is None else experts) + n_shared
    I, H = wl.I, wl.H
    gen_dev = device if wl.weights_on_device else "cpu"
    w1 = NVFP4Weights(torch.empty(E, 2 * I, H // 2, dtype=torch.uint8, device=device),
                      torch.empty(E, 2 * I, H // 16, dtype=torch.uint8, device=device),
                      torch.empty(E, 2, dtype=torch.float32, device=device), (0, I, 2 * I))
    w2 = NVFP4Weights(torch.empty(E, H, I // 2, dtype=torch.uint8, device=device),
                      torch.empty(E, H, I // 16, dtype=torch.uint8, device=device),
                      torch.empty(E, 1, dtype=torch.float32, device=device), (0, H))
    for e in range(E):
        for W, f in ((w1, workloads.moe_gate_up), (w2, workloads.moe_down)):
            m = f(wl, e, seed, gen_dev).to(device)
            for s in range(len(W.n_seg) - 1):
                r0, r1 = W.n_seg[s], W.n_seg[s + 1]
                ops.global_scale(m[r0:r1].reshape(1, -1), out=W.gs[e, s:s + 1])
                ops.quantize(m[r0:r1], W.gs[e, s:s + 1], codes=W.codes[e, r0:r1], scales=W.scales[e, r0:r1])
            del m
    if tiled:
        w1.prepare(drop_rows)
        w2.prepare(drop_rows)
    return w1, w2


def can_persist(w1, w2):
    """Whether the expert MLP can run as one persistent launch (tiled
    weights, H and I multiples of 256)."""
    G, N, K2 = w1.codes.shape
    return w1.can_fuse_silu() and w2.tiled is not None and (2 * K2) % 256 == 0 and (N // 2) % 256 == 0


def _expert_mlp(xc, xs, gs_x, off, R, w1, w2, gs_h, a_rows, a_row_index=None, xdq=None, fused=None,
                persistent=False):
    """L1 -> SiLU-requant -> L2 over R (gathered) rows.  With `fused` and a
    static gs_h the re-quantisation runs in the L1 epilogue; with `fused` and
    gs_h None (a scale from this batch) the L1 epilogue writes h in float32
    and the maxima of |h|, from which gs_h comes, and h is then quantised.
    Both give the unfused route's results bit for bit without its float32
    gate_up; None picks w1.fuse_by_default (static) or w1.can_fuse_silu_f32
    (dynamic).  With `persistent`, both GEMMs and the fused
    SiLU-requant run as one persistent launch (nvfp4_moe_expert_mlp; static
    gs_h): h is identical, y identical in the streaming regime.  Returns (y
    bf16, stages)."""
    if persistent:
        if gs_h is None or not can_persist(w1, w2):
            raise ValueError("the persistent launch needs a static gs_h and tiled weights with H, I % 256 == 0")
        G, N, K2 = w1.codes.shape
        hc, hs, y = ops.moe_expert_mlp(xc, xs, gs_x, a_row_index, off, w1.tiled, w1.gs, w2.tiled, w2.gs, R, 2 * K2,
                                       N // 2, gs_h)
        return y, dict(hc=hc, hs=hs, y=y, gs_h=gs_h)
    if fused is None:
        fused = w1.fuse_by_default(R, a_rows) if gs_h is not None else w1.can_fuse_silu_f32(R)
    if fused and not (w1.can_fuse_silu() if gs_h is not None else w1.can_fuse_silu_f32(R)):
        raise ValueError("the fused epilogue needs tiled W1 with I % 32 == 0 (and, for a dynamic gs_h, no split K)")
    dq2 = True if w2.reads_dq(R, R) else None
    st = {}
    if fused and gs_h is not None:
        hc, hs, *hdq = w1.gemm_silu_requant(xc, xs, gs_x, off, R, gs_h, a_row_index=a_row_index, a_dq=xdq,
                                            dq=dq2)
    elif fused:
        # dynamic gs_h: h in float32 and the maxima of |h| from the first
        # GEMM's epilogue, gs_h from those maxima, then h quantised (the
        # values, scale and codes of the unfused route, without its float32
        # gate_up)
        h32, part = w1.gemm_silu_f32(xc, xs, gs_x, off, R, a_row_index=a_row_index, a_dq=xdq)
        gs_h = ops.global_scale(part.view(1, -1))
        hc, hs, *hdq = ops.quantize(h32, gs_h, dq=dq2)
        st["h_f32"] = h32
    else:
        gu = w1.gemm(xc, xs, gs_x, off, R, a_row_index=a_row_index, out_dtype=torch.float32, a_dq=xdq)
        if gs_h is None:
            gs_h = ops.silu_mul_global_scale(gu)
        hc, hs, *hdq = ops.silu_mul_requant(gu, gs_h, dq=dq2)
        st["gate_up"] = gu
    y = w2.gemm(hc, hs, gs_h, off, R, out_dtype=torch.bfloat16, a_dq=hdq[0] if hdq else None)
    st.update(hc=hc, hs=hs, y=y, gs_h=gs_h)
    return y, st


def moe_layer(x, logits, k, w1, w2, gs_x, gs_h, keep=False, fused=None, n_shared=0, residual=None,
              persistent=False):
    """Routed MoE layer.  x [T, H] bf16, logits [T, E] f32, gs_x/gs_h
    1-element f32 tensors: static activation global scales (from a warmup
    batch), or None for dynamic ones computed on the device from this batch
    (gs_x = amax(x)/2688 before quantising x, gs_h = amax(SiLU(g)*u)/2688
    between the two GEMMs; the host never waits for them).  `fused` runs
    SiLU-requant in the first GEMM's epilogue (nvfp4_grouped_gemm_silu_requant;
    with a dynamic gs_h, nvfp4_grouped_gemm_silu_f32 and then nvfp4_quantize),
    None chooses by the first GEMM's kernel (see _expert_mlp); the results
    are identical either way.  With n_shared, w1/w2 also hold that many
    shared experts as their last groups: every token visits them with weight
    1 (moe_route_permute_shared), so one grouped GEMM per projection covers
    the routed and the shared experts, and the combine adds the shared
    outputs after the routed slots.  residual (bf16 [T, H]) is added by the
    combine before its one rounding.  `persistent` runs the expert MLP as
    one persistent launch (see _expert_mlp).  Returns out [T, H] bf16 (and
    the stages)."""
    T, H = x.shape
    if w1.codes.shape[0] != logits.shape[1] + n_shared:
        raise ValueError("w1 holds %d groups; expected %d routed + %d shared" %
                         (w1.codes.shape[0], logits.shape[1], n_shared))
    R = T * (k + n_shared)
    if gs_x is None:
        gs_x = ops.global_scale(x.reshape(1, -1))
    # the many-row GEMM tiles read A in exactly dequantised f16 form, which the
    # producers write alongside the codes when it will be read
    xc, xs, *xdq = ops.quantize(x, gs_x, dq=True if w1.reads_dq(R, T) and not persistent else None)
    ids, w, off, sorted_ids, inv = ops.route_permute(logits, k, n_shared)
    y, st = _expert_mlp(xc, xs, gs_x, off, R, w1, w2, gs_h, T, a_row_index=sorted_ids,
                        xdq=xdq[0] if xdq else None, fused=fused, persistent=persistent)
    out = ops.combine(y, inv, w, residual=residual)
    if keep:
        st.update(xc=xc, xs=xs, ids=ids, w=w, offsets=off, sorted_ids=sorted_ids, inv=inv, gs_x=gs_x)
        return out, st
    return out


_OFFSETS = {}


def one_group_offsets(T, device):
    """Device tensor [0, T] (int32) for one-group GEMMs, made once per (T,
    device) so that repeated calls (and graph capture) copy nothing from the
    host."""
    key = (int(T), str(device))
    t = _OFFSETS.get(key)
    if t is None:
        t = torch.tensor([0, T], dtype=torch.int32, device=device)
        _OFFSETS[key] = t
    return t


def shared_expert(x, w1, w2, gs_x, gs_h, keep=False, fused=None):
    """Shared expert: one group, no routing.  Returns y [T, H] bf16."""
    T = x.shape[0]
    off = one_group_offsets(T, x.device)
    xc, xs, *xdq = ops.quantize(x, gs_x, dq=True if w1.reads_dq(T, T) else None)
    y, st = _expert_mlp(xc, xs, gs_x, off, T, w1, w2, gs_h, T, xdq=xdq[0] if xdq else None, fused=fused)
    if keep:
        st.update(xc=xc, xs=xs)
        return y, st
    return y


def mla_projections(x1, x2, w_qakv, w_qb, gs_x1, gs_x2):
    """MLA projections: x1 [T, 7168] through fused q_a+kv (two segments, two
    global scales), x2 [T, 1536] through q_b.  Both outputs bf16."""
    T = x1.shape[0]
    off = one_group_offsets(T, x1.device)
    c1, s1, *d1 = ops.quantize(x1, gs_x1, dq=True if w_qakv.reads_dq(T, T) else None)
    o1 = w_qakv.gemm(c1, s1, gs_x1, off, T, out_dtype=torch.bfloat16, a_dq=d1[0] if d1 else None)
    c2, s2, *d2 = ops.quantize(x2, gs_x2, dq=True if w_qb.reads_dq(T, T) else None)
    o2 = w_qb.gemm(c2, s2, gs_x2, off, T, out_dtype=torch.bfloat16, a_dq=d2[0] if d2 else None)
    return o1, o2


def attention_output(x, wo_a_codes, wo_a_scales, w_ob, gs_o):
    """Attention output path: x [T, 128*512] bf16 through wo_a (FP8
    weight-only, bf16 out), then wo_b (NVFP4: the bf16 intermediate quantised
    with the static global scale gs_o).  Returns (o [T, o_lora], y [T, H]),
    both bf16."""
    T = x.shape[0]
    off = one_group_offsets(T, x.device)
    o = ops.fp8_weight_gemm(x, wo_a_codes, wo_a_scales, out_dtype=torch.bfloat16)
    oc, os_, *od = ops.quantize(o, gs_o, dq=True if w_ob.reads_dq(T, T) else None)
    y = w_ob.gemm(oc, os_, gs_o, off, T, out_dtype=torch.bfloat16, a_dq=od[0] if od else None)
    return o, y
