"""End-to-end parity of the HIP pipeline against the oracle on the five
workloads (tiny, shared expert, MLA projections, decode and prefill layers).

Both sides start from the same seeded float32 draws; each quantises them with
its own quantiser (checked bit-exact), then runs its own pipeline.  Gates:
* bit-exact: quantised x and weights, routing ids and weights, offsets,
  sorted token ids and the inverse permutation;
* L1 output: the float32 summation bound of the exact contraction (both sides
  have the same operands);
* re-quantised intermediate: identical except at rounding boundaries of the
  oracle's own pre-rounding values (audited);
* L2 output and the combined layer output: cosine >= 0.999 against the
  oracle, max-abs error reported (a boundary flip of one intermediate code
  legitimately moves one output by a few per cent of its RMS).
Full-size workloads are checked on sampled experts, rows and one token; the
sizes the oracle cannot do in seconds are noted per test.
"""
import numpy as np
import pytest
import torch

from _helpers import (F32, audit_code_flips, bf16_tensor, check_gemm, cosine, dev, exact_gemm_rows, log,
                      to_np)
from block_scaled_fp4_03_amd import ops, pipeline, workloads
from oracle import fp8, moe, quant

pytestmark = pytest.mark.gpu


def _oracle_moe_expert(wl, e, gen_device):
    """Oracle-quantised (W1 codes, scales, gs[2]), (W2 codes, scales, gs[1])
    of expert e from the seeded float32 draws."""
    I = wl.I
    m1 = workloads.moe_gate_up(wl, e, 0, gen_device).cpu().numpy()
    m2 = workloads.moe_down(wl, e, 0, gen_device).cpu().numpy()
    gg, gu = quant.global_scale(quant.amax(m1[:I])), quant.global_scale(quant.amax(m1[I:]))
    a, sa = quant.quantize(m1[:I], gg)
    b, sb = quant.quantize(m1[I:], gu)
    c2, s2, g2 = moe.quantize_weight(m2)
    return ((np.concatenate([a, b]), np.concatenate([sa, sb]), np.array([gg, gu], np.float32)),
            (c2, s2, np.array([g2], np.float32)))


def _check_weights(w_gpu, e, ow):
    assert np.array_equal(to_np(w_gpu.codes[e]), ow[0]), "codes of expert %d" % e
    assert np.array_equal(to_np(w_gpu.scales[e]), ow[1]), "scales of expert %d" % e
    assert np.array_equal(to_np(w_gpu.gs[e]), ow[2]), "global scales of expert %d" % e


def _l1_alpha(gs_x, g1, I):
    return np.concatenate([np.full(I, float(F32(gs_x * g1[0]))), np.full(I, float(F32(gs_x * g1[1])))])


def _expert_rows_check(wl, e, rows, tokens, xq, gs_x, gs_h, o1, o2, g_gu, g_hc, g_hs, g_y):
    """Per-stage checks on the rows of expert e (rows: permuted row ids,
    tokens: their token ids) with oracle weights o1/o2.  Returns the number of
    audited intermediate flips."""
    I, H = wl.I, wl.H
    ex, ab = exact_gemm_rows(xq[0][tokens], xq[1][tokens], o1[0], o1[1])
    check_gemm(g_gu[rows], ex, ab, _l1_alpha(gs_x, o1[2], I)[None, :], H, False, "L1 expert %d" % e)
    # oracle's own L1 output (rounded to float32) -> h -> NVFP4
    gu = (ex * _l1_alpha(gs_x, o1[2], I)[None, :]).astype(np.float32)
    h = moe.silu_mul(gu)
    hc, hs = quant.quantize(h, gs_h)
    pre_s, pre_v = quant.pre_rounding_values(h, gs_h)
    n_s, n_c = audit_code_flips(g_hc[rows], g_hs[rows], hc, hs, pre_s, pre_v)
    # L2 from the oracle's intermediate
    ex2, ab2 = exact_gemm_rows(hc, hs, o2[0], o2[1])
    alpha2 = float(F32(gs_h * o2[2][0]))
    same = np.all(g_hc[rows] == hc, axis=1) & np.all(g_hs[rows] == hs, axis=1)
    if same.any():
        check_gemm(g_y[rows][same], ex2[same], ab2[same], alpha2, I, True, "L2 expert %d" % e)
    if (~same).any():
        assert cosine(g_y[rows][~same], ex2[~same] * alpha2) >= 0.999
    return n_s + n_c


# --- tiny: the whole layer, every stage -------------------------------------------

def _fused_same(unfused, fused):
    """The layer with SiLU-requant in the first GEMM's epilogue must give the
    unfused layer's intermediate and output bit for bit."""
    (o0, g0), (o1, g1) = unfused, fused
    assert "gate_up" not in g1 and "gate_up" in g0    # the two paths really differ
    assert g1["hc"].data_ptr() != g0["hc"].data_ptr()
    for k_ in ("hc", "hs"):
        assert np.array_equal(to_np(g0[k_]), to_np(g1[k_])), k_
    assert np.array_equal(to_np(o0).view(np.uint32) if o0.dtype == torch.float32 else
                          o0.view(torch.int16).cpu().numpy(),
                          to_np(o1).view(np.uint32) if o1.dtype == torch.float32 else
                          o1.view(torch.int16).cpu().numpy())


def _tiny_setup(n_shared=0):
    wl = workloads.WORKLOADS["tiny"]
    d = dev()
    w1, w2 = pipeline.moe_weights(wl, d, n_shared=n_shared)
    ow = [_oracle_moe_expert(wl, e, "cpu") for e in range(wl.E + n_shared)]
    for e in range(wl.E + n_shared):
        _check_weights(w1, e, ow[e][0])
        _check_weights(w2, e, ow[e][1])
    W1 = (np.stack([o[0][0] for o in ow]), np.stack([o[0][1] for o in ow]), np.stack([o[0][2] for o in ow]))
    W2 = (np.stack([o[1][0] for o in ow]), np.stack([o[1][1] for o in ow]), np.stack([o[1][2] for o in ow]))
    return wl, d, w1, w2, ow, W1, W2


def _tiny_compare(wl, ow, W1, W2, b, gs_x, gs_h, out, g, n_shared=0):
    """Every stage of the GPU layer (out, stages g) against the oracle layer
    run with the same activation global scales."""
    ref, st = moe.moe_layer(b["x"].numpy(), b["logits"].numpy(), wl.k, W1, W2, gs_x, gs_h, return_stages=True,
                            n_shared=n_shared)
    assert np.array_equal(to_np(g["xc"]), st["xq"][0]) and np.array_equal(to_np(g["xs"]), st["xq"][1])
    for k_ in ("ids", "offsets", "sorted_ids", "inv"):
        assert np.array_equal(to_np(g[k_]), st[k_]), k_
    assert np.array_equal(to_np(g["w"]).view(np.uint32), st["w"].view(np.uint32))
    g_gu, g_hc, g_hs, g_y = to_np(g["gate_up"]), to_np(g["hc"]), to_np(g["hs"]), to_np(g["y"])
    off = st["offsets"]
    flips = 0
    for e in range(wl.E + n_shared):
        rows = np.arange(off[e], off[e + 1])
        if rows.size:
            flips += _expert_rows_check(wl, e, rows, st["sorted_ids"][rows], st["xq"], gs_x, gs_h, ow[e][0],
                                        ow[e][1], g_gu, g_hc, g_hs, g_y)
    o = to_np(out)
    c = cosine(o, ref)
    rel = np.abs(o - ref).max() / np.sqrt(np.mean(ref.astype(np.float64) ** 2))
    assert c >= 0.999
    if flips == 0:
        assert np.array_equal(o, ref) or rel <= 2e-2
    return c, rel, flips


def test_tiny_layer_end_to_end():
    log("pipeline tiny")
    wl, d, w1, w2, ow, W1, W2 = _tiny_setup()
    warm = workloads.warmup_batch(wl)
    gs_x = quant.global_scale(quant.amax(warm["x"].numpy()))
    _, wst = moe.moe_layer(warm["x"].numpy(), warm["logits"].numpy(), wl.k, W1, W2, gs_x, F32(1), return_stages=True)
    gs_h = quant.global_scale(quant.amax(wst["h"]))
    b = workloads.batch(wl)
    run = lambda fused: pipeline.moe_layer(b["x"].to(d, torch.bfloat16), b["logits"].to(d), wl.k, w1, w2,
                                           torch.tensor([gs_x], device=d), torch.tensor([gs_h], device=d),
                                           keep=True, fused=fused)
    out, g = run(False)
    c, rel, flips = _tiny_compare(wl, ow, W1, W2, b, gs_x, gs_h, out, g)
    _fused_same((out, g), run(True))
    log("  tiny: cosine %.7f, max-abs/rms %.3g, audited flips %d; fused epilogue identical" % (c, rel, flips))


def test_tiny_layer_dynamic_activation_scales():
    # gs_x and gs_h from this batch, on the device: gs_x must equal the
    # oracle's amax(x)/2688 of the same bf16 x, and gs_h the oracle's
    # amax(SiLU(g)*u)/2688 of the GPU's own L1 output (the stage's input);
    # the layer is then checked stage by stage with those scales
    log("pipeline tiny, dynamic activation scales")
    wl, d, w1, w2, ow, W1, W2 = _tiny_setup()
    b = workloads.batch(wl)
    out, g = pipeline.moe_layer(b["x"].to(d, torch.bfloat16), b["logits"].to(d), wl.k, w1, w2, None, None,
                                keep=True)
    gs_x = to_np(g["gs_x"])[0]
    gs_h = to_np(g["gs_h"])[0]
    assert gs_x == quant.global_scale(quant.amax(b["x"].numpy()))
    assert gs_h == quant.global_scale(quant.amax(moe.silu_mul(to_np(g["gate_up"]))))
    c, rel, flips = _tiny_compare(wl, ow, W1, W2, b, gs_x, gs_h, out, g)
    log("  tiny dynamic: gs_x %.6g, gs_h %.6g, cosine %.7f, audited flips %d" % (gs_x, gs_h, c, flips))


def test_tiny_layer_shared_expert_folded():
    # one shared expert folded into the routed layer as group E (every token,
    # weight 1, added after the routed slots): every stage against the oracle
    # layer with the same fold, both SiLU-requant paths identical
    log("pipeline tiny, shared expert folded in as group E")
    wl, d, w1, w2, ow, W1, W2 = _tiny_setup(n_shared=1)
    warm = workloads.warmup_batch(wl)
    gs_x = quant.global_scale(quant.amax(warm["x"].numpy()))
    _, wst = moe.moe_layer(warm["x"].numpy(), warm["logits"].numpy(), wl.k, W1, W2, gs_x, F32(1),
                           return_stages=True, n_shared=1)
    gs_h = quant.global_scale(quant.amax(wst["h"]))
    b = workloads.batch(wl)
    run = lambda fused: pipeline.moe_layer(b["x"].to(d, torch.bfloat16), b["logits"].to(d), wl.k, w1, w2,
                                           torch.tensor([gs_x], device=d), torch.tensor([gs_h], device=d),
                                           keep=True, fused=fused, n_shared=1)
    out, g = run(False)
    c, rel, flips = _tiny_compare(wl, ow, W1, W2, b, gs_x, gs_h, out, g, n_shared=1)
    _fused_same((out, g), run(True))
    assert to_np(g["offsets"])[wl.E + 1] - to_np(g["offsets"])[wl.E] == wl.T
    # a group-range view of the stack is the routed experts' own stack
    w1r, w2r = pipeline.moe_weights(wl, d)
    args = (b["x"].to(d, torch.bfloat16), b["logits"].to(d), wl.k)
    scales = (torch.tensor([gs_x], device=d), torch.tensor([gs_h], device=d))
    o_view = pipeline.moe_layer(*args, w1.groups(0, wl.E), w2.groups(0, wl.E), *scales)
    o_own = pipeline.moe_layer(*args, w1r, w2r, *scales)
    assert torch.equal(o_view, o_own)
    log("  tiny + shared: cosine %.7f, max-abs/rms %.3g, audited flips %d" % (c, rel, flips))


@pytest.mark.parametrize("n_shared", [0, 1])
def test_tiny_layer_one_token_and_empty_batch(n_shared):
    # one token: every stage against the oracle; no token: an empty output
    # (the route writes zero offsets, the GEMMs and the combine do nothing)
    log("pipeline tiny: T=1 and T=0, n_shared=%d" % n_shared)
    wl, d, w1, w2, ow, W1, W2 = _tiny_setup(n_shared=n_shared)
    b = workloads.batch(wl, seed=5, tokens=1)
    gs_x = quant.global_scale(quant.amax(b["x"].numpy()))
    _, st = moe.moe_layer(b["x"].numpy(), b["logits"].numpy(), wl.k, W1, W2, gs_x, F32(1), return_stages=True,
                          n_shared=n_shared)
    gs_h = quant.global_scale(quant.amax(st["h"]))
    out, g = pipeline.moe_layer(b["x"].to(d, torch.bfloat16), b["logits"].to(d), wl.k, w1, w2,
                                torch.tensor([gs_x], device=d), torch.tensor([gs_h], device=d), keep=True,
                                fused=False, n_shared=n_shared)
    _tiny_compare(wl, ow, W1, W2, b, gs_x, gs_h, out, g, n_shared=n_shared)
    x0 = torch.empty(0, wl.H, dtype=torch.bfloat16, device=d)
    l0 = torch.empty(0, wl.E, dtype=torch.float32, device=d)
    out0, g0 = pipeline.moe_layer(x0, l0, wl.k, w1, w2, torch.tensor([gs_x], device=d),
                                  torch.tensor([gs_h], device=d), keep=True, n_shared=n_shared)
    torch.cuda.synchronize()
    assert out0.shape == (0, wl.H)
    assert (to_np(g0["offsets"]) == 0).all() and g0["offsets"].shape == (wl.E + n_shared + 1,)


@pytest.mark.parametrize("n_shared", [0, 1])
def test_tiny_layer_graph_replays_match_eager(n_shared):
    # the routed layer (routing, permutation, both grouped GEMMs, SiLU-requant
    # in either place, combine) captured in a HIP graph gives the eager output
    # bit for bit on every replay, with eager work and synchronisation between
    # the replays; the inputs are refilled in place before each replay
    log("pipeline tiny: graph replays vs eager, n_shared=%d" % n_shared)
    wl = workloads.WORKLOADS["tiny"]
    d = dev()
    w1, w2 = pipeline.moe_weights(wl, d, n_shared=n_shared)
    b0, b1 = workloads.batch(wl, seed=0), workloads.batch(wl, seed=2)
    x = b0["x"].to(d, torch.bfloat16)
    logits = b0["logits"].to(d)
    gs_x = ops.global_scale(x.reshape(1, -1))
    gs_h = torch.tensor([0.01], dtype=torch.float32, device=d)
    for fused in (False, True):
        layer = lambda: pipeline.moe_layer(x, logits, wl.k, w1, w2, gs_x, gs_h, fused=fused, n_shared=n_shared)
        refs = []
        for bb in (b0, b1):
            x.copy_(bb["x"].to(d, torch.bfloat16))
            logits.copy_(bb["logits"].to(d))
            refs.append(to_np(layer().view(torch.int16)))
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            layer()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            out = layer()
        for r in range(4):
            bb = (b0, b1)[r % 2]
            x.copy_(bb["x"].to(d, torch.bfloat16))
            logits.copy_(bb["logits"].to(d))
            graph.replay()
            torch.cuda.synchronize()
            assert np.array_equal(to_np(out.view(torch.int16)), refs[r % 2]), "fused=%s replay %d" % (fused, r)
            layer()                      # eager work between replays
            torch.cuda.synchronize()
        del graph


# --- shared expert: full size -----------------------------------------------------

def test_shared_expert_full_size():
    log("pipeline shared expert T=128, 7168 -> 2x3072 -> 7168")
    wl = workloads.WORKLOADS["shared"]
    d = dev()
    w1, w2 = pipeline.moe_weights(wl, d, experts=1)
    o1, o2 = _oracle_moe_expert(wl, 0, "cpu")
    _check_weights(w1, 0, o1)
    _check_weights(w2, 0, o2)
    b = workloads.batch(wl)
    warm = workloads.warmup_batch(wl)
    gs_x = quant.global_scale(quant.amax(warm["x"].numpy()))
    W1 = tuple(a[None] for a in o1)
    W2 = tuple(a[None] for a in o2)
    _, wst = moe.shared_expert(warm["x"].numpy(), W1, W2, gs_x, F32(1), return_stages=True)
    gs_h = quant.global_scale(quant.amax(wst["h"]))
    ref, st = moe.shared_expert(b["x"].numpy(), W1, W2, gs_x, gs_h, return_stages=True)
    run = lambda fused: pipeline.shared_expert(b["x"].to(d, torch.bfloat16), w1, w2, torch.tensor([gs_x], device=d),
                                               torch.tensor([gs_h], device=d), keep=True, fused=fused)
    y, g = run(False)
    _fused_same((y, g), run(True))
    assert np.array_equal(to_np(g["xc"]), st["xq"][0]) and np.array_equal(to_np(g["xs"]), st["xq"][1])
    rows = np.arange(wl.T)
    flips = _expert_rows_check(wl, 0, rows, rows, st["xq"], gs_x, gs_h, o1, o2, to_np(g["gate_up"]),
                               to_np(g["hc"]), to_np(g["hs"]), to_np(y))
    c = cosine(to_np(y), ref)
    log("  shared: cosine %.7f, audited flips %d" % (c, flips))
    assert c >= 0.999


def test_shared_expert_graph_replays_match_eager():
    # the shared expert captured in a HIP graph (as the bench times it: split-K
    # GEMMs, their reductions, quantise and SiLU-requant) gives the eager
    # result on every replay, with eager work and synchronisation in between
    log("pipeline shared expert: graph replays vs eager")
    wl = workloads.WORKLOADS["shared"]
    d = dev()
    w1, w2 = pipeline.moe_weights(wl, d, experts=1)
    x = workloads.batch(wl)["x"].to(d, torch.bfloat16)
    gs_x = ops.global_scale(x.reshape(1, -1))
    off = pipeline.one_group_offsets(wl.T, d)
    xc, xs = ops.quantize(x, gs_x)
    gs_h = ops.silu_mul_global_scale(w1.gemm(xc, xs, gs_x, off, wl.T))
    ref = to_np(pipeline.shared_expert(x, w1, w2, gs_x, gs_h).view(torch.int16))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pipeline.shared_expert(x, w1, w2, gs_x, gs_h)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        y = pipeline.shared_expert(x, w1, w2, gs_x, gs_h)
    for r in range(4):
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_np(y.view(torch.int16)), ref), "replay %d" % r
        pipeline.shared_expert(x, w1, w2, gs_x, gs_h)     # eager work between replays
        torch.cuda.synchronize()


# --- MLA projections: full size, sampled rows ----------------------------------

def test_mla_projections_full_size():
    log("pipeline MLA T=4096: 7168 -> 1536+512 (dual gs), 1536 -> 65536")
    wl = workloads.WORKLOADS["mla"]
    d = dev()
    b = workloads.batch(wl)
    x1, x2 = b["x"].numpy(), b["x2"].numpy()
    f1, f2 = workloads.mla_weights(wl)
    f1, f2 = f1.numpy(), f2.numpy()
    nq = wl.n_qa
    gq, gk = quant.global_scale(quant.amax(f1[:nq])), quant.global_scale(quant.amax(f1[nq:]))
    cq, sq = quant.quantize(f1[:nq], gq)
    ck, sk = quant.quantize(f1[nq:], gk)
    cb, sb, gb = moe.quantize_weight(f2)
    wq = pipeline.quantize_stack([torch.from_numpy(f1)], (0, nq, f1.shape[0]), d)
    wb = pipeline.quantize_stack([torch.from_numpy(f2)], (0, f2.shape[0]), d)
    assert np.array_equal(to_np(wq.codes[0]), np.concatenate([cq, ck]))
    assert np.array_equal(to_np(wq.scales[0]), np.concatenate([sq, sk]))
    assert np.array_equal(to_np(wq.gs[0]), np.array([gq, gk], np.float32))
    assert np.array_equal(to_np(wb.codes[0]), cb) and np.array_equal(to_np(wb.scales[0]), sb)
    warm = workloads.warmup_batch(wl)
    g1 = quant.global_scale(quant.amax(warm["x"].numpy()))
    g2 = quant.global_scale(quant.amax(warm["x2"].numpy()))
    o1, o2 = pipeline.mla_projections(bf16_tensor(x1, d), bf16_tensor(x2, d), wq, wb,
                                      torch.tensor([g1], device=d), torch.tensor([g2], device=d))
    x1q = quant.quantize(x1, g1)
    x2q = quant.quantize(x2, g2)
    rows = np.random.default_rng(0).choice(wl.T, 48, replace=False)
    rows.sort()
    o1n, o2n = to_np(o1), to_np(o2)
    ex, ab = exact_gemm_rows(x1q[0][rows], x1q[1][rows], np.concatenate([cq, ck]), np.concatenate([sq, sk]))
    alpha = np.concatenate([np.full(nq, float(F32(g1 * gq))), np.full(wl.n_kv, float(F32(g1 * gk)))])
    check_gemm(o1n[rows], ex, ab, alpha[None, :], wl.H, True, "q_a+kv")
    cols = np.random.default_rng(1).choice(wl.n_qb, 4096, replace=False)
    cols.sort()
    ex, ab = exact_gemm_rows(x2q[0][rows], x2q[1][rows], cb[cols], sb[cols])
    check_gemm(o2n[rows][:, cols], ex, ab, float(F32(g2 * gb)), wl.q_lora, True, "q_b")
    assert np.isfinite(o1n).all() and np.isfinite(o2n).all()


# --- routed layers at full size: sampled token, its experts, their rows ------------

def _routed_full(name, max_rows_per_expert, n_shared=0):
    wl = workloads.WORKLOADS[name]
    d = dev()
    log("pipeline %s: T=%d, %d experts + %d shared, top-%d; drawing and quantising weights" % (
        name, wl.T, wl.E, n_shared, wl.k))
    w1, w2 = pipeline.moe_weights(wl, d, n_shared=n_shared)
    b = workloads.batch(wl)
    x, logits = b["x"].numpy(), b["logits"].numpy()
    warm = workloads.warmup_batch(wl)
    gs_x = quant.global_scale(quant.amax(warm["x"].numpy()))
    # routing and permutation: whole batch, bit-exact
    xq = quant.quantize(x, gs_x)
    ids, wts = moe.route_topk(logits, wl.k)
    if n_shared:
        ids, wts = moe.append_shared(ids, wts, wl.E, n_shared)
    off, srt, inv = moe.permute(ids, wl.E + n_shared)
    # the sampled token and its experts, quantised by the oracle
    t0 = 0
    experts = [int(e) for e in ids[t0]]
    log("  token %d routes to experts %s; quantising them in the oracle" % (t0, experts))
    ow = {e: _oracle_moe_expert(wl, e, d) for e in experts}
    # gs_h for this test: amax of the oracle's h over the sampled rows (the
    # oracle originates it; how the scalar is chosen does not affect parity)
    hs_all = []
    for e in experts:
        rows = np.arange(off[e], off[e + 1])[:max_rows_per_expert]
        ex, _ = exact_gemm_rows(xq[0][srt[rows]], xq[1][srt[rows]], ow[e][0][0], ow[e][0][1])
        gu = (ex * _l1_alpha(gs_x, ow[e][0][2], wl.I)[None, :]).astype(np.float32)
        hs_all.append(moe.silu_mul(gu))
    gs_h = quant.global_scale(max(quant.amax(h) for h in hs_all))
    run = lambda fused: pipeline.moe_layer(b["x"].to(d, torch.bfloat16), b["logits"].to(d), wl.k, w1, w2,
                                           torch.tensor([gs_x], device=d), torch.tensor([gs_h], device=d),
                                           keep=True, fused=fused, n_shared=n_shared)
    out, g = run(False)
    _fused_same((out, g), run(True))
    torch.cuda.synchronize()
    assert np.array_equal(to_np(g["xc"]), xq[0]) and np.array_equal(to_np(g["xs"]), xq[1])
    assert np.array_equal(to_np(g["ids"]), ids)
    assert np.array_equal(to_np(g["w"]).view(np.uint32), wts.view(np.uint32))
    assert np.array_equal(to_np(g["offsets"]), off)
    assert np.array_equal(to_np(g["sorted_ids"]), srt)
    assert np.array_equal(to_np(g["inv"]), inv)
    for e in experts:
        _check_weights(w1, e, ow[e][0])
        _check_weights(w2, e, ow[e][1])
    # per-stage rows of the sampled experts (the token's own row included)
    flips = 0
    g_gu, g_hc, g_hs, g_y = (to_np(g["gate_up"]), to_np(g["hc"]), to_np(g["hs"]), to_np(g["y"]))
    for j, e in enumerate(experts):
        rows = np.arange(off[e], off[e + 1])[:max_rows_per_expert]
        rows = np.union1d(rows, [inv[t0, j]])
        flips += _expert_rows_check(wl, e, rows, srt[rows], xq, gs_x, gs_h, ow[e][0], ow[e][1],
                                    g_gu, g_hc, g_hs, g_y)
    # the token's whole layer output from the oracle
    W1 = tuple(np.stack([ow[e][0][i] for e in experts]) for i in range(3))
    W2 = tuple(np.stack([ow[e][1][i] for e in experts]) for i in range(3))
    # the token's logits restricted to its own routed experts, in slot order:
    # routing over them reproduces the same slots and weights (the shared
    # experts follow as the last groups)
    ref = moe.moe_layer(x[t0:t0 + 1], logits[t0:t0 + 1, experts[:wl.k]], wl.k, W1, W2, gs_x, gs_h,
                        n_shared=n_shared)
    o = to_np(out)[t0]
    c = cosine(o, ref[0])
    log("  %s: token %d cosine %.7f, audited flips %d, experts touched %d" % (
        name, t0, c, flips, int((np.diff(off) > 0).sum())))
    assert c >= 0.999
    assert np.isfinite(to_np(out)).all()
    del w1, w2, out, g
    torch.cuda.empty_cache()


def test_decode_layer_full_size_sampled():
    _routed_full("decode", max_rows_per_expert=64)


def test_prefill_layer_full_size_sampled():
    _routed_full("prefill", max_rows_per_expert=24)


def test_decode_layer_shared_expert_folded_full_size_sampled():
    # the decode layer with one shared expert (7168 -> 2x3072 -> 7168) folded
    # in as group 384: 385 groups per GEMM, 7 slots per token
    _routed_full("decode", max_rows_per_expert=64, n_shared=1)


# --- attention output path (wo_a FP8, wo_b NVFP4): full size, sampled ----------

def test_attention_output_full_size_sampled():
    log("pipeline attention output T=4096: 65536 -(FP8)-> 1024 -(NVFP4)-> 7168")
    wl = workloads.WORKLOADS["attn_out"]
    d = dev()
    fa, fb = workloads.attn_out_weights(wl, device=d)
    codes, scales = ops.fp8_quantize_weight(fa)
    # the FP8 weights of two sampled 128-row blocks, bit-exact with the oracle
    blocks = [0, wl.o_lora // 128 - 1]
    cols = np.concatenate([np.arange(b * 128, (b + 1) * 128) for b in blocks])
    fa_s = fa[torch.from_numpy(cols).to(d)].cpu().numpy()
    c_ref = np.empty((cols.size, wl.n_qb), np.uint8)
    s_ref = np.empty((len(blocks), wl.n_qb // 128), np.float32)
    for i in range(len(blocks)):
        c_ref[i * 128:(i + 1) * 128], s_ref[i] = fp8.quantize_weight(fa_s[i * 128:(i + 1) * 128])
    assert np.array_equal(to_np(codes)[cols], c_ref)
    assert np.array_equal(to_np(scales)[blocks], s_ref)
    w_ob = pipeline.quantize_stack([fb], (0, wl.H), d)
    cb, sb, gb = moe.quantize_weight(fb.cpu().numpy())
    assert np.array_equal(to_np(w_ob.codes[0]), cb) and np.array_equal(to_np(w_ob.scales[0]), sb)
    del fa
    xw = workloads.warmup_batch(wl)["x"].to(d, torch.bfloat16)
    gs_o = ops.global_scale(ops.fp8_weight_gemm(xw, codes, scales).reshape(1, -1))
    x = workloads.batch(wl)["x"]
    o, y = pipeline.attention_output(x.to(d, torch.bfloat16), codes, scales, w_ob, gs_o)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(3).choice(wl.T, 32, replace=False))
    xs = x[torch.from_numpy(rows)].numpy()
    # wo_a on the sampled rows and blocks: the float32 summation bound
    W = fp8.dequantize_weight(c_ref, s_ref)        # the two sampled 128-row blocks
    exact = xs.astype(np.float64) @ W.T
    absum = np.abs(xs.astype(np.float64)) @ np.abs(W).T
    check_gemm(to_np(o)[rows][:, cols], exact, absum, 1.0, wl.n_qb, True, "wo_a")
    # wo_b from the GPU's own intermediate (teacher-forced): quantised with
    # gs_o by the oracle, then the NVFP4 GEMM bound
    g = to_np(gs_o)[0]
    o_rows = to_np(o)[rows]
    oq = quant.quantize(o_rows, g)
    ex2, ab2 = exact_gemm_rows(oq[0], oq[1], cb, sb)
    check_gemm(to_np(y)[rows], ex2, ab2, float(F32(F32(g) * gb)), wl.o_lora, True, "wo_b")
    log("  attention output: sampled rows within bound")
