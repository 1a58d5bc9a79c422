"""End-to-end parity of the HIP pipeline against the oracle on the five
workloads (tiny, shared expert, MLA projections, decode and prefill layers).

Both sides start from the same seeded float32 draws; each quantises them with
its own quantiser (checked bit-exact), then runs its own pipeline.  Gates:
* bit-exact: quantised x and weights, routing ids and weights, offsets,
  sorted token ids and the inverse permutation;
* every stage teacher-forced (the oracle fed the GPU's own input to that
  stage): L1 output within the float32 summation bound of the exact
  contraction, max-abs <= 2e-2 RMS and cosine >= 0.999; SiLU-requant of the
  GPU's L1 output bit-exact; L2 output (bf16) within the bound, the bf16
  rounding rule and the max-abs gate; the combine of the GPU's L2 output
  bit-exact;
* free-running (the oracle from the layer input alone): the re-quantised
  intermediate identical except at rounding boundaries of the oracle's own
  pre-rounding values (audited), and the layer output gated on max-abs <=
  2e-2 RMS and cosine >= 0.999 always.
Full-size routed layers cover every expert and every token: L1 and L2 on a
fixed set of 256 output columns of every row of every expert, SiLU-requant
and the combine on every row and token.
"""
import concurrent.futures

import numpy as np
import pytest
import torch

from _helpers import (F32, audit_code_flips, bf16_tensor, check_gemm, cosine, dev, exact_gemm_rows, layer_gate,
                      log, to_np)
from block_scaled_fp4_03_amd import ops, pipeline, workloads
from oracle import fp8, moe, quant

pytestmark = pytest.mark.gpu


def _oracle_moe_expert(wl, e, gen_device):
    """Oracle-quantised (W1 codes, scales, gs[2]), (W2 codes, scales, gs[1])
    of expert e from the seeded float32 draws."""
    return _oracle_quantize_expert(wl, workloads.moe_gate_up(wl, e, 0, gen_device).cpu().numpy(),
                                   workloads.moe_down(wl, e, 0, gen_device).cpu().numpy())


def _oracle_quantize_expert(wl, m1, m2):
    I = wl.I
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
    tokens: their token ids) with oracle weights o1/o2.  Teacher-forced: L1
    from x, SiLU-requant from the GPU's L1 output (bit-exact), L2 from the
    GPU's intermediate.  Free-running: the GPU's intermediate against the
    oracle's own (from its exact L1), differences audited.  Returns the
    number of audited intermediate flips."""
    I, H = wl.I, wl.H
    ex, ab = exact_gemm_rows(xq[0][tokens], xq[1][tokens], o1[0], o1[1])
    check_gemm(g_gu[rows], ex, ab, _l1_alpha(gs_x, o1[2], I)[None, :], H, False, "L1 expert %d" % e)
    hc_t, hs_t = moe.silu_mul_requant(g_gu[rows], gs_h)
    assert np.array_equal(g_hc[rows], hc_t) and np.array_equal(g_hs[rows], hs_t), "SiLU-requant expert %d" % e
    # oracle's own L1 output (rounded to float32) -> h -> NVFP4
    gu = (ex * _l1_alpha(gs_x, o1[2], I)[None, :]).astype(np.float32)
    h = moe.silu_mul(gu)
    hc, hs = quant.quantize(h, gs_h)
    pre_s, pre_v = quant.pre_rounding_values(h, gs_h)
    n_s, n_c = audit_code_flips(g_hc[rows], g_hs[rows], hc, hs, pre_s, pre_v)
    # L2 from the GPU's intermediate
    ex2, ab2 = exact_gemm_rows(g_hc[rows], g_hs[rows], o2[0], o2[1])
    alpha2 = float(F32(gs_h * o2[2][0]))
    check_gemm(g_y[rows], ex2, ab2, alpha2, I, True, "L2 expert %d" % e)
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


def _persistent_same(default, persistent):
    """The layer with the expert MLP as one persistent launch must give the
    default path's intermediate, second-GEMM output and layer output bit for
    bit (in the streaming regime both run the same tiles)."""
    (o0, g0), (o1, g1) = default, persistent
    for k_ in ("hc", "hs"):
        assert np.array_equal(to_np(g0[k_]), to_np(g1[k_])), k_
    assert torch.equal(g0["y"].view(torch.int16), g1["y"].view(torch.int16))
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))


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
    # the combine of the GPU's own L2 output: bit-exact
    assert np.array_equal(o.view(np.uint32), moe.combine(g_y, to_np(g["inv"]), to_np(g["w"])).view(np.uint32))
    # the layer output against the free-running oracle: max-abs and cosine
    c, rel = layer_gate(o, ref, "tiny layer output")
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
    # (the unfused route, which keeps the float32 gate_up for these checks);
    # the default route (h in float32 and the maxima of |h| from the first
    # GEMM's epilogue, then h quantised) must give its h, gs_h, intermediate
    # and output bit for bit
    log("pipeline tiny, dynamic activation scales")
    wl, d, w1, w2, ow, W1, W2 = _tiny_setup()
    b = workloads.batch(wl)
    run = lambda fused: pipeline.moe_layer(b["x"].to(d, torch.bfloat16), b["logits"].to(d), wl.k, w1, w2, None,
                                           None, keep=True, fused=fused)
    out, g = run(False)
    gs_x = to_np(g["gs_x"])[0]
    gs_h = to_np(g["gs_h"])[0]
    assert gs_x == quant.global_scale(quant.amax(b["x"].numpy()))
    assert gs_h == quant.global_scale(quant.amax(moe.silu_mul(to_np(g["gate_up"]))))
    c, rel, flips = _tiny_compare(wl, ow, W1, W2, b, gs_x, gs_h, out, g)
    out2, g2 = run(None)
    assert "gate_up" not in g2 and "h_f32" in g2
    assert np.array_equal(to_np(g2["h_f32"]).view(np.uint32), moe.silu_mul(to_np(g["gate_up"])).view(np.uint32))
    assert to_np(g2["gs_h"])[0] == gs_h
    for k_ in ("hc", "hs"):
        assert np.array_equal(to_np(g[k_]), to_np(g2[k_])), k_
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    log("  tiny dynamic: gs_x %.6g, gs_h %.6g, cosine %.7f, audited flips %d; float32-h route identical" % (
        gs_x, gs_h, c, flips))


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
    c, rel = layer_gate(to_np(y), ref, "shared expert output")
    log("  shared: cosine %.7f, max-abs/rms %.3g, audited flips %d" % (c, rel, flips))


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
    o1n, o2n = to_np(o1), to_np(o2)
    # every row, on 256 sampled columns of each projection (q_a and kv
    # columns both, so both global scales are covered)
    c1 = np.sort(np.concatenate([np.random.default_rng(0).choice(nq, 192, replace=False),
                                 nq + np.random.default_rng(2).choice(wl.n_kv, 64, replace=False)]))
    wqc, wqs = np.concatenate([cq, ck]), np.concatenate([sq, sk])
    ex, ab = exact_gemm_rows(x1q[0], x1q[1], wqc[c1], wqs[c1])
    alpha = np.concatenate([np.full(nq, float(F32(g1 * gq))), np.full(wl.n_kv, float(F32(g1 * gk)))])
    check_gemm(o1n[:, c1], ex, ab, alpha[None, c1], wl.H, True, "q_a+kv")
    cols = np.sort(np.random.default_rng(1).choice(wl.n_qb, 256, replace=False))
    ex, ab = exact_gemm_rows(x2q[0], x2q[1], cb[cols], sb[cols])
    check_gemm(o2n[:, cols], ex, ab, float(F32(g2 * gb)), wl.q_lora, True, "q_b")
    assert np.isfinite(o1n).all() and np.isfinite(o2n).all()


# --- routed layers at full size: every expert, every token ---------------------

def _dq_cols(codes, scales, cols):
    """float64 [len(cols), K] block-scaled values of the weight rows `cols`
    (exact), from host copies of codes [N, K/2] and scales [N, K/16]."""
    return quant.dequantize_blocks(codes[cols], scales[cols])


def _routed_full(name, n_shared=0, n_cols=256):
    """The routed layer at its full size.  Bit-exact: quantised x, routing,
    permutation, and the weights of experts 0, 1, E-1 and five seeded random
    ones (against the oracle's quantiser of the same float32 draws).  Then,
    teacher-forced, for EVERY row of EVERY expert: L1 on n_cols fixed output
    columns (half gate, and the matching up columns) against the exact
    contraction; SiLU-requant of the GPU's L1 output bit-exact; L2 on n_cols
    fixed output columns from the GPU's intermediate; the combine of the
    GPU's L2 output bit-exact for every token.  Free-running: token 0's whole
    output from the oracle's own weights and pipeline, and the intermediate
    of the spot-checked experts audited against the oracle's own."""
    wl = workloads.WORKLOADS[name]
    d = dev()
    E, k, I, H, T = wl.E, wl.k, wl.I, wl.H, wl.T
    G = E + n_shared
    log("pipeline %s: T=%d, %d experts + %d shared, top-%d; drawing and quantising weights" % (
        name, T, E, n_shared, k))
    w1, w2 = pipeline.moe_weights(wl, d, n_shared=n_shared)
    b = workloads.batch(wl)
    x, logits = b["x"].numpy(), b["logits"].numpy()
    warm = workloads.warmup_batch(wl)
    gs_x = quant.global_scale(quant.amax(warm["x"].numpy()))
    xq = quant.quantize(x, gs_x)
    ids, wts = moe.route_topk(logits, k)
    if n_shared:
        ids, wts = moe.append_shared(ids, wts, E, n_shared)
    off, srt, inv = moe.permute(ids, G)
    # spot-checked experts: 0, 1, E-1, five random ones, token 0's experts
    rng = np.random.default_rng(1234)
    spot = sorted(set([0, 1, E - 1] + rng.choice(np.arange(2, E - 1), 5, replace=False).tolist()
                      + [int(e) for e in ids[0]]))
    log("  oracle-quantising the weights of experts %s" % spot)
    mats = {e: (workloads.moe_gate_up(wl, e, 0, d).cpu().numpy(), workloads.moe_down(wl, e, 0, d).cpu().numpy())
            for e in spot}
    with concurrent.futures.ThreadPoolExecutor(8) as ex_:
        ow = dict(zip(spot, ex_.map(lambda e: _oracle_quantize_expert(wl, *mats[e]), spot)))
    del mats
    # rows of a spot expert that the free-running checks recompute with all
    # 2I and H columns: its first and last 32 (all, if fewer)
    some = lambda r: np.union1d(r[:32], r[-32:])
    # gs_h: amax of the oracle's own h over those rows (the oracle
    # originates the scalar; its choice does not affect parity)
    hs_all = [np.zeros((1, I), np.float32)]
    for e in spot:
        rows = some(np.arange(off[e], off[e + 1]))
        if rows.size:
            ex, _ = exact_gemm_rows(xq[0][srt[rows]], xq[1][srt[rows]], ow[e][0][0], ow[e][0][1])
            hs_all.append(moe.silu_mul((ex * _l1_alpha(gs_x, ow[e][0][2], I)[None, :]).astype(np.float32)))
    gs_h = quant.global_scale(max(quant.amax(h) for h in hs_all))
    run = lambda fused: pipeline.moe_layer(b["x"].to(d, torch.bfloat16), b["logits"].to(d), k, w1, w2,
                                           torch.tensor([gs_x], device=d), torch.tensor([gs_h], device=d),
                                           keep=True, fused=fused, n_shared=n_shared)
    out, g = run(False)
    fused = run(True)
    _fused_same((out, g), fused)
    if name == "decode":
        # the expert MLP as one persistent launch: identical intermediate,
        # second-GEMM output and layer output
        _persistent_same(fused, pipeline.moe_layer(b["x"].to(d, torch.bfloat16), b["logits"].to(d), k, w1, w2,
                                                   torch.tensor([gs_x], device=d), torch.tensor([gs_h], device=d),
                                                   keep=True, n_shared=n_shared, persistent=True))
    del fused
    torch.cuda.synchronize()
    assert np.array_equal(to_np(g["xc"]), xq[0]) and np.array_equal(to_np(g["xs"]), xq[1])
    assert np.array_equal(to_np(g["ids"]), ids)
    assert np.array_equal(to_np(g["w"]).view(np.uint32), wts.view(np.uint32))
    assert np.array_equal(to_np(g["offsets"]), off)
    assert np.array_equal(to_np(g["sorted_ids"]), srt)
    assert np.array_equal(to_np(g["inv"]), inv)
    for e in spot:
        _check_weights(w1, e, ow[e][0])
        _check_weights(w2, e, ow[e][1])
    # fixed output columns: n_cols/2 gate columns and the same up columns
    # (so the SiLU pairs are covered), n_cols columns of the down projection
    c_gate = np.sort(np.random.default_rng(5).choice(I, n_cols // 2, replace=False))
    c1 = np.concatenate([c_gate, c_gate + I])
    c2 = np.sort(np.random.default_rng(6).choice(H, n_cols, replace=False))
    # host copies of the GPU's weights on those columns, for every expert
    # (the spot-checked ones are bit-exact with the oracle's above; for the
    # rest the weights are the stage's input, as x is)
    i1, i2 = torch.from_numpy(c1).to(d), torch.from_numpy(c2).to(d)
    w1c, w1s, w1g = to_np(w1.codes.index_select(1, i1)), to_np(w1.scales.index_select(1, i1)), to_np(w1.gs)
    w2c, w2s, w2g = to_np(w2.codes.index_select(1, i2)), to_np(w2.scales.index_select(1, i2)), to_np(w2.gs)
    g_gu = to_np(g["gate_up"])
    g_hc, g_hs, g_y = to_np(g["hc"]), to_np(g["hs"]), to_np(g["y"])
    xdq = quant.dequantize_blocks(xq[0], xq[1])              # float64 [T, H], exact
    worst1 = worst2 = 0.0
    n_rows = 0
    for e in range(G):
        rows = np.arange(off[e], off[e + 1])
        if not rows.size:
            continue
        n_rows += rows.size
        # L1, teacher-forced from x: the n_cols columns of every row
        A = xdq[srt[rows]]
        W = quant.dequantize_blocks(w1c[e], w1s[e])
        alpha1 = np.concatenate([np.full(n_cols // 2, float(F32(gs_x * w1g[e, 0]))),
                                 np.full(n_cols // 2, float(F32(gs_x * w1g[e, 1])))])
        worst1 = max(worst1, check_gemm(g_gu[rows][:, c1], A @ W.T, np.abs(A) @ np.abs(W).T, alpha1[None, :], H,
                                        False, "L1 expert %d" % e))
        # SiLU-requant of the GPU's L1 output, every row: bit-exact
        hc_t, hs_t = moe.silu_mul_requant(g_gu[rows], gs_h)
        assert np.array_equal(g_hc[rows], hc_t) and np.array_equal(g_hs[rows], hs_t), "SiLU-requant expert %d" % e
        # L2 from the GPU's intermediate: the n_cols columns of every row
        A2 = quant.dequantize_blocks(g_hc[rows], g_hs[rows])
        W2 = quant.dequantize_blocks(w2c[e], w2s[e])
        worst2 = max(worst2, check_gemm(g_y[rows][:, c2], A2 @ W2.T, np.abs(A2) @ np.abs(W2).T,
                                        float(F32(gs_h * w2g[e, 0])), I, True, "L2 expert %d" % e))
    assert n_rows == T * (k + n_shared)
    # the combine of the GPU's L2 output, every token: bit-exact
    o = to_np(out)
    assert np.array_equal(o.view(np.uint32), moe.combine(g_y, inv, wts).view(np.uint32))
    # free-running: the spot experts' intermediate against the oracle's own
    flips = 0
    for e in spot:
        rows = some(np.arange(off[e], off[e + 1]))
        if rows.size:
            flips += _expert_rows_check(wl, e, rows, srt[rows], xq, gs_x, gs_h, ow[e][0], ow[e][1], g_gu, g_hc,
                                        g_hs, g_y)
    # free-running: token 0's whole output from the oracle's weights
    t0 = 0
    experts = [int(e) for e in ids[t0]]
    W1 = tuple(np.stack([ow[e][0][i] for e in experts]) for i in range(3))
    W2 = tuple(np.stack([ow[e][1][i] for e in experts]) for i in range(3))
    # the token's logits restricted to its own routed experts, in slot order:
    # routing over them reproduces the same slots and weights (the shared
    # experts follow as the last groups)
    ref = moe.moe_layer(x[t0:t0 + 1], logits[t0:t0 + 1, experts[:k]], k, W1, W2, gs_x, gs_h, n_shared=n_shared)
    c, rel = layer_gate(o[t0], ref[0], "%s token %d output" % (name, t0))
    log("  %s: every row of %d experts (%d rows) checked on %d L1 and %d L2 columns, worst err/rms %.3g / %.3g; "
        "token %d free-running cosine %.7f, max-abs/rms %.3g; audited flips %d" % (
            name, int((np.diff(off) > 0).sum()), n_rows, n_cols, n_cols, worst1, worst2, t0, c, rel, flips))
    assert np.isfinite(o).all()
    del w1, w2, out, g
    torch.cuda.empty_cache()


def test_decode_layer_full_size_every_expert():
    _routed_full("decode")


def test_prefill_layer_full_size_every_expert():
    _routed_full("prefill")


def test_decode_layer_shared_expert_folded_full_size_every_expert():
    # the decode layer with one shared expert (7168 -> 2x3072 -> 7168) folded
    # in as group 384: 385 groups per GEMM, 7 slots per token
    _routed_full("decode", n_shared=1)


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
