#!/usr/bin/env python3
"""Throughput of the NVFP4 MoE expert pipeline on one MI355X.

One step = one pass of the whole routed MoE layer over one batch that is
already resident in HBM: NVFP4 quantisation of x, top-6 routing and the
group-by-expert permutation, the L1 grouped GEMM over the stacked gate_up
weights, SiLU(gate)*up re-quantised to NVFP4, the L2 grouped GEMM over the
down weights, and the weighted combine back to token order (bf16 out).

Default workload: the decode layer, T=256 tokens, hidden 7168, expert
intermediate 3072, 384 experts, top-6, seeded synthetic inputs (x ~ N(0,1)
in bf16, router logits ~ N(0,1), weights ~ N(0, 0.02^2) drawn on the GPU and
quantised to NVFP4 by the library).  `--workload prefill` runs the T=8192
layer with Zipf(1.1)-skewed expert popularity; the default run also measures
it and reports it under "prefill".

Prints ONE JSON line.  `value` is tokens/s of the whole layer; `roofline`
is the dominant kernel (the L1 grouped GEMM) against its bound; `cpu_baseline`
is the CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
F16_MFMA_PEAK_TFLOPS = 2500.0    # MI355X dense bf16/f16 matrix peak, TFLOP/s
FP4_MFMA_PEAK_TFLOPS = 10100.0   # MI355X dense fp4/fp6 matrix peak, TFLOP/s (not an exact path for NVFP4)
NVFP4_BYTES_PER_ELEM = 0.5 + 1.0 / 16.0
PROFILE_DIR = os.path.join(ROOT, "profiles")
GEMM_SRC = os.path.join(ROOT, "block_scaled_fp4_03_amd", "csrc", "grouped_gemm.hip")
METRIC = "MoE layer tokens/s + TFLOP/s (% HBM roofline decode, % MFMA peak prefill)"


def kernel_source_hash():
    h = hashlib.sha256()
    with open(GEMM_SRC, "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


# untimed layer steps run once after the weights are prepared (see run_gpu)
SETTLE_STEPS = 40
# the two ways of running SiLU-requant, as the bench line names them
SILU_PATHS = {True: "fused into the first GEMM's epilogue", False: "separate kernel"}
# where the per-batch global scale of h comes from on the dynamic-scale path
DYN_PATHS = {True: "maxima of |h| written by the first GEMM's epilogue with h in float32, then h quantised",
             False: "amax of SiLU(gate)*up over the float32 gate_up, then SiLU-requant"}


def measured_traffic(workload, silu_path):
    """HBM bytes per L1 launch from committed rocprofv3 counter runs (FETCH_SIZE
    and WRITE_SIZE, scaled by the same counters on a copy of known size), or
    None when no summary exists, the kernel source changed since or the
    summary covers the other SiLU-requant path's launch."""
    path = os.path.join(PROFILE_DIR, "grouped_gemm_l1_%s_traffic.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha256_16") != kernel_source_hash() or d.get("silu_requant") != silu_path:
        return None
    return d.get("bytes_per_launch")


class Layer:
    """The routed layer on the GPU: weights, inputs, activation scales."""

    def __init__(self, wl, device):
        import torch
        from block_scaled_fp4_03_amd import lib, ops, pipeline, workloads
        self.wl = wl
        self.dev = device
        t0 = time.time()
        self.w1, self.w2 = pipeline.moe_weights(wl, device, drop_rows=True)
        torch.cuda.synchronize()
        self.weight_setup_s = time.time() - t0
        b = workloads.batch(wl, seed=0)
        self.x = b["x"].to(device=device, dtype=torch.bfloat16)
        self.logits = b["logits"].to(device)
        # activation global scales from the warmup batch (seed 1), computed by
        # the library: gs_x from amax(x_warm); gs_h from amax(SiLU(g)*u) of the
        # warmup batch's L1 output
        warm = workloads.warmup_batch(wl)
        xw = warm["x"].to(device=device, dtype=torch.bfloat16)
        self.gs_x = ops.global_scale(xw.reshape(1, -1))
        xc, xs = ops.quantize(xw, self.gs_x)
        ids, w, off, srt, inv = ops.route_permute(warm["logits"].to(device), wl.k)
        gu = self.w1.gemm(xc, xs, self.gs_x, off, xw.shape[0] * wl.k, a_row_index=srt)
        self.gs_h = ops.silu_mul_global_scale(gu)
        # whether the GEMMs take A's f16 form from its producer (many-row tiles)
        R = self.x.shape[0] * wl.k
        self.dq1 = True if self.w1.reads_dq(R, self.x.shape[0]) else None
        self.dq2 = True if self.w2.reads_dq(R, R) else None
        # the pipeline's default SiLU-requant path for this shape (in the first
        # GEMM's epilogue unless it splits K)
        self.fused_default = self.w1.fuse_by_default(R, self.x.shape[0])
        # with a per-batch gs_h: h in float32 and its maxima from the first
        # GEMM's epilogue, unless it splits K
        self.fused_dynamic = self.w1.can_fuse_silu_f32(R)
        # the one-launch expert MLP streams every tile in 32-row slots: timed
        # where the first GEMM streams its weights too (few rows per expert)
        self.streams = self.dq1 is None
        # workspace of the one-launch expert MLP (tile queue, slot counters)
        self.mlp_ws = torch.empty(max(16, lib.load().nvfp4_moe_expert_mlp_workspace_size(wl.E, R)),
                                  dtype=torch.uint8, device=device)
        torch.cuda.synchronize()

    def step(self, ev=None, dynamic=False, fused=False, persistent=False):
        """One layer pass; if ev is given, record events around each op.  With
        `dynamic`, the activation global scales come from this batch on the
        device (amax of x before quantising it, amax of SiLU(g)*u before the
        re-quantisation) instead of the warmup scalars; with `fused`, SiLU-requant
        runs in the first GEMM's epilogue (static scales only); with
        `persistent`, both GEMMs and the fused SiLU-requant run as one
        persistent launch (nvfp4_moe_expert_mlp)."""
        from block_scaled_fp4_03_amd import ops
        import torch
        wl = self.wl
        T = self.x.shape[0]
        R = T * wl.k
        rec = (lambda name: ev[name].append(torch.cuda.Event(enable_timing=True)) or ev[name][-1].record()) \
            if ev is not None else (lambda name: None)
        rec("start")
        gs_x = ops.global_scale(self.x.reshape(1, -1)) if dynamic else self.gs_x
        xc, xs, *xdq = ops.quantize(self.x, gs_x, dq=self.dq1)
        rec("quantize")
        ids, w, off, srt, inv = ops.route_permute(self.logits, wl.k)
        rec("route_permute")
        if persistent:
            G = self.w1.gs.shape[0]
            hc, hs, y = ops.moe_expert_mlp(xc, xs, gs_x, srt, off, self.w1.tiled, self.w1.gs, self.w2.tiled,
                                           self.w2.gs, R, wl.H, wl.I, self.gs_h, workspace=self.mlp_ws)
            rec("gemm_l1")
            rec("silu_mul_requant")
            rec("gemm_l2")
            out = ops.combine(y, inv, w)
            rec("combine")
            self._off = off
            return out
        if not fused:
            gu = self.w1.gemm(xc, xs, gs_x, off, R, a_row_index=srt, a_dq=xdq[0] if xdq else None)
            rec("gemm_l1")
            gs_h = ops.silu_mul_global_scale(gu) if dynamic else self.gs_h
            hc, hs, *hdq = ops.silu_mul_requant(gu, gs_h, dq=self.dq2)
            rec("silu_mul_requant")
        elif dynamic:
            # per-batch gs_h: h in float32 and the maxima of |h| from the first
            # GEMM's epilogue, then gs_h from the maxima and h quantised
            h32, part = self.w1.gemm_silu_f32(xc, xs, gs_x, off, R, a_row_index=srt, a_dq=xdq[0] if xdq else None)
            rec("gemm_l1")
            gs_h = ops.global_scale(part.view(1, -1))
            hc, hs, *hdq = ops.quantize(h32, gs_h, dq=self.dq2)
            rec("silu_mul_requant")
        else:
            # static gs_h: SiLU-requant runs in the first GEMM's epilogue
            gs_h = self.gs_h
            hc, hs, *hdq = self.w1.gemm_silu_requant(xc, xs, gs_x, off, R, gs_h, a_row_index=srt,
                                                     a_dq=xdq[0] if xdq else None, dq=self.dq2)
            rec("gemm_l1")
            rec("silu_mul_requant")
        y = self.w2.gemm(hc, hs, gs_h, off, R, out_dtype=torch.bfloat16, a_dq=hdq[0] if hdq else None)
        rec("gemm_l2")
        out = ops.combine(y, inv, w)
        rec("combine")
        self._off = off
        return out

    def saturation(self):
        """Share of the measured batch's 16-element blocks whose E4M3 scale
        saturates at 448 with the warmup's activation global scales: of x,
        and of the intermediate h (counted on one untimed pass)."""
        import torch
        from block_scaled_fp4_03_amd import ops
        wl = self.wl
        T = self.x.shape[0]
        R = T * wl.k
        xc, xs = ops.quantize(self.x, self.gs_x)
        ids, w, off, srt, inv = ops.route_permute(self.logits, wl.k)
        gu = self.w1.gemm(xc, xs, self.gs_x, off, R, a_row_index=srt)
        hc, hs = ops.silu_mul_requant(gu, self.gs_h)
        sat_x = int((xs == 0x7E).sum().item())
        sat_h = int((hs == 0x7E).sum().item())
        out = {"x_blocks": int(xs.numel()), "x_saturated": sat_x, "h_blocks": int(hs.numel()),
               "h_saturated": sat_h}
        del gu
        torch.cuda.empty_cache()
        return out

    def touched_experts(self):
        import torch
        off = self._off.cpu().numpy()
        return int((np.diff(off) > 0).sum())


def time_layer(layer, steps, warmup, dynamic=False, fused=False, persistent=False):
    """Mean ms per step over `steps` back-to-back steps (after `warmup`), the
    mean per-op ms, and the p10/p50/p90 of the per-step times.  The timed
    block holds the steps alone; the per-op and per-step figures come from
    the same number of steps run after it with an event around every op
    (those events cost about 1% of a decode step, so they stay out of the
    timed block)."""
    import torch
    for _ in range(warmup):
        layer.step(dynamic=dynamic, fused=fused, persistent=persistent)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(steps):
        layer.step(dynamic=dynamic, fused=fused, persistent=persistent)
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    names = ["start", "quantize", "route_permute", "gemm_l1", "silu_mul_requant", "gemm_l2", "combine"]
    ev = {n: [] for n in names}
    for _ in range(steps):
        layer.step(ev, dynamic=dynamic, fused=fused, persistent=persistent)
    torch.cuda.synchronize()
    per_op = {}
    for i in range(1, len(names)):
        a, b = names[i - 1], names[i]
        per_op[b] = float(np.mean([ev[a][s].elapsed_time(ev[b][s]) for s in range(steps)]))
    per_step = [ev["start"][s].elapsed_time(ev["combine"][s]) for s in range(steps)]
    pct = {"p10": float(np.percentile(per_step, 10)), "p50": float(np.percentile(per_step, 50)),
           "p90": float(np.percentile(per_step, 90))}
    return total_ms / steps, per_op, pct


def algorithmic(wl, n_touched, fused):
    """Algorithmic FLOPs of one layer and bytes of one L1 launch: the touched
    experts' W1, x in NVFP4, and the launch's output (h in NVFP4 when
    SiLU-requant runs in its epilogue, else gate_up in float32)."""
    T, H, I, k = wl.T, wl.H, wl.I, wl.k
    R = T * k
    flops = 6.0 * R * H * I
    w1_bytes = 2 * I * H * NVFP4_BYTES_PER_ELEM
    out_bytes = R * I * NVFP4_BYTES_PER_ELEM if fused else R * 2 * I * 4
    l1_bytes = n_touched * w1_bytes + T * H * NVFP4_BYTES_PER_ELEM + out_bytes
    l1_flops = 4.0 * R * H * I
    return flops, l1_bytes, l1_flops


def layer_bytes(wl, n_touched):
    """Algorithmic HBM bytes of one layer pass: the touched experts' weights
    (codes and block scales of W1 and W2), x in bf16, the router logits and
    the bf16 output."""
    per_expert = 3 * wl.H * wl.I * NVFP4_BYTES_PER_ELEM
    return n_touched * per_expert + wl.T * wl.H * 2 + wl.T * wl.E * 4 + wl.T * wl.H * 2


def measure_ceilings(steps=10):
    """What the simplest kernels reach on this chip: a 4 GiB read with the
    weight stream's non-temporal 16-byte loads (GB/s), and eight independent
    f16 32x32x16 matrix-core chains per wave on register operands (TFLOP/s),
    each timed with HIP events on the stream it runs on."""
    import torch
    from block_scaled_fp4_03_amd import ops
    dev = torch.device("cuda:0")
    sink = torch.zeros(4, dtype=torch.float32, device=dev)
    buf = torch.empty(1 << 32, dtype=torch.uint8, device=dev).fill_(3)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps * 1e-3

    t_read = timed(lambda: ops.probe_hbm_read(buf, sink))
    del buf
    iters, wgs = 20000, 512
    flops = ops.probe_mfma_f16(iters, wgs, sink)
    t_mfma = timed(lambda: ops.probe_mfma_f16(iters, wgs, sink))
    torch.cuda.empty_cache()
    return {"hbm_read_gbs": round((1 << 32) / t_read / 1e9, 1),
            "hbm_read_probe": "4 GiB read once, each of 8192 waves one contiguous 512 KiB chunk, 16 non-temporal 1 KiB wave-loads in flight",
            "f16_mfma_tflops": round(flops / t_mfma / 1e12, 1),
            "f16_mfma_probe": "v_mfma_f32_32x32x16_f16, 8 independent chains per wave, 4 waves per "
                              "workgroup, 512 workgroups, operands alternating between two random sets"}


def run_gpu(workload, steps, warmup, tokens=None):
    import dataclasses
    import torch
    from block_scaled_fp4_03_amd import workloads
    wl = workloads.WORKLOADS[workload]
    if tokens:
        wl = dataclasses.replace(wl, T=tokens)
    dev = torch.device("cuda:0")
    print("[bench] %s: preparing weights (%d experts) and inputs" % (workload, wl.E), file=sys.stderr, flush=True)
    layer = Layer(wl, dev)
    print("[bench] %s: weights ready in %.1fs, timing %d+%d steps" % (workload, layer.weight_setup_s, warmup, steps),
          file=sys.stderr, flush=True)
    # the pipeline's default path (see pipeline._expert_mlp)
    fused = layer.fused_default
    # untimed steps before the first timed block: right after the weight
    # preparation the first blocks of steps measure about 2% slow
    for _ in range(SETTLE_STEPS):
        layer.step(fused=fused)
    torch.cuda.synchronize()
    ms, per_op, pct = time_layer(layer, steps, warmup, fused=fused)
    n_touched = layer.touched_experts()
    flops, l1_bytes, l1_flops = algorithmic(wl, n_touched, fused)
    res = dict(ms=ms, per_op_ms=per_op, step_pct=pct, n_touched=n_touched, tokens_per_s=wl.T / (ms * 1e-3),
               tflops=flops / (ms * 1e-3) / 1e12, l1_bytes=l1_bytes, l1_flops=l1_flops, layer=layer, wl=wl,
               fused=fused, wl_default_T=workloads.WORKLOADS[workload].T,
               layer_bytes=layer_bytes(wl, n_touched), saturation=layer.saturation())
    # the same layer with per-batch activation global scales computed on the
    # device (an amax pass over x; gs_h from the maxima of |h| that the first
    # GEMM's epilogue writes with h in float32, then h quantised; where the
    # first GEMM splits K, from the float32 gate_up), timed the same way
    dms, dper_op, _ = time_layer(layer, steps, warmup, dynamic=True, fused=layer.fused_dynamic)
    res["dynamic"] = dict(ms=dms, per_op_ms=dper_op, tokens_per_s=wl.T / (dms * 1e-3), fused=layer.fused_dynamic)
    # and with the other SiLU-requant path (fused into the first GEMM's
    # epilogue, or as its own kernel)
    if layer.w1.can_fuse_silu():
        oms, oper_op, _ = time_layer(layer, steps, warmup, fused=not fused)
        res["other"] = dict(fused=not fused, ms=oms, l1_ms=oper_op["gemm_l1"], tokens_per_s=wl.T / (oms * 1e-3))
    # and with the expert MLP as one persistent launch (where the first GEMM
    # streams its weights: the regime that launch is built for)
    if fused and layer.streams:
        pms, pper_op, ppct = time_layer(layer, steps, warmup, persistent=True)
        res["persistent"] = dict(ms=pms, mlp_ms=pper_op["gemm_l1"] + pper_op["silu_mul_requant"] + pper_op["gemm_l2"],
                                 tokens_per_s=wl.T / (pms * 1e-3), step_pct=ppct)
    return res


def roofline(res, bound, ceilings=None):
    l1_ms = res["per_op_ms"]["gemm_l1"]
    if bound == "hbm":
        ach = res["l1_bytes"] / (l1_ms * 1e-3) / 1e9
        peak = HBM_PEAK_GBS
        unit = "GB/s"
        ceil = ceilings and ceilings["hbm_read_gbs"]
    else:
        ach = res["l1_flops"] / (l1_ms * 1e-3) / 1e12
        peak = F16_MFMA_PEAK_TFLOPS
        unit = "TFLOP/s"
        ceil = ceilings and ceilings["f16_mfma_tflops"]
    # (the committed counter runs cover the workloads at their own token counts)
    traffic = measured_traffic(res["wl"].name, SILU_PATHS[res["fused"]]) \
        if res["wl"].T == res["wl_default_T"] else None
    out = {"bound": bound, "achieved": round(ach, 1), "peak": peak, "unit": unit, "frac": round(ach / peak, 4),
           "traffic": traffic,
           "algorithmic_bytes": int(res["l1_bytes"]),
           "traffic_over_algorithmic": round(traffic / res["l1_bytes"], 3) if traffic else None,
           "kernel": "nvfp4_grouped_gemm_silu_requant L1 (gate_up, SiLU-requant epilogue)" if res["fused"]
           else "nvfp4_grouped_gemm L1 (gate_up)",
           "kernel_ms": round(l1_ms, 4)}
    if bound == "mfma":
        out["frac_of_fp4_peak"] = round(ach / FP4_MFMA_PEAK_TFLOPS, 4)
    if ceil:
        out["measured_ceiling"] = ceil
        out["frac_of_measured_ceiling"] = round(ach / ceil, 4)
    return out


def layer_roofline(res, bound, ceilings):
    """The whole layer against its bound: at decode the algorithmic bytes of
    the layer (touched experts' weights, x, logits, out) per step against HBM;
    at prefill its algorithmic flops per step against the dense f16 and fp4
    matrix peaks.  Second denominators: the measured ceilings."""
    ms = res["ms"]
    if bound == "hbm":
        gbs = res["layer_bytes"] / (ms * 1e-3) / 1e9
        out = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_step": int(res["layer_bytes"])}
        if ceilings:
            out["measured_ceiling"] = ceilings["hbm_read_gbs"]
            out["frac_of_measured_ceiling"] = round(gbs / ceilings["hbm_read_gbs"], 4)
        return out
    tf = res["tflops"]
    out = {"bound": "mfma", "achieved": round(tf, 1), "peak": F16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
           "frac": round(tf / F16_MFMA_PEAK_TFLOPS, 4),
           "frac_of_fp4_peak": round(tf / FP4_MFMA_PEAK_TFLOPS, 4),
           "fp4_peak": FP4_MFMA_PEAK_TFLOPS,
           "flops_per_step": 6.0 * res["wl"].T * res["wl"].k * res["wl"].H * res["wl"].I}
    if ceilings:
        out["measured_ceiling"] = ceilings["f16_mfma_tflops"]
        out["frac_of_measured_ceiling"] = round(tf / ceilings["f16_mfma_tflops"], 4)
    return out


def cpu_baseline(res, n_experts=24):
    """The oracle, in its float32 mode (dequantise to float32, float32 BLAS
    matmul), timed on the host on a bounded sample: n_experts of the touched
    experts with all their routed rows (L1, SiLU-requant, L2), plus the
    per-token steps (quantise, route, permute, combine) for the whole batch;
    the expert part is scaled by touched/n_experts."""
    import torch
    from block_scaled_fp4_03_amd import workloads
    from oracle import moe, quant
    layer, wl = res["layer"], res["wl"]
    x = layer.x.float().cpu().numpy()
    logits = layer.logits.cpu().numpy()
    gs_x = np.float32(layer.gs_x.item())
    gs_h = np.float32(layer.gs_h.item())
    # untimed: oracle-quantised weights of the sampled experts (from the
    # same seeded float32 weights the GPU quantised)
    ids, _ = moe.route_topk(logits, wl.k)
    experts = sorted(set(ids.reshape(-1).tolist()))[:n_experts]
    gen = "cuda:0" if wl.weights_on_device else "cpu"
    mats = [(workloads.moe_gate_up(wl, e, 0, gen).cpu().numpy(), workloads.moe_down(wl, e, 0, gen).cpu().numpy())
            for e in experts]

    def prep(m):
        m1, m2 = m
        gg = quant.global_scale(quant.amax(m1[:wl.I]))
        gu = quant.global_scale(quant.amax(m1[wl.I:]))
        cg, sg = quant.quantize(m1[:wl.I], gg)
        cu, su = quant.quantize(m1[wl.I:], gu)
        c2, s2, g2 = moe.quantize_weight(m2)
        return np.concatenate([cg, cu]), np.concatenate([sg, su]), [gg, gu], c2, s2, [g2]

    import concurrent.futures
    with concurrent.futures.ThreadPoolExecutor(8) as ex:     # setup only, not timed
        prepared = list(ex.map(prep, mats))
    del mats
    w1c, w1s, w1g, w2c, w2s, w2g = (list(z) for z in zip(*prepared))
    w1 = (np.stack(w1c), np.stack(w1s), np.array(w1g, np.float32))
    w2 = (np.stack(w2c), np.stack(w2s), np.array(w2g, np.float32))
    # timed: per-token part over the whole batch
    t0 = time.perf_counter()
    xq = quant.quantize(x, gs_x)
    ids, wts = moe.route_topk(logits, wl.k)
    off, srt, inv = moe.permute(ids, wl.E)
    t_tok = time.perf_counter() - t0
    # timed: expert part on the sampled experts with all their rows
    rows = np.concatenate([np.arange(off[e], off[e + 1]) for e in experts])
    counts = [int(off[e + 1] - off[e]) for e in experts]
    soff = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    t1 = time.perf_counter()
    gu = moe.grouped_gemm(xq[0], xq[1], gs_x, w1[0], w1[1], w1[2], [0, wl.I, 2 * wl.I], soff,
                          a_row_index=srt[rows], mode="f32")
    hq = moe.silu_mul_requant(gu, gs_h)
    y = moe.grouped_gemm(hq[0], hq[1], gs_h, w2[0], w2[1], w2[2], [0, wl.H], soff, out_dtype="bf16", mode="f32")
    t_exp = time.perf_counter() - t1
    # combine over the whole batch with stand-in rows (same arithmetic)
    yfull = np.zeros((wl.T * wl.k, wl.H), np.float32)
    yfull[rows] = y
    t2 = time.perf_counter()
    moe.combine(yfull, inv, wts)
    t_tok += time.perf_counter() - t2
    n_t = res["n_touched"]
    est = t_tok + t_exp * n_t / len(experts)
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    cpu_model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    flops = 6.0 * wl.T * wl.k * wl.H * wl.I
    return {"value": round(wl.T / est, 4), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "gflops": round(flops / est / 1e9, 2),
            "sample": "oracle in its float32 mode (dequantise to float32, float32 library matmul); "
                      "%d of %d touched experts with all their %d routed rows (L1, SiLU-requant, L2), "
                      "scaled by %d/%d; quantise, route, permute and combine over all %d tokens; "
                      "timed %.1fs of CPU work; host %d logical CPUs (%s)" % (
                          len(experts), n_t, int(sum(counts)), n_t, len(experts), wl.T, t_tok + t_exp,
                          os.cpu_count(), cpu_model)}


def time_scrubbed(step, steps, warmup):
    """Per-step times (HIP events around each step only) with a 1 GiB buffer
    rewritten between steps, so weights that would fit in the 256 MB
    Infinity Cache come from HBM every step.  The step (a handful of short
    kernels) is captured once in a HIP graph and replayed, as a
    latency-sensitive caller would run it; the host's launch cost is then
    outside the timed span.  Returns (median, p10, p90) ms."""
    import torch
    scrub = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0")
    for _ in range(warmup):
        scrub.fill_(1.0)
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                       # allocations of the capture pool's first use
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    times = []
    for _ in range(steps):
        scrub.fill_(1.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        times.append((e0, e1))
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in times]
    del scrub
    return float(np.median(ms)), float(np.percentile(ms, 10)), float(np.percentile(ms, 90))


def side_line(name, ms, p10, p90, flops, bytes_):
    tf = flops / (ms * 1e-3) / 1e12
    gbs = bytes_ / (ms * 1e-3) / 1e9
    return {"workload": name, "ms_median": round(ms, 4), "ms_p10": round(p10, 4), "ms_p90": round(p90, 4),
            "tflops": round(tf, 2), "frac_f16_mfma_peak": round(tf / F16_MFMA_PEAK_TFLOPS, 4),
            "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "algorithmic_flops": flops, "algorithmic_bytes": int(bytes_)}


def run_shared(steps, warmup):
    """Shared expert, T=128 (one group, no routing): x -> L1 -> SiLU-requant -> L2."""
    import torch
    from block_scaled_fp4_03_amd import ops, pipeline, workloads
    wl = workloads.WORKLOADS["shared"]
    dev = torch.device("cuda:0")
    w1, w2 = pipeline.moe_weights(wl, dev, experts=1, drop_rows=True)
    x = workloads.batch(wl)["x"].to(dev, torch.bfloat16)
    xw = workloads.warmup_batch(wl)["x"].to(dev, torch.bfloat16)
    gs_x = ops.global_scale(xw.reshape(1, -1))
    xc, xs = ops.quantize(xw, gs_x)
    off = torch.tensor([0, xw.shape[0]], dtype=torch.int32, device=dev)
    gs_h = ops.silu_mul_global_scale(w1.gemm(xc, xs, gs_x, off, xw.shape[0]))
    ms, p10, p90 = time_scrubbed(lambda: pipeline.shared_expert(x, w1, w2, gs_x, gs_h), steps, warmup)
    T, H, I = wl.T, wl.H, wl.I
    flops = 6.0 * T * H * I
    bytes_ = 3 * H * I * NVFP4_BYTES_PER_ELEM + 2 * T * H * 2
    return side_line("shared expert: T=%d, %d -> 2x%d -> %d, one group" % (T, H, I, H), ms, p10, p90, flops, bytes_)


def time_eager(step, steps, warmup):
    """ms per step of `steps` back-to-back eager steps (HIP events around
    the whole run), after `warmup` untimed ones."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def run_decode_shared(steps, warmup):
    """The decode layer with one shared expert (7168 -> 2x3072 -> 7168):
    folded in as group 384 of both grouped GEMMs (every token visits it with
    weight 1, added after the routed slots in the combine), against the
    routed layer followed by the shared expert on its own (one-group GEMMs
    with split K), on the same weights (group-range views of one stack) and
    the same activation global scales."""
    import torch
    from block_scaled_fp4_03_amd import ops, pipeline, workloads
    wl = workloads.WORKLOADS["decode"]
    dev = torch.device("cuda:0")
    E, k = wl.E, wl.k
    w1, w2 = pipeline.moe_weights(wl, dev, drop_rows=True, n_shared=1)
    b = workloads.batch(wl)
    x = b["x"].to(dev, torch.bfloat16)
    logits = b["logits"].to(dev)
    warm = workloads.warmup_batch(wl)
    xw = warm["x"].to(dev, torch.bfloat16)
    gs_x = ops.global_scale(xw.reshape(1, -1))
    xc, xs = ops.quantize(xw, gs_x)
    _, _, off, srt, _ = ops.route_permute(warm["logits"].to(dev), k, n_shared=1)
    gs_h = ops.silu_mul_global_scale(w1.gemm(xc, xs, gs_x, off, xw.shape[0] * (k + 1), a_row_index=srt))
    w1r, w2r, w1s, w2s = w1.groups(0, E), w2.groups(0, E), w1.groups(E, E + 1), w2.groups(E, E + 1)

    def folded():
        return pipeline.moe_layer(x, logits, k, w1, w2, gs_x, gs_h, n_shared=1)

    def separate():
        pipeline.moe_layer(x, logits, k, w1r, w2r, gs_x, gs_h)
        return pipeline.shared_expert(x, w1s, w2s, gs_x, gs_h)

    tf, ts = [], []
    for _ in range(2):                   # alternated, against drift of the clock
        tf.append(time_eager(folded, steps, warmup))
        ts.append(time_eager(separate, steps, warmup))
    out, st = pipeline.moe_layer(x, logits, k, w1, w2, gs_x, gs_h, keep=True, n_shared=1)
    n_touched = int((np.diff(st["offsets"].cpu().numpy()[:E + 1]) > 0).sum())
    ms_f, ms_s = float(np.median(tf)), float(np.median(ts))
    T, H, I = wl.T, wl.H, wl.I
    flops = 6.0 * T * (k + 1) * H * I
    bytes_ = (n_touched + 1) * 3 * H * I * NVFP4_BYTES_PER_ELEM + T * H * 2 * 2 + T * E * 4
    del w1, w2, w1r, w2r, w1s, w2s
    return {"workload": "decode MoE layer + 1 shared expert: T=%d, %d routed experts top-%d, shared expert "
                        "folded in as group %d" % (T, E, k, E),
            "ms_per_step": round(ms_f, 4), "tokens_per_s": round(T / (ms_f * 1e-3), 1),
            "tflops": round(flops / (ms_f * 1e-3) / 1e12, 2),
            "gbs": round(bytes_ / (ms_f * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(bytes_ / (ms_f * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "separate_ms_per_step": round(ms_s, 4),
            "separate": "routed layer, then the shared expert's own one-group GEMMs (split K)",
            "experts_touched": n_touched, "algorithmic_bytes": int(bytes_)}


def run_mla(steps, warmup):
    """MLA projections, T=4096: fused q_a+kv (dual gs), then q_b."""
    import torch
    from block_scaled_fp4_03_amd import ops, pipeline, workloads
    wl = workloads.WORKLOADS["mla"]
    dev = torch.device("cuda:0")
    f1, f2 = workloads.mla_weights(wl, device=dev)
    wq = pipeline.quantize_stack([f1], (0, wl.n_qa, f1.shape[0]), dev)
    wb = pipeline.quantize_stack([f2], (0, f2.shape[0]), dev)
    del f1, f2
    b = workloads.batch(wl)
    x1, x2 = b["x"].to(dev, torch.bfloat16), b["x2"].to(dev, torch.bfloat16)
    warm = workloads.warmup_batch(wl)
    g1 = ops.global_scale(warm["x"].to(dev, torch.bfloat16).reshape(1, -1))
    g2 = ops.global_scale(warm["x2"].to(dev, torch.bfloat16).reshape(1, -1))
    ms, p10, p90 = time_scrubbed(lambda: pipeline.mla_projections(x1, x2, wq, wb, g1, g2), steps, warmup)
    T, H = wl.T, wl.H
    n1, n2 = wl.n_qa + wl.n_kv, wl.n_qb
    flops = 2.0 * T * n1 * H + 2.0 * T * n2 * wl.q_lora
    bytes_ = (n1 * H + n2 * wl.q_lora) * NVFP4_BYTES_PER_ELEM + T * (H + wl.q_lora) * 2 + T * (n1 + n2) * 2
    torch.cuda.empty_cache()
    return side_line("MLA projections: T=%d, %d -> %d+%d (dual gs), %d -> %d" % (
        T, H, wl.n_qa, wl.n_kv, wl.q_lora, n2), ms, p10, p90, flops, bytes_)


def run_attn_out(steps, warmup):
    """Attention output path, T=4096: wo_a (FP8 weight-only, 65536 -> 1024)
    then wo_b (NVFP4, 1024 -> 7168); and wo_a alone."""
    import torch
    from block_scaled_fp4_03_amd import ops, pipeline, workloads
    wl = workloads.WORKLOADS["attn_out"]
    dev = torch.device("cuda:0")
    fa, fb = workloads.attn_out_weights(wl, device=dev)
    codes, scales = ops.fp8_quantize_weight(fa)
    del fa
    w_ob = pipeline.quantize_stack([fb], (0, wl.H), dev)
    del fb
    xw = workloads.warmup_batch(wl)["x"].to(dev, torch.bfloat16)
    gs_o = ops.global_scale(ops.fp8_weight_gemm(xw, codes, scales).reshape(1, -1))
    x = workloads.batch(wl)["x"].to(dev, torch.bfloat16)
    T, H, D, R = wl.T, wl.H, wl.n_qb, wl.o_lora
    ms, p10, p90 = time_scrubbed(lambda: pipeline.attention_output(x, codes, scales, w_ob, gs_o), steps, warmup)
    flops = 2.0 * T * (D * R + R * H)
    bytes_ = T * D * 2 + R * D * (1 + 4.0 / (128 * 128)) + H * R * NVFP4_BYTES_PER_ELEM + T * R * 2 + T * H * 2
    line = side_line("attention output: T=%d, %d -(FP8 wo_a)-> %d -(NVFP4 wo_b)-> %d" % (T, D, R, H), ms, p10, p90,
                     flops, bytes_)
    ams, ap10, ap90 = time_scrubbed(lambda: ops.fp8_weight_gemm(x, codes, scales), steps, warmup)
    line["wo_a_alone"] = side_line("wo_a: %d x %d x %d, bf16 x E4M3 (128x128 block scales)" % (T, R, D), ams, ap10,
                                   ap90, 2.0 * T * D * R, T * D * 2 + R * D + T * R * 2)
    del x, codes, scales, w_ob
    torch.cuda.empty_cache()
    return line


def persistent_line(res):
    f = res.get("persistent")
    if f is None:
        return None
    return {"expert_mlp": "one persistent launch (nvfp4_moe_expert_mlp)", "value": round(f["tokens_per_s"], 1),
            "unit": "tokens/s", "ms_per_step": round(f["ms"], 4), "expert_mlp_ms": round(f["mlp_ms"], 4),
            "layer_frac_hbm": round(res["layer_bytes"] / (f["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "ms_per_step_pct": {k: round(v, 4) for k, v in f["step_pct"].items()}}


def other_path_line(res):
    f = res.get("other")
    if f is None:
        return None
    return {"silu_requant": SILU_PATHS[f["fused"]], "value": round(f["tokens_per_s"], 1), "unit": "tokens/s",
            "ms_per_step": round(f["ms"], 4), "gemm_l1_ms": round(f["l1_ms"], 4)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode", choices=["decode", "prefill"])
    ap.add_argument("--no-prefill", action="store_true", help="skip the secondary prefill measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tokens", type=int, default=0,
                    help="tokens per step of the timed layer instead of the workload's own (the secondary "
                         "prefill and side measurements are then skipped)")
    ap.add_argument("--cpu-experts", type=int, default=24)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a device-to-device copy of this many MiB (x3); used to calibrate the "
                         "HBM byte counters of rocprofv3 against a transfer of known size")
    args = ap.parse_args()
    if args.copy_probe_mib:
        import torch
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 3}))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)
    print("[bench] measured ceilings (HBM read probe, f16 MFMA loop)", file=sys.stderr, flush=True)
    ceilings = measure_ceilings()
    main_res = run_gpu(args.workload, args.steps, args.warmup, args.tokens or None)
    if args.tokens:
        args.no_prefill = True
    bound = "hbm" if args.workload == "decode" else "mfma"
    wl = main_res["wl"]
    line = {
        "metric": METRIC,
        "value": round(main_res["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "%s MoE layer: T=%d, hidden %d, intermediate %d, %d experts, top-%d%s" % (
            wl.name, wl.T, wl.H, wl.I, wl.E, wl.k, ", Zipf(1.1) expert popularity" if wl.zipf else ""),
            "tokens": wl.T, "experts_touched": main_res["n_touched"],
            "weights": "NVFP4 (E2M1 codes, E4M3 scale per 16, FP32 global scale per projection)"},
        "tflops": round(main_res["tflops"], 2),
        "ms_per_step_pct": {k: round(v, 4) for k, v in main_res["step_pct"].items()},
        "per_op_ms": {k: round(v, 4) for k, v in main_res["per_op_ms"].items()},
        "dynamic_activation_scales": {"value": round(main_res["dynamic"]["tokens_per_s"], 1), "unit": "tokens/s",
                                      "ms_per_step": round(main_res["dynamic"]["ms"], 4),
                                      "gs_h": DYN_PATHS[main_res["dynamic"]["fused"]]},
        "silu_requant": SILU_PATHS[main_res["fused"]],
        "other_silu_requant_path": other_path_line(main_res),
        "persistent_expert_mlp": persistent_line(main_res),
        "roofline": roofline(main_res, bound, ceilings),
        "layer_roofline": layer_roofline(main_res, bound, ceilings),
        "measured_ceilings": ceilings,
        "block_scale_saturation": main_res["saturation"],
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(main_res, args.cpu_experts)
    del main_res
    if args.workload == "decode" and not args.no_prefill:
        torch.cuda.empty_cache()
        pre = run_gpu("prefill", max(3, args.steps // 4), max(1, args.warmup // 2))
        line["prefill"] = {"value": round(pre["tokens_per_s"], 1), "unit": "tokens/s",
                           "ms_per_step": round(pre["ms"], 4), "tflops": round(pre["tflops"], 2),
                           "ms_per_step_pct": {k: round(v, 4) for k, v in pre["step_pct"].items()},
                           "dynamic_activation_scales": {"value": round(pre["dynamic"]["tokens_per_s"], 1),
                                                         "unit": "tokens/s",
                                                         "ms_per_step": round(pre["dynamic"]["ms"], 4),
                                                         "gs_h": DYN_PATHS[pre["dynamic"]["fused"]]},
                           "silu_requant": SILU_PATHS[pre["fused"]],
                           "other_silu_requant_path": other_path_line(pre),
                           "experts_touched": pre["n_touched"],
                           "per_op_ms": {k: round(v, 4) for k, v in pre["per_op_ms"].items()},
                           "roofline": roofline(pre, "mfma", ceilings),
                           "layer_roofline": layer_roofline(pre, "mfma", ceilings),
                           "block_scale_saturation": pre["saturation"]}
    if args.workload == "decode" and not args.no_prefill:
        print("[bench] shared expert and MLA projections", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        line["shared_expert"] = run_shared(args.steps, args.warmup)
        torch.cuda.empty_cache()
        line["mla_projections"] = run_mla(args.steps, args.warmup)
        torch.cuda.empty_cache()
        line["attention_output"] = run_attn_out(args.steps, args.warmup)
        torch.cuda.empty_cache()
        print("[bench] decode layer with the shared expert folded in", file=sys.stderr, flush=True)
        line["decode_with_shared_expert"] = run_decode_shared(args.steps, args.warmup)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
