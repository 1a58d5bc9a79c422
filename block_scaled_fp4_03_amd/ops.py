"""Thin torch binding over the C ABI: argument marshalling only.

Every function takes CUDA (HIP) tensors, allocates its outputs with torch
(device memory is all torch is used for here), and enqueues the library's
kernels on torch's current stream.  All arithmetic happens in the HIP
kernels; a missing library or a non-GPU tensor raises.
"""
import ctypes

import torch

from . import lib as _lib

_DT = {torch.float32: _lib.DTYPE_F32, torch.bfloat16: _lib.DTYPE_BF16}


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _check_dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("nvfp4moe ops take GPU tensors only")


def _dtype(t):
    if t.dtype not in _DT:
        raise ValueError("unsupported dtype %s" % t.dtype)
    return _DT[t.dtype]


def _dq_out(dq, rows, cols, device):
    if dq is True:
        return torch.empty(rows, cols, dtype=torch.float16, device=device)
    if dq is not None and (dq.dtype != torch.float16 or tuple(dq.shape) != (rows, cols)
                           or not dq.is_contiguous()):
        raise ValueError("dq must be a contiguous float16 [%d, %d] tensor" % (rows, cols))
    return dq


def quantize(x, gs, codes=None, scales=None, dq=None):
    """x [rows, cols] f32/bf16 (row pitch x.stride(0)), gs: 1-element f32
    tensor.  Returns (codes uint8 [rows, cols/2], scales uint8 [rows, cols/16]).
    With dq (True, or a float16 [rows, cols] tensor to fill) it also writes
    the dequantised values without the global scale and returns
    (codes, scales, dq)."""
    _check_dev(x, gs, None if dq is True else dq)
    rows, cols = x.shape
    if x.stride(1) != 1:
        raise ValueError("x must have unit column stride")
    if codes is None:
        codes = torch.empty(rows, cols // 2, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(rows, cols // 16, dtype=torch.uint8, device=x.device)
    want_dq = dq is not None
    dq = _dq_out(dq, rows, cols, x.device)
    _lib.call("nvfp4_quantize", _p(x), _dtype(x), rows, cols, x.stride(0), _p(gs), _p(codes),
              _p(scales), _p(dq), _stream())
    return (codes, scales, dq) if want_dq else (codes, scales)


def global_scale(x, out=None):
    """Per-slice global scales amax/2688 of x [batch, n] (or a 1-D x)."""
    _check_dev(x)
    x2 = x.reshape(1, -1) if x.dim() == 1 else x
    if x2.stride(1) != 1:
        raise ValueError("x must have unit inner stride")
    batch, n = x2.shape
    if out is None:
        out = torch.empty(batch, dtype=torch.float32, device=x.device)
    lib = _lib.load()
    ws_bytes = lib.nvfp4_global_scale_workspace_size(batch, n)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=x.device)
    _lib.call("nvfp4_global_scale", _p(x2), _dtype(x2), batch, n, x2.stride(0), _p(out), _p(ws),
              ws.numel(), _stream())
    return out


def global_scale_noalloc(x, out):
    """global_scale into a caller-given out [batch] float32, through the entry
    point that allocates nothing (its partial maxima use the library's
    per-device scratch); no torch allocation either."""
    _check_dev(x, out)
    x2 = x.reshape(1, -1) if x.dim() == 1 else x
    if x2.stride(1) != 1:
        raise ValueError("x must have unit inner stride")
    batch, n = x2.shape
    if out.dtype != torch.float32 or out.numel() < batch or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor of at least %d elements" % batch)
    _lib.call("nvfp4_global_scale_noalloc", _p(x2), _dtype(x2), batch, n, x2.stride(0), _p(out), _stream())
    return out


def route_permute(logits, k, n_shared=0):
    """logits [T, E] f32 -> (ids [T,kk] i32, w [T,kk] f32, offsets [E+n_shared+1] i32,
    sorted_token_ids [T*kk] i32, inv [T,kk] i32) with kk = k + n_shared: the
    k routed slots, then n_shared always-on shared experts E, E+1, ... with
    weight 1 (moe_route_permute_shared; n_shared = 0 is moe_route_permute)."""
    _check_dev(logits)
    if logits.dtype != torch.float32 or not logits.is_contiguous():
        raise ValueError("logits must be contiguous float32")
    T, E = logits.shape
    kk = k + n_shared
    dev = logits.device
    ids = torch.empty(T, kk, dtype=torch.int32, device=dev)
    w = torch.empty(T, kk, dtype=torch.float32, device=dev)
    off = torch.empty(E + n_shared + 1, dtype=torch.int32, device=dev)
    sorted_ids = torch.empty(T * kk, dtype=torch.int32, device=dev)
    inv = torch.empty(T, kk, dtype=torch.int32, device=dev)
    if n_shared:
        _lib.call("moe_route_permute_shared", _p(logits), T, E, k, n_shared, _p(ids), _p(w), _p(off),
                  _p(sorted_ids), _p(inv), _stream())
    else:
        _lib.call("moe_route_permute", _p(logits), T, E, k, _p(ids), _p(w), _p(off), _p(sorted_ids),
                  _p(inv), _stream())
    return ids, w, off, sorted_ids, inv


def gemm_reads_dq(G, M, K, a_rows, tiled):
    """Whether grouped_gemm with these sizes reads the float16 form of A."""
    return bool(_lib.load().nvfp4_grouped_gemm_reads_dq(G, M, K, a_rows,
                                                         _lib.LAYOUT_TILED if tiled else _lib.LAYOUT_ROWS))


def gemm_workspace_size(G, M, N, K, tiled):
    """Bytes of split-K workspace grouped_gemm uses for these sizes (0: none)."""
    return _lib.load().nvfp4_grouped_gemm_workspace_size(G, M, N, K,
                                                          _lib.LAYOUT_TILED if tiled else _lib.LAYOUT_ROWS)


def prepared_weight_bytes(G, N, K):
    return _lib.load().nvfp4_prepared_weight_bytes(G, N, K)


def prepare_weights(w_codes, w_scales, out=None):
    """Row-major NVFP4 weights [G, N, K/2] + [G, N, K/16] -> the tiled buffer
    (uint8, 1-D) that grouped_gemm streams (see nvfp4_prepare_weights)."""
    _check_dev(w_codes, w_scales)
    G, N, K2 = w_codes.shape
    K = 2 * K2
    if out is None:
        out = torch.empty(prepared_weight_bytes(G, N, K), dtype=torch.uint8, device=w_codes.device)
    _lib.call("nvfp4_prepare_weights", _p(w_codes), _p(w_scales), G, N, K, _p(out), _stream())
    return out


def grouped_gemm(a_codes, a_scales, a_gs, w_codes, w_scales, w_gs, n_seg, group_offsets, M,
                 a_row_index=None, out_dtype=torch.float32, out=None, w_tiled=None, a_dq=None, workspace=None):
    """out [M, N] = alpha * A . W^T per group (see nvfp4_grouped_gemm).
    w_codes/w_scales give G, N, K; if w_tiled (the prepare_weights buffer) is
    passed, the kernel reads the weights from it instead.  a_dq is the
    optional float16 form of A written by quantize / silu_mul_requant.
    workspace: None allocates the split-K workspace the library asks for
    (nvfp4_grouped_gemm_workspace_size), False runs without one, or a uint8
    tensor to use."""
    _check_dev(a_codes, a_scales, a_gs, w_gs, group_offsets, a_row_index, w_tiled, a_dq)
    G, N, K2 = w_codes.shape
    K = 2 * K2
    if out is None:
        out = torch.empty(M, N, dtype=out_dtype, device=a_codes.device)
    seg = (ctypes.c_int32 * len(n_seg))(*[int(v) for v in n_seg])
    if w_tiled is not None:
        wc, ws, layout = w_tiled, None, _lib.LAYOUT_TILED
    else:
        _check_dev(w_codes, w_scales)
        wc, ws, layout = w_codes, w_scales, _lib.LAYOUT_ROWS
    if a_dq is not None and (a_dq.dtype != torch.float16 or tuple(a_dq.shape) != (a_codes.shape[0], K)
                             or not a_dq.is_contiguous()):
        raise ValueError("a_dq must be a contiguous float16 [a_rows, K] tensor")
    ws_bytes = _lib.load().nvfp4_grouped_gemm_workspace_size(G, M, N, K, layout) if (workspace is None and M > 0) \
        else (0 if workspace is None or workspace is False else workspace.numel())
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=out.device)
    wsp = workspace if workspace is not None and workspace is not False else None
    _lib.call("nvfp4_grouped_gemm", _p(a_codes), _p(a_scales), _p(a_gs), a_codes.shape[0],
              _p(a_row_index), _p(a_dq), _p(wc), _p(ws), layout, _p(w_gs), seg, len(n_seg) - 1,
              _p(group_offsets), G, M, N, K, _p(out), _dtype(out), out.stride(0), _p(wsp),
              ws_bytes if wsp is not None else 0, _stream())
    return out


def grouped_gemm_silu_requant(a_codes, a_scales, a_gs, w_tiled, w_gs, group_offsets, M, I, K, gs_h,
                              a_row_index=None, a_dq=None, dq=None, codes=None, scales=None, workspace=None):
    """First GEMM of the expert MLP with SiLU(gate)*up re-quantised in its
    epilogue: the same codes and scales (and f16 copy with dq) as
    silu_mul_requant over grouped_gemm's float32 [M, 2I] output, without
    that output.  w_tiled: prepare_weights buffer of the stacked [G, 2I, K]
    weights; w_gs [G, 2].  workspace as for grouped_gemm (None allocates the
    split-K workspace the library asks for, False runs without one)."""
    _check_dev(a_codes, a_scales, a_gs, w_tiled, w_gs, group_offsets, gs_h, a_row_index, a_dq,
               None if dq is True else dq)
    G = w_gs.shape[0]
    dev = a_codes.device
    if codes is None:
        codes = torch.empty(M, I // 2, dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(M, I // 16, dtype=torch.uint8, device=dev)
    want_dq = dq is not None
    dq = _dq_out(dq, M, I, dev)
    ws_bytes = _lib.load().nvfp4_grouped_gemm_workspace_size(G, M, 2 * I, K, _lib.LAYOUT_TILED) \
        if (workspace is None and M > 0) else (0 if workspace is None or workspace is False else workspace.numel())
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    wsp = workspace if workspace is not None and workspace is not False else None
    _lib.call("nvfp4_grouped_gemm_silu_requant", _p(a_codes), _p(a_scales), _p(a_gs), a_codes.shape[0],
              _p(a_row_index), _p(a_dq), _p(w_tiled), _p(w_gs), _p(group_offsets), G, M, I, K, _p(gs_h),
              _p(codes), _p(scales), _p(dq), _p(wsp), ws_bytes if wsp is not None else 0, _stream())
    return (codes, scales, dq) if want_dq else (codes, scales)


def grouped_gemm_silu_f32(a_codes, a_scales, a_gs, w_tiled, w_gs, group_offsets, M, I, K, a_row_index=None,
                          a_dq=None, h=None, partials=None):
    """First GEMM of the expert MLP with h = SiLU(gate)*up written in float32
    (nvfp4_grouped_gemm_silu_f32): returns (h [M, I] float32, partial maxima
    of |h| [n] float32, whose maximum is max |h|)."""
    _check_dev(a_codes, a_scales, a_gs, w_tiled, w_gs, group_offsets, a_row_index, a_dq, h, partials)
    G = w_gs.shape[0]
    dev = a_codes.device
    if h is None:
        h = torch.empty(M, I, dtype=torch.float32, device=dev)
    elif h.dtype != torch.float32 or tuple(h.shape) != (M, I) or not h.is_contiguous():
        raise ValueError("h must be a contiguous float32 [%d, %d] tensor" % (M, I))
    if partials is not None and (partials.dtype != torch.float32 or not partials.is_contiguous()):
        raise ValueError("partials must be a contiguous float32 tensor")
    n = _lib.load().nvfp4_grouped_gemm_silu_f32_partials(G, M, I) if M > 0 else 8
    if partials is None:
        partials = torch.empty(max(n, 8), dtype=torch.float32, device=dev)
    _lib.call("nvfp4_grouped_gemm_silu_f32", _p(a_codes), _p(a_scales), _p(a_gs), a_codes.shape[0],
              _p(a_row_index), _p(a_dq), _p(w_tiled), _p(w_gs), _p(group_offsets), G, M, I, K, _p(h),
              _p(partials), partials.numel(), _stream())
    return h, partials


def moe_expert_mlp(x_codes, x_scales, x_gs, sorted_ids, offsets, w1_tiled, w1_gs, w2_tiled, w2_gs, R, H, I, gs_h,
                   workspace=None):
    """The experts' MLP in one persistent launch (nvfp4_moe_expert_mlp):
    returns (h_codes [R, I/2], h_scales [R, I/16], y bf16 [R, H]).  The
    workspace (the tile queue and per-slot counters) is allocated here
    unless given."""
    _check_dev(x_codes, x_scales, x_gs, sorted_ids, offsets, w1_tiled, w1_gs, w2_tiled, w2_gs, gs_h, workspace)
    G = w1_gs.shape[0]
    dev = x_codes.device
    hc = torch.empty(R, I // 2, dtype=torch.uint8, device=dev)
    hs = torch.empty(R, I // 16, dtype=torch.uint8, device=dev)
    y = torch.empty(R, H, dtype=torch.bfloat16, device=dev)
    need = _lib.load().nvfp4_moe_expert_mlp_workspace_size(G, R)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _lib.call("nvfp4_moe_expert_mlp", _p(x_codes), _p(x_scales), _p(x_gs), x_codes.shape[0], _p(sorted_ids),
              _p(offsets), G, R, _p(w1_tiled), _p(w1_gs), _p(w2_tiled), _p(w2_gs), H, I, _p(gs_h), _p(hc), _p(hs),
              _p(y), _p(workspace), workspace.numel() * workspace.element_size(), _stream())
    return hc, hs, y


def silu_mul_requant(gate_up, gs_h, codes=None, scales=None, dq=None):
    """gate_up [M, 2I] f32/bf16 -> NVFP4 h (codes [M, I/2], scales [M, I/16]);
    dq as in quantize."""
    _check_dev(gate_up, gs_h, None if dq is True else dq)
    M, I2 = gate_up.shape
    I = I2 // 2
    if codes is None:
        codes = torch.empty(M, I // 2, dtype=torch.uint8, device=gate_up.device)
    if scales is None:
        scales = torch.empty(M, I // 16, dtype=torch.uint8, device=gate_up.device)
    want_dq = dq is not None
    dq = _dq_out(dq, M, I, gate_up.device)
    _lib.call("silu_mul_requant", _p(gate_up), _dtype(gate_up), M, I, gate_up.stride(0), _p(gs_h),
              _p(codes), _p(scales), _p(dq), _stream())
    return (codes, scales, dq) if want_dq else (codes, scales)


def silu_mul_global_scale(gate_up, out=None):
    """Global scale amax(SiLU(gate)*up)/2688 of gate_up [M, 2I]."""
    _check_dev(gate_up)
    M, I2 = gate_up.shape
    I = I2 // 2
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=gate_up.device)
    lib = _lib.load()
    ws_bytes = lib.silu_mul_global_scale_workspace_size(M, I)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=gate_up.device)
    _lib.call("silu_mul_global_scale", _p(gate_up), _dtype(gate_up), M, I, gate_up.stride(0), _p(out),
              _p(ws), ws.numel(), _stream())
    return out


def combine(y, inv, w, out=None, residual=None):
    """y [T*k, H] f32/bf16, inv [T, k], w [T, k] -> out [T, H] bf16; with
    residual (bf16 [T, H], contiguous) it is added before the rounding."""
    _check_dev(y, inv, w, residual)
    T, k = inv.shape
    H = y.shape[1]
    if residual is not None and (residual.dtype != torch.bfloat16 or tuple(residual.shape) != (T, H)
                                 or not residual.is_contiguous()):
        raise ValueError("residual must be a contiguous bfloat16 [%d, %d] tensor" % (T, H))
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=y.device)
    _lib.call("moe_combine", _p(y), _dtype(y), _p(inv), _p(w), T, k, H, _p(residual), _p(out), _stream())
    return out


def fp8_quantize_weight(w):
    """w [N, K] float32 -> (codes uint8 [N, K] E4M3, scales float32
    [ceil(N/128), K/128]): one scale per 128 x 128 block."""
    _check_dev(w)
    if w.dtype != torch.float32 or w.stride(1) != 1:
        raise ValueError("w must be float32 with unit column stride")
    N, K = w.shape
    codes = torch.empty(N, K, dtype=torch.uint8, device=w.device)
    scales = torch.empty((N + 127) // 128, K // 128, dtype=torch.float32, device=w.device)
    _lib.call("fp8_quantize_weight", _p(w), N, K, w.stride(0), _p(codes), _p(scales), _stream())
    return codes, scales


def fp8_weight_gemm(x, codes, scales, out_dtype=torch.bfloat16, out=None):
    """x [M, K] bf16 . (E4M3 weights [N, K] with 128x128 block scales)^T -> [M, N]."""
    _check_dev(x, codes, scales)
    if x.dtype != torch.bfloat16 or x.stride(1) != 1:
        raise ValueError("x must be bfloat16 with unit column stride")
    M, K = x.shape
    N = codes.shape[0]
    if out is None:
        out = torch.empty(M, N, dtype=out_dtype, device=x.device)
    _lib.call("fp8_weight_gemm", _p(x), M, K, x.stride(0), _p(codes), _p(scales), N, _p(out), _dtype(out),
              out.stride(0), _stream())
    return out


def probe_hbm_read(buf, sink):
    """Measurement probe: read all of buf (a contiguous GPU tensor) once."""
    _check_dev(buf, sink)
    _lib.call("nvfp4_probe_hbm_read", _p(buf), buf.numel() * buf.element_size() // 16 * 16, _p(sink), _stream())


def probe_mfma_f16(iters, workgroups, sink):
    """Measurement probe: workgroups * 4 * iters * 8 * 32768 f16 matrix-core
    flops on register operands.  Returns that flop count."""
    _check_dev(sink)
    _lib.call("nvfp4_probe_mfma_f16", int(iters), int(workgroups), _p(sink), _stream())
    return float(workgroups) * 4 * iters * 8 * 32768
