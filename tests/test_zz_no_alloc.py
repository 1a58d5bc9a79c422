"""The no-allocation entry point nvfp4_global_scale_noalloc against the
workspace entry point nvfp4_global_scale, called through the C ABI: two
calls in a row on the library's per-device scratch, the second with a
smaller input, each bit-exact with the workspace call (and with the
oracle's amax / 2688)."""
import ctypes

import numpy as np
import pytest
import torch

from _helpers import dev, log, to_np
from block_scaled_fp4_03_amd import lib
from oracle import quant

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _with_workspace(x, dtype):
    L = lib.load()
    batch, n = x.shape
    out = torch.empty(batch, dtype=torch.float32, device=x.device)
    ws_bytes = L.nvfp4_global_scale_workspace_size(batch, n)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=x.device)
    lib.call("nvfp4_global_scale", _p(x), dtype, batch, n, x.stride(0), _p(out), _p(ws), ws.numel(), _stream())
    return out


def _noalloc(x, dtype, out):
    batch, n = x.shape
    lib.call("nvfp4_global_scale_noalloc", _p(x), dtype, batch, n, x.stride(0), _p(out), _stream())
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_global_scale_matches_workspace_entry_point(dtype):
    d = dev()
    tdt, cdt = (torch.bfloat16, lib.DTYPE_BF16) if dtype == "bf16" else (torch.float32, lib.DTYPE_F32)
    rng = np.random.default_rng(7)
    # first call: the largest scratch the limit allows (64 slices x 1024
    # partial maxima = 256 KiB), slices with different ranges
    n1 = 16384 * 1024 if dtype == "bf16" else 16384 * 256
    b1 = 64 if dtype == "bf16" else 16
    x1 = torch.randn(b1, n1, generator=torch.Generator(device=d).manual_seed(1), device=d).to(tdt)
    x1 *= torch.linspace(0.01, 30.0, b1, device=d).to(tdt)[:, None]
    # second call: fewer, shorter slices (a smaller part of the scratch,
    # whose older contents must not leak in)
    x2 = torch.from_numpy((rng.standard_normal((5, 4096)) * 0.5).astype(np.float32)).to(d).to(tdt)
    for x in (x1, x2):
        log("noalloc global scale", dtype, tuple(x.shape))
        want = _with_workspace(x, cdt)
        out = torch.full((x.shape[0],), -1.0, dtype=torch.float32, device=d)
        got = _noalloc(x, cdt, out)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(got).view(np.uint32), to_np(want).view(np.uint32))
        rows = sorted({0, 1, x.shape[0] - 1})         # and the oracle's amax / 2688 on a few slices
        xn = to_np(x[rows].float())
        ref = np.array([quant.global_scale(quant.amax(r)) for r in xn], np.float32)
        assert np.array_equal(to_np(got)[rows].view(np.uint32), ref.view(np.uint32))
    # over the limit: rejected before any launch, output untouched
    big = torch.empty(65, 16, dtype=tdt, device=d)
    out = torch.full((65,), -1.0, dtype=torch.float32, device=d)
    L = lib.load()
    assert L.nvfp4_global_scale_noalloc(_p(big), cdt, 65, 16384 * 1024, 16384 * 1024, _p(out), _stream()) == \
        lib.ESHAPE
    torch.cuda.synchronize()
    assert (to_np(out) == -1.0).all()
