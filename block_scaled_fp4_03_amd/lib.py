"""ctypes loader of libnvfp4moe.so: argument and return types of every C
entry point declared in include/nvfp4moe.h.  No computation happens here."""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnvfp4moe.so")

OK, EINVAL, ESHAPE, EALIGN, EHIP = 0, 1, 2, 3, 4
DTYPE_F32, DTYPE_BF16 = 0, 1
LAYOUT_ROWS, LAYOUT_TILED = 0, 1
MAX_EXPERTS, MAX_TOPK, MAX_SEGMENTS = 1024, 16, 4
NOALLOC_SCRATCH_BYTES = 262144

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

# name -> (restype, argtypes)
SIGNATURES = {
    "nvfp4_last_error": (ctypes.c_char_p, []),
    "nvfp4_version": (_I32, []),
    "nvfp4_quantize": (_I32, [_P, _I32, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "nvfp4_global_scale_workspace_size": (_SZ, [_I64, _I64]),
    "nvfp4_global_scale": (_I32, [_P, _I32, _I64, _I64, _I64, _P, _P, _SZ, _P]),
    "nvfp4_global_scale_noalloc": (_I32, [_P, _I32, _I64, _I64, _I64, _P, _P]),
    "moe_route_permute": (_I32, [_P, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P]),
    "moe_route_permute_shared": (_I32, [_P, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P]),
    "nvfp4_grouped_gemm": (_I32, [_P, _P, _P, _I64, _P, _P, _P, _P, _I32, _P, ctypes.POINTER(_I32), _I32,
                                  _P, _I32, _I64, _I64, _I64, _P, _I32, _I64, _P, _SZ, _P]),
    "nvfp4_grouped_gemm_workspace_size": (_SZ, [_I32, _I64, _I64, _I64, _I32]),
    "nvfp4_grouped_gemm_silu_requant": (_I32, [_P, _P, _P, _I64, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I64,
                                               _P, _P, _P, _P, _P, _SZ, _P]),
    "nvfp4_grouped_gemm_silu_f32_partials": (_SZ, [_I32, _I64, _I64]),
    "nvfp4_grouped_gemm_silu_f32": (_I32, [_P, _P, _P, _I64, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I64,
                                           _P, _P, _I64, _P]),
    "nvfp4_grouped_gemm_reads_dq": (_I32, [_I32, _I64, _I64, _I64, _I32]),
    "nvfp4_moe_expert_mlp_workspace_size": (_SZ, [_I32, _I64]),
    "nvfp4_moe_expert_mlp": (_I32, [_P, _P, _P, _I64, _P, _P, _I32, _I64, _P, _P, _P, _P, _I64, _I64, _P, _P, _P,
                                    _P, _P, _SZ, _P]),
    "nvfp4_prepared_weight_bytes": (_SZ, [_I64, _I64, _I64]),
    "nvfp4_prepare_weights": (_I32, [_P, _P, _I64, _I64, _I64, _P, _P]),
    "silu_mul_requant": (_I32, [_P, _I32, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "silu_mul_global_scale_workspace_size": (_SZ, [_I64, _I64]),
    "silu_mul_global_scale": (_I32, [_P, _I32, _I64, _I64, _I64, _P, _P, _SZ, _P]),
    "fp8_quantize_weight": (_I32, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "fp8_weight_gemm": (_I32, [_P, _I64, _I64, _I64, _P, _P, _I64, _P, _I32, _I64, _P]),
    "moe_combine": (_I32, [_P, _I32, _P, _P, _I64, _I32, _I64, _P, _P, _P]),
    "nvfp4_probe_hbm_read": (_I32, [_P, _I64, _P, _P]),
    "nvfp4_probe_mfma_f16": (_I32, [_I64, _I64, _P, _P]),
}

_lib = None


class Nvfp4Error(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__("%s failed with status %d: %s" % (fn, status, msg))
        self.status = status


def load():
    """Load the library once.  A missing library is an error: there is no
    other implementation to fall back to."""
    global _lib
    if _lib is None:
        # torch first: its HIP runtime is then the one the library binds to
        # (loading the library first would bring a second runtime into the
        # process, which torch's tensors are not visible to)
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("%s is not built; run __graft_entry__.build() or "
                               "python -m block_scaled_fp4_03_amd.build" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def call(name, *args):
    """Call an entry point returning a status; raise Nvfp4Error on failure."""
    lib = load()
    st = getattr(lib, name)(*args)
    if st != OK:
        raise Nvfp4Error(name, st, lib.nvfp4_last_error().decode())
    return st
