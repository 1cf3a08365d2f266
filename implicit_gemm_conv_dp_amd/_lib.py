"""ctypes binding of libskgemm.so: the C ABI declared in include/skgemm.h,
under the same names.  Argument marshalling only -- every step of the hot
path runs in the library's HIP kernels.  There is no fallback: if the
library is missing, loading it raises.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libskgemm.so")

SKG_OK, SKG_ERR_HIP, SKG_ERR_UNSUPPORTED = 0, -1, -2
F16, BF16, F8E4M3, F32, F8E5M2 = 0, 1, 2, 3, 4
SCALE_ROWCOL, SCALE_TENSOR, SCALE_MX_E8M0 = 0, 1, 2
MODE_DP, MODE_DP_SK, MODE_PERSISTENT, MODE_SPLITK, MODE_AUTO = 0, 1, 2, 3, 4
RED_LINEAR, RED_TREE, RED_ATOMIC, RED_WORKSPACE, RED_AUTO, RED_SCATTER = 0, 1, 2, 3, 4, 5
OP_GEMM, OP_WGRAD, OP_FWD, OP_DGRAD = 0, 1, 2, 3
TILE_128x128x32, TILE_256x256x64, TILE_256x256x128, TILE_32x64x64, TILE_128x128x64, \
    TILE_256x128x64, TILE_128x128x128, TILE_64x144x32, TILE_128x64x32 = range(9)
TILE_COUNT = 9

MODES = {"dp": MODE_DP, "dp_sk": MODE_DP_SK, "persistent": MODE_PERSISTENT,
         "splitk": MODE_SPLITK, "auto": MODE_AUTO}
REDUCTIONS = {"linear": RED_LINEAR, "tree": RED_TREE, "atomic": RED_ATOMIC,
              "workspace": RED_WORKSPACE, "auto": RED_AUTO, "scatter": RED_SCATTER}
DTYPES = {"f16": F16, "bf16": BF16, "e4m3": F8E4M3, "f32": F32, "e5m2": F8E5M2}
SCALE_MODES = {"rowcol": SCALE_ROWCOL, "tensor": SCALE_TENSOR, "mx": SCALE_MX_E8M0}
SK_ORDER_AUTO, SK_ORDER_BLOCK, SK_ORDER_XCD, SK_ORDER_KMAJOR = 0, 1, 2, 3
SK_ORDERS = {"auto": SK_ORDER_AUTO, "block": SK_ORDER_BLOCK, "xcd": SK_ORDER_XCD,
             "kmajor": SK_ORDER_KMAJOR}
TILES = {"128x128x32": TILE_128x128x32, "256x256x64": TILE_256x256x64,
         "256x256x128": TILE_256x256x128, "32x64x64": TILE_32x64x64,
         "128x128x64": TILE_128x128x64, "256x128x64": TILE_256x128x64,
         "128x128x128": TILE_128x128x128, "64x144x32": TILE_64x144x32,
         "128x64x32": TILE_128x64x32}


class skg_tile_info_t(ctypes.Structure):
    _fields_ = [("tm", ctypes.c_int32), ("tn", ctypes.c_int32), ("tk", ctypes.c_int32),
                ("n_waves", ctypes.c_int32), ("gemm_dtypes", ctypes.c_int32),
                ("wgrad_dtypes", ctypes.c_int32), ("conv_dtypes", ctypes.c_int32),
                ("group_block", ctypes.c_int32)]


class skg_gemm_args_t(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("dtype_ab", ctypes.c_int32), ("dtype_c", ctypes.c_int32),
                ("A", ctypes.c_void_p), ("lda", ctypes.c_int64),
                ("B", ctypes.c_void_p), ("ldb", ctypes.c_int64),
                ("C", ctypes.c_void_p), ("ldc", ctypes.c_int64),
                ("scale_a", ctypes.c_void_p), ("scale_b", ctypes.c_void_p),
                ("tile_id", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("reduction", ctypes.c_int32), ("ctas", ctypes.c_int32),
                ("scale_mode", ctypes.c_int32), ("sk_order", ctypes.c_int32)]


class skg_wgrad_args_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n", "h", "w", "c", "k", "r", "s", "stride_h", "stride_w", "pad_h", "pad_w",
                 "groups", "dtype")] + \
               [("x", ctypes.c_void_p), ("dy", ctypes.c_void_p), ("dw", ctypes.c_void_p)] + \
               [(n, ctypes.c_int32) for n in ("tile_id", "mode", "reduction", "ctas", "sk_order")]


class skg_conv_args_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n", "h", "w", "c", "k", "r", "s", "stride_h", "stride_w", "pad_h", "pad_w",
                 "groups", "dtype", "dtype_out")] + \
               [("act", ctypes.c_void_p), ("filt", ctypes.c_void_p), ("out", ctypes.c_void_p)] + \
               [(n, ctypes.c_int32) for n in ("tile_id", "mode", "reduction", "ctas", "sk_order")]


class skg_plan_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("tm", "tn", "tk", "n_waves", "mode", "reduction")] + \
               [(n, ctypes.c_int64) for n in
                ("tiles_m", "tiles_n", "tiles", "iters_per_tile", "pool", "dp_tiles", "sk_tiles",
                 "sk_ctas", "sk_iters", "iters_per_sk_cta", "extra_iters", "grid", "max_contrib",
                 "linear_partners", "tree_rounds", "flags_bytes", "partials_bytes",
                 "workspace_bytes")] + \
               [(n, ctypes.c_int32) for n in ("requested_mode", "slices", "sk_order")] + \
               [("aux_bytes", ctypes.c_int64)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


EXPORTS = {
    "skg_last_error": (ctypes.c_char_p, []),
    "skg_tile_info": (ctypes.c_int, [ctypes.c_int32, ctypes.POINTER(skg_tile_info_t)]),
    "skg_default_pool": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.POINTER(ctypes.c_int32)]),
    "skg_device_info": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.POINTER(ctypes.c_int32),
                                       ctypes.POINTER(ctypes.c_int32)]),
    "skg_plan_gemm": (ctypes.c_int, [ctypes.POINTER(skg_gemm_args_t), ctypes.POINTER(skg_plan_t)]),
    "skg_plan_wgrad": (ctypes.c_int, [ctypes.POINTER(skg_wgrad_args_t), ctypes.POINTER(skg_plan_t)]),
    "skg_run_gemm": (ctypes.c_int, [ctypes.POINTER(skg_gemm_args_t), ctypes.c_void_p,
                                    ctypes.c_size_t, ctypes.c_void_p]),
    "skg_run_wgrad": (ctypes.c_int, [ctypes.POINTER(skg_wgrad_args_t), ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_void_p]),
    "skg_profile_events": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p]),
    "skg_gemm_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(skg_gemm_args_t),
                                                ctypes.POINTER(ctypes.c_size_t)]),
    "skg_wgrad_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(skg_wgrad_args_t),
                                                 ctypes.POINTER(ctypes.c_size_t)]),
    "skg_fixup_timeouts": (ctypes.c_int, [ctypes.POINTER(ctypes.c_uint32), ctypes.c_int32]),
    "skg_run_wgrad_static": (ctypes.c_int, [ctypes.POINTER(skg_wgrad_args_t), ctypes.c_void_p]),
    "skg_plan_fwd": (ctypes.c_int, [ctypes.POINTER(skg_conv_args_t), ctypes.POINTER(skg_plan_t)]),
    "skg_plan_dgrad": (ctypes.c_int, [ctypes.POINTER(skg_conv_args_t), ctypes.POINTER(skg_plan_t)]),
    "skg_run_fwd": (ctypes.c_int, [ctypes.POINTER(skg_conv_args_t), ctypes.c_void_p,
                                   ctypes.c_size_t, ctypes.c_void_p]),
    "skg_run_dgrad": (ctypes.c_int, [ctypes.POINTER(skg_conv_args_t), ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_void_p]),
}

# Bytes of the library's own scratch array used by skg_run_wgrad_static.
STATIC_SCRATCH_BYTES = 33 << 20

_lib = None


def load(path=None):
    """Load libskgemm.so (once).  Raises OSError when it is not built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise OSError("libskgemm.so not built (run python -m implicit_gemm_conv_dp_amd.build): "
                      + p)
    lib = ctypes.CDLL(p)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def last_error():
    return load().skg_last_error().decode()


class SkgError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("status %d: %s" % (status, msg))
        self.status = status
        self.msg = msg


def check(status):
    if status != SKG_OK:
        raise SkgError(status, last_error())
    return status


# Same names as the C entry points.
def skg_tile_info(tile_id):
    out = skg_tile_info_t()
    check(load().skg_tile_info(tile_id, ctypes.byref(out)))
    return out


def skg_default_pool(reduction, num_cus, resident_per_cu):
    out = ctypes.c_int32()
    check(load().skg_default_pool(reduction, num_cus, resident_per_cu, ctypes.byref(out)))
    return out.value


def skg_device_info(op, tile_id, dtype_ab):
    cus, per_cu = ctypes.c_int32(), ctypes.c_int32()
    check(load().skg_device_info(op, tile_id, dtype_ab, ctypes.byref(cus), ctypes.byref(per_cu)))
    return cus.value, per_cu.value


def skg_plan_gemm(args):
    out = skg_plan_t()
    check(load().skg_plan_gemm(ctypes.byref(args), ctypes.byref(out)))
    return out


def skg_plan_wgrad(args):
    out = skg_plan_t()
    check(load().skg_plan_wgrad(ctypes.byref(args), ctypes.byref(out)))
    return out


def skg_run_gemm(args, ws_ptr, ws_bytes, stream_ptr):
    return check(load().skg_run_gemm(ctypes.byref(args), ws_ptr, ws_bytes, stream_ptr))


def skg_run_wgrad(args, ws_ptr, ws_bytes, stream_ptr):
    return check(load().skg_run_wgrad(ctypes.byref(args), ws_ptr, ws_bytes, stream_ptr))


def skg_profile_events(start_ptr, stop_ptr):
    return check(load().skg_profile_events(start_ptr, stop_ptr))


def skg_gemm_workspace_bytes(args):
    out = ctypes.c_size_t()
    check(load().skg_gemm_workspace_bytes(ctypes.byref(args), ctypes.byref(out)))
    return out.value


def skg_wgrad_workspace_bytes(args):
    out = ctypes.c_size_t()
    check(load().skg_wgrad_workspace_bytes(ctypes.byref(args), ctypes.byref(out)))
    return out.value


def skg_run_wgrad_static(args, stream_ptr):
    return check(load().skg_run_wgrad_static(ctypes.byref(args), stream_ptr))


def skg_fixup_timeouts(reset=False):
    out = ctypes.c_uint32()
    check(load().skg_fixup_timeouts(ctypes.byref(out), 1 if reset else 0))
    return out.value


def skg_plan_fwd(args):
    out = skg_plan_t()
    check(load().skg_plan_fwd(ctypes.byref(args), ctypes.byref(out)))
    return out


def skg_plan_dgrad(args):
    out = skg_plan_t()
    check(load().skg_plan_dgrad(ctypes.byref(args), ctypes.byref(out)))
    return out


def skg_run_fwd(args, ws_ptr, ws_bytes, stream_ptr):
    return check(load().skg_run_fwd(ctypes.byref(args), ws_ptr, ws_bytes, stream_ptr))


def skg_run_dgrad(args, ws_ptr, ws_bytes, stream_ptr):
    return check(load().skg_run_dgrad(ctypes.byref(args), ws_ptr, ws_bytes, stream_ptr))
