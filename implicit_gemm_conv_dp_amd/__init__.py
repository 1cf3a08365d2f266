"""Stream-K GEMM and conv-wgrad engine for MI355X (gfx950).

The compute path is the HIP library ``libskgemm.so`` (C ABI in
``include/skgemm.h``); this package only marshals torch device tensors and
streams into its calls.  PyTorch provides device memory and streams.

    import implicit_gemm_conv_dp_amd as skg
    plan = skg.gemm(A, B, C, M=..., N=..., K=..., dtype_ab="bf16", dtype_c="bf16",
                    tile="256x256x64", mode="dp_sk", reduction="tree", ctas=256)

``A`` is M x K row-major, ``B`` is K x N column-major (N rows of K), ``C`` is
M x N row-major; tensors are passed as raw storage (any torch dtype), their
element type is ``dtype_ab`` / ``dtype_c``.  ``wgrad`` takes NHWC ``x`` and
``dy`` and writes the fp32 KRSC filter gradient ``dw``.
"""

from . import _lib
from ._lib import (SkgError, skg_default_pool, skg_device_info, skg_plan_gemm,  # noqa: F401
                   skg_plan_wgrad, skg_profile_events, skg_run_gemm, skg_run_wgrad,
                   skg_tile_info, skg_gemm_workspace_bytes, skg_wgrad_workspace_bytes,
                   skg_fixup_timeouts, skg_run_wgrad_static, skg_plan_fwd, skg_plan_dgrad,
                   skg_run_fwd, skg_run_dgrad, MODES, REDUCTIONS, DTYPES, TILES, SCALE_MODES,
                   SK_ORDERS)

__all__ = ["gemm", "wgrad", "fwd", "dgrad", "plan_gemm", "plan_wgrad", "plan_fwd", "plan_dgrad",
           "gemm_args", "wgrad_args", "conv_args",
           "workspace_for", "SkgError", "MODES", "REDUCTIONS", "DTYPES", "TILES", "SCALE_MODES",
           "SK_ORDERS",
           "skg_default_pool", "skg_device_info", "skg_plan_gemm", "skg_plan_wgrad",
           "skg_run_gemm", "skg_run_wgrad", "skg_tile_info", "skg_profile_events",
           "skg_gemm_workspace_bytes", "skg_wgrad_workspace_bytes", "skg_fixup_timeouts",
           "skg_run_wgrad_static", "skg_plan_fwd", "skg_plan_dgrad", "skg_run_fwd",
           "skg_run_dgrad"]


def _enum(table, v, what):
    if isinstance(v, int):
        return v
    try:
        return table[v]
    except KeyError:
        raise ValueError("unknown %s %r" % (what, v)) from None


def _ptr(t):
    return 0 if t is None else t.data_ptr()


def gemm_args(A=None, B=None, C=None, *, M, N, K, dtype_ab, dtype_c, lda=None, ldb=None,
              ldc=None, scale_a=None, scale_b=None, scale_mode="rowcol", tile, mode, reduction,
              ctas, sk_order="auto"):
    a = _lib.skg_gemm_args_t()
    a.M, a.N, a.K = M, N, K
    a.dtype_ab = _enum(DTYPES, dtype_ab, "dtype")
    a.dtype_c = _enum(DTYPES, dtype_c, "dtype")
    a.A, a.B, a.C = _ptr(A), _ptr(B), _ptr(C)
    a.lda = K if lda is None else lda
    a.ldb = K if ldb is None else ldb
    a.ldc = N if ldc is None else ldc
    a.scale_a, a.scale_b = _ptr(scale_a), _ptr(scale_b)
    a.tile_id = _enum(TILES, tile, "tile")
    a.mode = _enum(MODES, mode, "mode")
    a.reduction = _enum(REDUCTIONS, reduction, "reduction")
    a.ctas = ctas
    a.scale_mode = _enum(SCALE_MODES, scale_mode, "scale mode")
    a.sk_order = _enum(SK_ORDERS, sk_order, "stream-K order")
    return a


def wgrad_args(x=None, dy=None, dw=None, *, n, h, w, c, k, r, s, stride=(1, 1), pad=(0, 0),
               groups=1, dtype, tile, mode, reduction, ctas, sk_order="auto"):
    a = _lib.skg_wgrad_args_t()
    a.n, a.h, a.w, a.c, a.k, a.r, a.s = n, h, w, c, k, r, s
    a.stride_h, a.stride_w = stride
    a.pad_h, a.pad_w = pad
    a.groups = groups
    a.dtype = _enum(DTYPES, dtype, "dtype")
    a.x, a.dy, a.dw = _ptr(x), _ptr(dy), _ptr(dw)
    a.tile_id = _enum(TILES, tile, "tile")
    a.mode = _enum(MODES, mode, "mode")
    a.reduction = _enum(REDUCTIONS, reduction, "reduction")
    a.ctas = ctas
    a.sk_order = _enum(SK_ORDERS, sk_order, "stream-K order")
    return a


def conv_args(act=None, filt=None, out=None, *, n, h, w, c, k, r, s, stride=(1, 1), pad=(0, 0),
              groups=1, dtype, dtype_out, tile, mode, reduction, ctas, sk_order="auto"):
    """Arguments of a forward convolution (act = X, out = Y) or of its input
    gradient (act = dY, out = dX); filt is the KRSC filter W either way."""
    a = _lib.skg_conv_args_t()
    a.n, a.h, a.w, a.c, a.k, a.r, a.s = n, h, w, c, k, r, s
    a.stride_h, a.stride_w = stride
    a.pad_h, a.pad_w = pad
    a.groups = groups
    a.dtype = _enum(DTYPES, dtype, "dtype")
    a.dtype_out = _enum(DTYPES, dtype_out, "dtype")
    a.act, a.filt, a.out = _ptr(act), _ptr(filt), _ptr(out)
    a.tile_id = _enum(TILES, tile, "tile")
    a.mode = _enum(MODES, mode, "mode")
    a.reduction = _enum(REDUCTIONS, reduction, "reduction")
    a.ctas = ctas
    a.sk_order = _enum(SK_ORDERS, sk_order, "stream-K order")
    return a


def plan_gemm(**kw):
    return skg_plan_gemm(gemm_args(**kw)).as_dict()


def plan_wgrad(**kw):
    return skg_plan_wgrad(wgrad_args(**kw)).as_dict()


def plan_fwd(**kw):
    return skg_plan_fwd(conv_args(**kw)).as_dict()


def plan_dgrad(**kw):
    return skg_plan_dgrad(conv_args(**kw)).as_dict()


def workspace_for(plan, device):
    """A device buffer large enough for ``plan`` (torch owns the memory)."""
    import torch
    return torch.empty(max(int(plan["workspace_bytes"]), 1), dtype=torch.uint8, device=device)


def _launch_stream(stream):
    import torch
    return torch.cuda.current_stream() if stream is None else stream


def _run(run, args, plan, device, workspace, stream):
    """One run call.  A workspace the call allocates itself is handed to the
    caching allocator as used by the launch stream (record_stream), so its
    memory is not given to another allocation before the kernel is done
    with it, whichever stream the caller passed."""
    s = _launch_stream(stream)
    ws = workspace
    if ws is None:
        ws = workspace_for(plan, device)
        ws.record_stream(s)
    run(args, ws.data_ptr(), ws.numel() * ws.element_size(), s.cuda_stream)


def gemm(A, B, C, scale_a=None, scale_b=None, workspace=None, stream=None, **kw):
    """Enqueue C = epilogue(A @ B) on ``stream`` (default: torch's current
    stream).  Returns the plan (a dict)."""
    args = gemm_args(A, B, C, scale_a=scale_a, scale_b=scale_b, **kw)
    plan = skg_plan_gemm(args).as_dict()
    _run(skg_run_gemm, args, plan, C.device, workspace, stream)
    return plan


def wgrad(x, dy, dw, workspace=None, stream=None, **kw):
    """Enqueue dw = wgrad(x, dy) on ``stream``.  Returns the plan (a dict)."""
    args = wgrad_args(x, dy, dw, **kw)
    plan = skg_plan_wgrad(args).as_dict()
    _run(skg_run_wgrad, args, plan, dw.device, workspace, stream)
    return plan


def fwd(x, filt, y, workspace=None, stream=None, **kw):
    """Enqueue the forward convolution y = conv(x, filt) on ``stream``.
    Returns the plan (a dict)."""
    args = conv_args(x, filt, y, **kw)
    plan = skg_plan_fwd(args).as_dict()
    _run(skg_run_fwd, args, plan, y.device, workspace, stream)
    return plan


def dgrad(dy, filt, dx, workspace=None, stream=None, **kw):
    """Enqueue the input gradient dx = dgrad(dy, filt) on ``stream``.
    Returns the plan (a dict)."""
    args = conv_args(dy, filt, dx, **kw)
    plan = skg_plan_dgrad(args).as_dict()
    _run(skg_run_dgrad, args, plan, dx.device, workspace, stream)
    return plan
