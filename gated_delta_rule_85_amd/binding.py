"""Python binding of the C ABI in include/gdr.h -- argument marshalling only.

The functions named like the C entry points (``gdr_forward_chunked``,
``gdr_decode_step``, ...) take a ``GdrArgs`` structure and raw device
pointers exactly as the C functions do.  ``make_args`` fills that structure
from torch tensors (shapes, dtypes and ``data_ptr()``), and ``forward`` /
``decode_step`` allocate outputs and workspace with torch and call the
library.  Every step of the computation runs in the HIP kernels of
``libgdr.so``; if the library is missing, ``lib()`` raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# GDR_LIB selects another build of the library (the host-sanitizer build of the tests)
LIB_PATH = os.environ.get("GDR_LIB") or os.path.join(PKG, "libgdr.so")

VARIANTS = {"deltanet": 0, "gated_deltanet": 1, "kda": 2, "gdn2": 3, "kla": 4}
GDR_F32, GDR_BF16 = 0, 1
GDR_FLAG_QK_L2NORM, GDR_FLAG_RAW_GATES = 1, 2
STATUS = {0: "GDR_OK", 1: "GDR_ERR_INVALID_ARGUMENT", 2: "GDR_ERR_UNSUPPORTED",
          3: "GDR_ERR_WORKSPACE", 4: "GDR_ERR_HIP"}

_vp = ctypes.c_void_p


class GdrArgs(ctypes.Structure):
    """Mirror of ``struct gdr_args``."""
    _fields_ = [
        ("variant", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64),
        ("dk", ctypes.c_int64), ("dv", ctypes.c_int64),
        ("chunk", ctypes.c_int32), ("flags", ctypes.c_int32),
        ("q", _vp), ("k", _vp), ("v", _vp),
        ("alpha", _vp), ("beta", _vp), ("erase_b", _vp), ("write_w", _vp),
        ("eps", ctypes.c_float), ("decay_scale", ctypes.c_float),
        ("state_in", _vp), ("state_out", _vp), ("o", _vp),
        ("v_route", _vp), ("delta_out", _vp),
    ]


class GdrGrads(ctypes.Structure):
    """Mirror of ``struct gdr_grads``."""
    _fields_ = [
        ("d_o", _vp), ("d_state_out", _vp),
        ("d_q", _vp), ("d_k", _vp), ("d_v", _vp), ("d_alpha", _vp), ("d_beta", _vp),
        ("d_erase_b", _vp), ("d_write_w", _vp), ("d_state_in", _vp),
    ]


class GdrError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


_lib = None


def lib(path: str | None = None):
    """Load libgdr.so (built by ``gated_delta_rule_85_amd.build``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with "
                           "`python -m gated_delta_rule_85_amd.build`")
    L = ctypes.CDLL(p)
    A = ctypes.POINTER(GdrArgs)
    L.gdr_check_args.argtypes = [A, ctypes.c_int]
    L.gdr_check_args.restype = ctypes.c_int
    L.gdr_forward_workspace_size.argtypes = [A]
    L.gdr_forward_workspace_size.restype = ctypes.c_size_t
    L.gdr_forward_chunked.argtypes = [A, _vp, ctypes.c_size_t, _vp]
    L.gdr_forward_chunked.restype = ctypes.c_int
    L.gdr_forward_chunked_noalloc.argtypes = [A, _vp]
    L.gdr_forward_chunked_noalloc.restype = ctypes.c_int
    L.gdr_decode_step.argtypes = [A, _vp]
    L.gdr_decode_step.restype = ctypes.c_int
    G = ctypes.POINTER(GdrGrads)
    L.gdr_backward_workspace_size.argtypes = [A]
    L.gdr_backward_workspace_size.restype = ctypes.c_size_t
    L.gdr_backward_chunked.argtypes = [A, G, _vp, ctypes.c_size_t, _vp]
    L.gdr_backward_chunked.restype = ctypes.c_int
    L.gdr_forward_chunked_save.argtypes = [A, _vp, ctypes.c_size_t, _vp]
    L.gdr_forward_chunked_save.restype = ctypes.c_int
    L.gdr_backward_chunked_saved.argtypes = [A, G, _vp, ctypes.c_size_t, _vp]
    L.gdr_backward_chunked_saved.restype = ctypes.c_int
    L.gdr_status_string.argtypes = [ctypes.c_int]
    L.gdr_status_string.restype = ctypes.c_char_p
    L.gdr_last_error_detail.argtypes = []
    L.gdr_last_error_detail.restype = ctypes.c_char_p
    if path is None:
        _lib = L
    return L


# ---- the C entry points, one to one ----------------------------------------------

def gdr_check_args(args: GdrArgs, for_decode: int) -> int:
    return lib().gdr_check_args(ctypes.byref(args), int(for_decode))


def gdr_forward_workspace_size(args: GdrArgs) -> int:
    return lib().gdr_forward_workspace_size(ctypes.byref(args))


def gdr_forward_chunked(args: GdrArgs, workspace: int, ws_bytes: int, stream: int) -> int:
    return lib().gdr_forward_chunked(ctypes.byref(args), workspace or None, ws_bytes,
                                     stream or None)


# GDR_NOALLOC_WORKSPACE_MAX of gdr.h: the static workspace of the allocation-free forward
NOALLOC_WORKSPACE_MAX = 256 << 20


def gdr_forward_chunked_noalloc(args: GdrArgs, stream: int) -> int:
    return lib().gdr_forward_chunked_noalloc(ctypes.byref(args), stream or None)


def gdr_decode_step(args: GdrArgs, stream: int) -> int:
    return lib().gdr_decode_step(ctypes.byref(args), stream or None)


def gdr_backward_workspace_size(args: GdrArgs) -> int:
    return lib().gdr_backward_workspace_size(ctypes.byref(args))


def gdr_backward_chunked(args: GdrArgs, grads: GdrGrads, workspace: int, ws_bytes: int,
                         stream: int) -> int:
    return lib().gdr_backward_chunked(ctypes.byref(args), ctypes.byref(grads),
                                      workspace or None, ws_bytes, stream or None)


def gdr_forward_chunked_save(args: GdrArgs, workspace: int, ws_bytes: int, stream: int) -> int:
    return lib().gdr_forward_chunked_save(ctypes.byref(args), workspace or None, ws_bytes,
                                          stream or None)


def gdr_backward_chunked_saved(args: GdrArgs, grads: GdrGrads, workspace: int, ws_bytes: int,
                               stream: int) -> int:
    return lib().gdr_backward_chunked_saved(ctypes.byref(args), ctypes.byref(grads),
                                            workspace or None, ws_bytes, stream or None)


def gdr_status_string(status: int) -> str:
    return lib().gdr_status_string(int(status)).decode()


def gdr_last_error_detail() -> str:
    return lib().gdr_last_error_detail().decode()


def check(status: int) -> None:
    if status != 0:
        raise GdrError(status, gdr_last_error_detail())


# ---- marshalling from torch tensors ----------------------------------------------

def _ptr(t):
    return None if t is None else t.data_ptr()


def make_args(variant: str, q, k, v, o, alpha=None, beta=None, erase_b=None,
              write_w=None, eps: float = 0.0, state_in=None, state_out=None,
              chunk: int = 0, flags: int = 0, decay_scale: float = 0.0,
              v_route=None, delta_out=None) -> GdrArgs:
    """Fill GdrArgs from contiguous tensors q, k [B,T,H,dk], v, o [B,T,H,dv].
    ``flags`` (GDR_FLAG_*) and ``decay_scale`` select the on-load transforms;
    ``v_route`` and ``delta_out`` ([B,T,H,dv], q's dtype) the cross-layer
    routing input and output."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("alpha", alpha),
                    ("beta", beta), ("erase_b", erase_b), ("write_w", write_w),
                    ("state_in", state_in), ("state_out", state_out),
                    ("v_route", v_route), ("delta_out", delta_out)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dtype == torch.bfloat16:
        dt = GDR_BF16
    elif q.dtype == torch.float32:
        dt = GDR_F32
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    return GdrArgs(VARIANTS[variant], dt, B, T, H, dk, dv, chunk, int(flags),
                   _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                   _ptr(erase_b), _ptr(write_w), float(eps), float(decay_scale),
                   _ptr(state_in), _ptr(state_out), _ptr(o), _ptr(v_route), _ptr(delta_out))


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def forward(variant: str, q, k, v, alpha=None, beta=None, erase_b=None,
            write_w=None, eps: float = 0.0, state_in=None, output_state: bool = True,
            o=None, state_out=None, workspace=None, stream=None, flags: int = 0,
            decay_scale: float = 0.0, v_route=None, want_delta: bool = False):
    """Chunked forward on device tensors.  Returns (o, state_out or None), and
    with ``want_delta`` also the per-token written residual [B,T,H,dv]."""
    import torch

    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    if output_state and state_out is None:
        state_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    delta = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device) if want_delta else None
    a = make_args(variant, q, k, v, o, alpha, beta, erase_b, write_w, eps,
                  state_in, state_out, flags=flags, decay_scale=decay_scale,
                  v_route=v_route, delta_out=delta)
    check(gdr_check_args(a, 0))
    need = gdr_forward_workspace_size(a)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    check(gdr_forward_chunked(a, workspace.data_ptr(), workspace.numel(),
                              _stream_handle(stream)))
    return (o, state_out, delta) if want_delta else (o, state_out)


def forward_noalloc(variant: str, q, k, v, alpha=None, beta=None, erase_b=None,
                    write_w=None, eps: float = 0.0, state_in=None, o=None, state_out=None,
                    stream=None, flags: int = 0, decay_scale: float = 0.0, v_route=None,
                    delta_out=None):
    """gdr_forward_chunked_noalloc on device tensors: the outputs (o, and
    state_out if given) must be passed in, so that nothing is allocated.
    Returns (o, state_out)."""
    a = make_args(variant, q, k, v, o, alpha, beta, erase_b, write_w, eps,
                  state_in, state_out, flags=flags, decay_scale=decay_scale,
                  v_route=v_route, delta_out=delta_out)
    check(gdr_forward_chunked_noalloc(a, _stream_handle(stream)))
    return o, state_out


def workspace_bytes(variant: str, q, k, v) -> int:
    """Workspace size gdr_forward_chunked needs for these shapes."""
    import torch
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    a = GdrArgs(VARIANTS[variant], GDR_BF16 if q.dtype == torch.bfloat16 else GDR_F32,
                B, T, H, dk, dv, 0, 0, 16, 16, 16,
                16 if variant != "deltanet" else None,
                16 if variant != "gdn2" else None,
                16 if variant == "gdn2" else None, 16 if variant == "gdn2" else None,
                1e-6 if variant == "kla" else 0.0, 0.0, None, None, 32, None, None)
    return gdr_forward_workspace_size(a)


def decode_step(variant: str, q, k, v, state, alpha=None, beta=None, erase_b=None,
                write_w=None, eps: float = 0.0, o=None, state_out=None, stream=None,
                flags: int = 0, decay_scale: float = 0.0, v_route=None, delta_out=None):
    """One decode step: q, k [B,1,H,dk], v [B,1,H,dv]; updates ``state`` in
    place unless ``state_out`` is given.  ``v_route`` / ``delta_out`` are the
    routing input and output (optional).  Returns o [B,1,H,dv]."""
    import torch

    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    a = make_args(variant, q, k, v, o, alpha, beta, erase_b, write_w, eps,
                  state, state if state_out is None else state_out, flags=flags,
                  decay_scale=decay_scale, v_route=v_route, delta_out=delta_out)
    check(gdr_decode_step(a, _stream_handle(stream)))
    return o


def forward_save(variant: str, q, k, v, alpha=None, beta=None, erase_b=None, write_w=None,
                 eps: float = 0.0, state_in=None, output_state: bool = True, workspace=None,
                 stream=None):
    """gdr_forward_chunked_save on device tensors: the forward of a training
    step.  Returns (o, state_out or None, workspace); pass the same inputs and
    that workspace to ``backward(..., saved=workspace)``."""
    import torch

    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    state_out = (torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
                 if output_state else None)
    a = make_args(variant, q, k, v, o, alpha, beta, erase_b, write_w, eps, state_in, state_out)
    need = gdr_backward_workspace_size(a)   # 0 for invalid args: the call below reports why
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    check(gdr_forward_chunked_save(a, workspace.data_ptr(), workspace.numel(),
                                   _stream_handle(stream)))
    return o, state_out, workspace


def backward(variant: str, q, k, v, alpha=None, beta=None, erase_b=None, write_w=None,
             eps: float = 0.0, state_in=None, d_o=None, d_state_out=None,
             want_state_grad: bool = True, workspace=None, stream=None, saved=None):
    """Gradient of the chunked forward on device tensors.  ``d_o`` [B,T,H,dv] (in
    q's dtype) and ``d_state_out`` [B,H,dk,dv] float32 are the upstream gradients
    (None = zero).  ``saved``: the workspace that ``forward_save`` returned for
    the same inputs (then gdr_backward_chunked_saved runs in it).  Returns a dict
    of float32 gradients keyed q, k, v, alpha, beta, erase_b, write_w, state_in
    (None where the variant takes no such input)."""
    import torch

    B, T, H, dk = q.shape
    dv = v.shape[-1]
    for name, t in (("d_o", d_o), ("d_state_out", d_state_out)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    dev = q.device
    f32 = torch.float32
    out = {
        "q": torch.empty((B, T, H, dk), dtype=f32, device=dev),
        "k": torch.empty((B, T, H, dk), dtype=f32, device=dev),
        "v": torch.empty((B, T, H, dv), dtype=f32, device=dev),
        "alpha": None if alpha is None else torch.empty(alpha.shape, dtype=f32, device=dev),
        "beta": None if beta is None else torch.empty(beta.shape, dtype=f32, device=dev),
        "erase_b": None if erase_b is None else torch.empty(erase_b.shape, dtype=f32, device=dev),
        "write_w": None if write_w is None else torch.empty(write_w.shape, dtype=f32, device=dev),
        "state_in": (torch.empty((B, H, dk, dv), dtype=f32, device=dev)
                     if want_state_grad else None),
    }
    a = make_args(variant, q, k, v, None, alpha, beta, erase_b, write_w, eps, state_in, None)
    g = GdrGrads(_ptr(d_o), _ptr(d_state_out), _ptr(out["q"]), _ptr(out["k"]), _ptr(out["v"]),
                 _ptr(out["alpha"]), _ptr(out["beta"]), _ptr(out["erase_b"]),
                 _ptr(out["write_w"]), _ptr(out["state_in"]))
    if saved is not None:
        check(gdr_backward_chunked_saved(a, g, saved.data_ptr(), saved.numel(),
                                         _stream_handle(stream)))
        return out
    need = gdr_backward_workspace_size(a)   # 0 for invalid args: the call below reports why
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    check(gdr_backward_chunked(a, g, workspace.data_ptr(), workspace.numel(),
                               _stream_handle(stream)))
    return out
