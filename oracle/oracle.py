"""Parity oracle for the gated delta-rule forward pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The GPU library never calls it and it
never calls the GPU library: the two share no code.

It wraps ``gdr_oracle.c`` (plain sequential double-precision recurrences, one
function per variant) with ctypes and runs independent heads (b, h) on a
thread pool.  Inputs are the exact stored values (bf16 or fp32) upcast to
float64; results come back as float64 numpy arrays.

``frontend`` holds the optional input transforms (q/k L2 normalisation, gate
activations from pre-activations) in plain numpy float64.

Parity status: every variant is pinned by the tests in ``tests/test_oracle_*``
(exact rational brute force on short sequences, the Kaczmarz projection and
line-search properties, variant reductions, closed forms), and the front-end by
closed forms and library routines; none is unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

VARIANTS = ("deltanet", "gated_deltanet", "kda", "gdn2", "kla")
_ENTRY = {
    "deltanet": "oracle_deltanet_head",
    "gated_deltanet": "oracle_gated_deltanet_head",
    "kda": "oracle_kda_head",
    "gdn2": "oracle_gdn2_head",
    "kla": "oracle_kla_head",
}

_dp = ctypes.POINTER(ctypes.c_double)


class _Problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_long), ("T", ctypes.c_long), ("H", ctypes.c_long),
        ("dk", ctypes.c_long), ("dv", ctypes.c_long),
        ("q", _dp), ("k", _dp), ("v", _dp),
        ("alpha", _dp), ("beta", _dp), ("erase_b", _dp), ("write_w", _dp),
        ("eps", ctypes.c_double),
        ("state_in", _dp), ("state_out", _dp), ("o", _dp), ("delta", _dp),
    ]


_lib = None
_lib_lock = threading.Lock()


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", out, src]
    subprocess.run(cmd, check=True)
    return out


def load(path: str | None = None):
    """Load (building first if needed) the oracle shared library."""
    global _lib
    with _lib_lock:
        if path is not None:
            lib = ctypes.CDLL(path)
        else:
            if _lib is not None:
                return _lib
            # GDR_ORACLE_LIB selects another build of the oracle (the tests'
            # sanitizer build); otherwise the default one, rebuilt when stale.
            other = os.environ.get("GDR_ORACLE_LIB")
            if other:
                lib = ctypes.CDLL(other)
            else:
                if (not os.path.exists(_LIB)
                        or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
                    build()
                lib = ctypes.CDLL(_LIB)
        for name in _ENTRY.values():
            fn = getattr(lib, name)
            fn.argtypes = [ctypes.POINTER(_Problem), ctypes.c_long, ctypes.c_long]
            fn.restype = ctypes.c_int
        if path is None:
            _lib = lib
        return lib


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: exact upcast of bf16/fp32 values
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# Front-end options (input transforms applied before the recurrence).
QK_L2NORM = 1      # q and k divided by their L2 norm over the key dimension
RAW_GATES = 2      # gate tensors hold pre-activations
L2NORM_EPS = 1e-6  # added to the sum of squares before the square root


def softplus(x):
    """log(1 + e^x), evaluated without overflow: max(x, 0) + log1p(e^-|x|)."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x):
    """1 / (1 + e^-x), evaluated without overflow on either side."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def l2normalize(x):
    """x / sqrt(sum_i x_i^2 + L2NORM_EPS) over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + L2NORM_EPS)


def frontend(variant: str, q, k, alpha=None, beta=None, erase_b=None, write_w=None,
             flags: int = 0, decay_scale: float = 0.0):
    """The input transforms in float64, in this order, each on its own tensor:
    with QK_L2NORM, q and k become l2normalize(q), l2normalize(k); with
    RAW_GATES, alpha becomes exp(-decay_scale * softplus(alpha)) and beta
    (eta for KLA), erase_b and write_w become sigmoid of themselves.  The
    recurrence then runs on the results exactly as on stored gates."""
    q, k = _f64(q), _f64(k)
    alpha, beta, erase_b, write_w = _f64(alpha), _f64(beta), _f64(erase_b), _f64(write_w)
    if flags & QK_L2NORM:
        q, k = l2normalize(q), l2normalize(k)
    if flags & RAW_GATES:
        if alpha is not None:
            alpha = np.exp(-decay_scale * softplus(alpha))
        beta = None if beta is None else sigmoid(beta)
        erase_b = None if erase_b is None else sigmoid(erase_b)
        write_w = None if write_w is None else sigmoid(write_w)
    return q, k, alpha, beta, erase_b, write_w


def forward(variant: str, q, k, v, alpha=None, beta=None, erase_b=None,
            write_w=None, eps: float = 0.0, state_in=None, heads=None,
            threads: int | None = None, lib=None, flags: int = 0, decay_scale: float = 0.0,
            v_route=None, want_delta: bool = False):
    """Run the sequential recurrence for ``variant``.

    q, k: [B, T, H, dk]; v: [B, T, H, dv]; gates as documented in
    ``gdr_oracle.c``.  ``flags`` / ``decay_scale`` select the input transforms
    of ``frontend``.  ``v_route`` ([B, T, H, dv], optional) is a value routed in
    from another layer: the recurrence uses v + v_route as its value
    ("Linear Attention Architectures", cross-layer routing: CLVR passes the
    value target on).  ``heads`` optionally restricts the work to a list of
    (b, h) pairs; outputs of other heads are left as NaN.  Returns
    ``(o [B,T,H,dv], state_out [B,H,dk,dv])`` in float64, and with
    ``want_delta`` also the residual each token writes, delta [B,T,H,dv]
    (S_t = S~_t + k_t delta_t^T).
    """
    if variant not in _ENTRY:
        raise ValueError(f"unknown variant {variant!r}")
    if flags:
        q, k, alpha, beta, erase_b, write_w = frontend(variant, q, k, alpha, beta, erase_b,
                                                       write_w, flags, decay_scale)
    q, k, v = _f64(q), _f64(k), _f64(v)
    if v_route is not None:
        v = v + _f64(v_route)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    arrays = dict(alpha=_f64(alpha), beta=_f64(beta), erase_b=_f64(erase_b),
                  write_w=_f64(write_w), state_in=_f64(state_in))
    o = np.full((B, T, H, dv), np.nan)
    s_out = np.full((B, H, dk, dv), np.nan)
    delta = np.full((B, T, H, dv), np.nan) if want_delta else None
    prob = _Problem(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                    _ptr(arrays["alpha"]), _ptr(arrays["beta"]),
                    _ptr(arrays["erase_b"]), _ptr(arrays["write_w"]),
                    float(eps), _ptr(arrays["state_in"]), _ptr(s_out), _ptr(o), _ptr(delta))
    lib = lib if lib is not None else load()
    fn = getattr(lib, _ENTRY[variant])
    todo = list(heads) if heads is not None else [(b, h) for b in range(B) for h in range(H)]

    def run(bh):
        rc = fn(ctypes.byref(prob), bh[0], bh[1])
        if rc != 0:
            raise MemoryError("oracle allocation failed")

    n = max(1, min(threads or default_threads(), len(todo)))
    if n == 1:
        for bh in todo:
            run(bh)
    else:
        with ThreadPoolExecutor(max_workers=n) as ex:
            list(ex.map(run, todo))
    # keep the argument arrays alive until the calls are done
    del arrays
    return (o, s_out, delta) if want_delta else (o, s_out)
