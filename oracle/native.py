"""ctypes loader for the C fp64 oracle (test infrastructure only).

``build()`` compiles ``gdr_oracle.c`` with gcc into ``liboracle.so`` next to
it; ``forward()`` marshals NumPy (or CPU torch) arrays into it.
"""
import ctypes
import os
import subprocess

import numpy as np

KIND_NONE, KIND_SCALAR, KIND_CHANNEL = 0, 1, 2
ORDER_ERASE_THEN_DECAY, ORDER_DECAY_THEN_ERASE = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def library_path():
    return _LIB


def build(force=True):
    """Compile the oracle with gcc (-O2, OpenMP, strict IEEE fp64: no fast-math)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        ci = ctypes.c_int
        lib.gdr_oracle_forward.argtypes = [i64, i64, i64, i64, i64, p, p, p, p, ci, p, ci, p, ci,
                                           ci, p, p, p, ci]
        lib.gdr_oracle_forward.restype = ci
        lib.gdr_oracle_version.restype = ci
        _lib = lib
    return _lib


def _as_f32(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # CPU torch tensor
        x = x.detach().to("cpu").float().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _kind(g, full_rank):
    """Gate kind from its shape: None -> NONE, [B,T,H] -> SCALAR, [B,T,H,D] -> CHANNEL."""
    if g is None:
        return KIND_NONE
    return KIND_CHANNEL if g.ndim == full_rank else KIND_SCALAR


def forward(q, k, v, log_alpha=None, b=None, w=None, S0=None,
            order=ORDER_ERASE_THEN_DECAY, n_threads=0):
    """fp64 recurrence. q,k [B,T,H,DK]; v [B,T,H,DV]; gates [B,T,H] or [B,T,H,D] or None;
    S0 [B,H,DK,DV] (any float dtype; upcast to fp64) or None.
    Returns (o [B,T,H,DV] float64, S_T [B,H,DK,DV] float64)."""
    lib = _load()
    q, k, v = _as_f32(q), _as_f32(k), _as_f32(v)
    log_alpha, b, w = _as_f32(log_alpha), _as_f32(b), _as_f32(w)
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == (B, T, H)
    for g, width in ((log_alpha, DK), (b, DK), (w, DV)):
        if g is not None:
            assert g.shape in ((B, T, H), (B, T, H, width)), g.shape
    if S0 is not None:
        if hasattr(S0, "detach"):
            S0 = S0.detach().to("cpu").double().numpy()
        S0 = np.ascontiguousarray(np.asarray(S0, dtype=np.float64))
        assert S0.shape == (B, H, DK, DV)
    o = np.zeros((B, T, H, DV), dtype=np.float64)
    S_T = np.zeros((B, H, DK, DV), dtype=np.float64)

    def ptr(a):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    rc = lib.gdr_oracle_forward(B, H, T, DK, DV, ptr(q), ptr(k), ptr(v),
                                ptr(log_alpha), _kind(log_alpha, 4), ptr(b), _kind(b, 4),
                                ptr(w), _kind(w, 4), int(order), ptr(S0), ptr(o), ptr(S_T),
                                int(n_threads))
    if rc != 0:
        raise ValueError("gdr_oracle_forward rejected its arguments (rc=%d)" % rc)
    return o, S_T
