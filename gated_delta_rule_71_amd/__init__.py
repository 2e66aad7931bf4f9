"""Gated delta-rule linear attention on AMD Instinct MI355X (gfx950).

Thin Python binding over libgdr.so (include/gdr.h).  PyTorch only provides device memory and
the current stream; every step of the computation runs in the library's HIP kernels.  If the
library is missing, every call raises: there is no CPU or eager fallback.

    o, S_T = chunk_fwd(q, k, v, log_alpha, b, w, S0)      # prefill over T tokens
    o = decode_step(q, k, v, log_alpha, b, w, S)           # one token, S updated in place
    grads = chunk_bwd(q, k, v, log_alpha, b, w, S0, do, dS_T)  # gradients of the prefill

Layouts: q, k [B,T,Hqk,dk]; v [B,T,H,dv] (H a multiple of Hqk: grouped key / value heads, value
head h reading q / k head h // (H // Hqk)); gates [B,T,H] (one value per token and head) or
[B,T,H,dk] / [B,T,H,dv] (per channel) or None; states [B,H,dk,dv] float32.  q, k, v and the
gates share one dtype, bfloat16 or float32.  The recurrence:

    S_t = Diag(exp(log_alpha_t)) (I - k_t^T (b_t . k_t)) S_{t-1} + k_t^T (w_t . v_t)
    o_t = q_t S_t

("Recurrent Memory: Write, Erase, Decay, Read", section 05, with the Gated DeltaNet-2
channel-wise erase and write gates).  ``order="decay_then_erase"`` applies the decay before the
erase instead.
"""
from . import _native
from ._native import GdrError, abi_version, make_problem, status_string

__all__ = ["chunk_fwd", "chunk_bwd", "decode_step", "abi_version", "status_string", "GdrError", "make_problem"]

_ORDERS = {"erase_then_decay": _native.ERASE_THEN_DECAY, "decay_then_erase": _native.DECAY_THEN_ERASE}


def _torch():
    import torch
    return torch


def _io_dtype(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return _native.GDR_BF16
    if t.dtype == torch.float32:
        return _native.GDR_FP32
    raise TypeError("q/k/v must be bfloat16 or float32, got %s" % t.dtype)


def _gate_kind(g, B, T, H, width, name, dtype, device):
    if g is None:
        return _native.GATE_NONE
    if g.dtype != dtype or g.device != device:
        raise TypeError("%s must be %s on %s" % (name, dtype, device))
    if tuple(g.shape) == (B, T, H):
        return _native.GATE_SCALAR
    if tuple(g.shape) == (B, T, H, width):
        return _native.GATE_CHANNEL
    raise ValueError("%s has shape %s; expected %s or %s" % (name, tuple(g.shape), (B, T, H),
                                                          (B, T, H, width)))


def _ptr(t):
    return 0 if t is None else t.data_ptr()


def _check_contig(**tensors):
    for name, t in tensors.items():
        if t is not None and not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)


def _check_buffer(name, t, shape, dtype, device):
    """A caller-supplied tensor the kernels read or write through a raw pointer: it must have
    exactly this shape, dtype and device and be contiguous, or the kernels would touch memory
    outside it (or a host address)."""
    if t is None:
        return
    if t.device != device:
        raise ValueError("%s is on %s; expected %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s; expected %s" % (name, t.dtype, dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s; expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _check_workspace(workspace, need, device):
    if workspace is None:
        return
    if workspace.device != device:
        raise ValueError("workspace is on %s; expected %s" % (workspace.device, device))
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace must be a device tensor of at least %d bytes" % need)


def _require_gpu(dev):
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU (got %s)" % dev)


def _stream(device):
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def chunk_fwd(q, k, v, log_alpha=None, b=None, w=None, S0=None, order="erase_then_decay",
              out=None, final_state=True, workspace=None, phase_event=None):
    """Chunkwise prefill.  Returns (o [B,T,H,dv] in q's dtype, S_T [B,H,dk,dv] float32 or None).

    ``S0`` (float32 [B,H,dk,dv] or None for zeros) is read before S_T is written; pass
    ``final_state=S0`` to update the state in place.  ``workspace`` is an optional uint8
    device tensor of at least ``workspace_bytes(...)`` bytes; one is allocated when absent.
    ``phase_event`` (a torch.cuda.Event) is recorded between the chunk-local kernel and the
    per-state kernel, for timing the two separately."""
    torch = _torch()
    B, T, HQ, DK = q.shape
    H, DV = v.shape[2], v.shape[-1]
    dt, dev = q.dtype, q.device
    if k.shape != q.shape or v.dim() != 4 or tuple(v.shape[:2]) != (B, T) or HQ == 0 or H % HQ != 0:
        raise ValueError("shape mismatch: q %s k %s v %s (v heads must be a multiple of q / k "
                         "heads)" % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    if k.dtype != dt or v.dtype != dt or k.device != dev or v.device != dev:
        raise TypeError("q, k, v must share dtype and device")
    _io_dtype(q)
    if order not in _ORDERS:
        raise ValueError("order must be one of %s" % sorted(_ORDERS))
    ak = _gate_kind(log_alpha, B, T, H, DK, "log_alpha", dt, dev)
    bk = _gate_kind(b, B, T, H, DK, "b", dt, dev)
    wk = _gate_kind(w, B, T, H, DV, "w", dt, dev)
    _check_contig(q=q, k=k, v=v, log_alpha=log_alpha, b=b, w=w)
    _check_buffer("S0", S0, (B, H, DK, DV), torch.float32, dev)
    _check_buffer("out", out, (B, T, H, DV), dt, dev)
    if final_state is True or final_state is False or final_state is None:
        S_T = None
    else:
        _check_buffer("final_state", final_state, (B, H, DK, DV), torch.float32, dev)
        S_T = final_state
    prob = make_problem(B, H, T, DK, DV, _io_dtype(q), ak, bk, wk, _ORDERS[order],
                        qk_heads=0 if HQ == H else HQ)
    need = _native.workspace_bytes(prob)
    _check_workspace(workspace, need, dev)
    _require_gpu(dev)
    o = out if out is not None else torch.empty((B, T, H, DV), dtype=dt, device=dev)
    if final_state is True:
        S_T = torch.empty((B, H, DK, DV), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev) if need else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if phase_event is None:
        rc = _native.chunk_fwd_raw(prob, _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b),
                                   _ptr(w), _ptr(S0), _ptr(o), _ptr(S_T), _ptr(workspace),
                                   ws_bytes, _stream(dev))
    else:
        if not phase_event.cuda_event:  # torch creates the HIP event at its first record
            phase_event.record(torch.cuda.current_stream(dev))
        rc = _native.chunk_fwd_marked_raw(prob, _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                                          _ptr(b), _ptr(w), _ptr(S0), _ptr(o), _ptr(S_T),
                                          _ptr(workspace), ws_bytes, _stream(dev),
                                          phase_event.cuda_event)
    if rc != _native.GDR_OK:
        raise GdrError(rc, "gdr_chunk_fwd")
    return o, S_T


def chunk_bwd(q, k, v, log_alpha=None, b=None, w=None, S0=None, do=None, dS_T=None,
              order="erase_then_decay", workspace=None):
    """Gradients of ``chunk_fwd`` for the output gradient ``do`` ([B,T,H,dv], q's dtype) and the
    final-state gradient ``dS_T`` (float32 [B,H,dk,dv] or None).  Returns a dict with dq, dk, dv
    (q's dtype), dlog_alpha, db, dw (shaped like the gates; None for an absent gate) and dS0
    (float32).  With one shared beta passed as both b and w, its gradient is db + dw.  With
    grouped q / k heads, dq and dk are summed over the value heads that share them.  Every
    problem chunk_fwd accepts is supported: the chunkwise adjoint for the bf16 shapes of the
    Gated DeltaNet, KDA and Gated DeltaNet-2 models, the exact token adjoint for the rest."""
    torch = _torch()
    B, T, HQ, DK = q.shape
    H, DV = v.shape[2], v.shape[-1]
    dt, dev = q.dtype, q.device
    if k.shape != q.shape or v.dim() != 4 or tuple(v.shape[:2]) != (B, T) or HQ == 0 or H % HQ != 0:
        raise ValueError("shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    if k.dtype != dt or v.dtype != dt or k.device != dev or v.device != dev:
        raise TypeError("q, k, v must share dtype and device")
    _io_dtype(q)
    if order not in _ORDERS:
        raise ValueError("order must be one of %s" % sorted(_ORDERS))
    if do is None:
        raise ValueError("chunk_bwd needs do, the gradient of o")
    _check_buffer("do", do, tuple(v.shape), dt, dev)
    ak = _gate_kind(log_alpha, B, T, H, DK, "log_alpha", dt, dev)
    bk = _gate_kind(b, B, T, H, DK, "b", dt, dev)
    wk = _gate_kind(w, B, T, H, DV, "w", dt, dev)
    _check_contig(q=q, k=k, v=v, log_alpha=log_alpha, b=b, w=w)
    _check_buffer("S0", S0, (B, H, DK, DV), torch.float32, dev)
    _check_buffer("dS_T", dS_T, (B, H, DK, DV), torch.float32, dev)
    prob = make_problem(B, H, T, DK, DV, _io_dtype(q), ak, bk, wk, _ORDERS[order],
                        qk_heads=0 if HQ == H else HQ)
    need = _native.bwd_workspace_bytes(prob)
    _check_workspace(workspace, need, dev)
    _require_gpu(dev)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    like = lambda x: None if x is None else torch.empty_like(x)
    g = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
         "dlog_alpha": like(log_alpha), "db": like(b), "dw": like(w),
         "dS0": torch.empty((B, H, DK, DV), dtype=torch.float32, device=dev)}
    rc = _native.chunk_bwd_raw(prob, _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w),
                               _ptr(S0), _ptr(do), _ptr(dS_T), _ptr(g["dq"]), _ptr(g["dk"]),
                               _ptr(g["dv"]), _ptr(g["dlog_alpha"]), _ptr(g["db"]), _ptr(g["dw"]),
                               _ptr(g["dS0"]), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(dev))
    if rc != _native.GDR_OK:
        raise GdrError(rc, "gdr_chunk_bwd")
    return g


def workspace_bytes(q, v, log_alpha=None, b=None, w=None, order="erase_then_decay"):
    """Workspace bytes ``chunk_fwd`` needs for these inputs (0 when it needs none)."""
    B, T, HQ, DK = q.shape
    H, DV = v.shape[2], v.shape[-1]
    ak = _gate_kind(log_alpha, B, T, H, DK, "log_alpha", q.dtype, q.device)
    bk = _gate_kind(b, B, T, H, DK, "b", q.dtype, q.device)
    wk = _gate_kind(w, B, T, H, DV, "w", q.dtype, q.device)
    return _native.workspace_bytes(make_problem(B, H, T, DK, DV, _io_dtype(q), ak, bk, wk,
                                                _ORDERS[order], qk_heads=0 if HQ == H else HQ))


def decode_step(q, k, v, log_alpha=None, b=None, w=None, S=None, order="erase_then_decay",
                out=None):
    """One decode step on tokens [B,1,H,*]; S [B,H,dk,dv] float32 is updated in place.
    Returns o [B,1,H,dv]."""
    torch = _torch()
    if S is None:
        raise ValueError("decode_step needs the state S")
    B, T, HQ, DK = q.shape
    H, DV = v.shape[2], v.shape[-1]
    if T != 1:
        raise ValueError("decode_step takes one token per sequence (T = 1)")
    dt, dev = q.dtype, q.device
    if k.shape != q.shape or v.dim() != 4 or tuple(v.shape[:2]) != (B, 1) or HQ == 0 or H % HQ != 0:
        raise ValueError("shape mismatch (v heads must be a multiple of q / k heads)")
    if k.dtype != dt or v.dtype != dt or k.device != dev or v.device != dev:
        raise TypeError("q, k, v must share dtype and device")
    _io_dtype(q)
    if order not in _ORDERS:
        raise ValueError("order must be one of %s" % sorted(_ORDERS))
    ak = _gate_kind(log_alpha, B, 1, H, DK, "log_alpha", dt, dev)
    bk = _gate_kind(b, B, 1, H, DK, "b", dt, dev)
    wk = _gate_kind(w, B, 1, H, DV, "w", dt, dev)
    _check_contig(q=q, k=k, v=v, log_alpha=log_alpha, b=b, w=w)
    _check_buffer("S", S, (B, H, DK, DV), torch.float32, dev)
    _check_buffer("out", out, (B, 1, H, DV), dt, dev)
    _require_gpu(dev)
    o = out if out is not None else torch.empty((B, 1, H, DV), dtype=dt, device=dev)
    prob = make_problem(B, H, 1, DK, DV, _io_dtype(q), ak, bk, wk, _ORDERS[order],
                        qk_heads=0 if HQ == H else HQ)
    rc = _native.decode_step_raw(prob, _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b),
                                 _ptr(w), _ptr(S), _ptr(o), _stream(dev))
    if rc != _native.GDR_OK:
        raise GdrError(rc, "gdr_decode_step")
    return o


def mfma_probe(iters, blocks, device=None):
    """Calibration: runs gdr_mfma_probe (register-only bf16 16x16x32 products, 8 chains per wave,
    512-thread workgroups) on the current stream and returns (out, flop): out holds one float per
    wave, exactly 4 * iters; flop is the dense work of the call.  Timing is the caller's."""
    torch = _torch()
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    _require_gpu(dev)
    if iters < 0 or not 1 <= blocks <= 65535:
        raise ValueError("iters >= 0 and 1 <= blocks <= 65535")
    out = torch.empty((blocks * 8,), dtype=torch.float32, device=dev)
    rc = _native.mfma_probe_raw(iters, blocks, _ptr(out), _stream(dev))
    if rc != _native.GDR_OK:
        raise GdrError(rc, "gdr_mfma_probe")
    return out, _native.mfma_probe_flop(iters, blocks)


def build():
    """Compile libgdr.so in-tree for gfx950 (hipcc)."""
    from .buildlib import build as _b
    return _b()
