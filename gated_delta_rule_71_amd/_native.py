"""ctypes view of libgdr.so's C ABI (include/gdr.h).  Argument marshalling only."""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdr.so")

GDR_OK = 0
GDR_ERR_INVALID_ARGUMENT = 1
GDR_ERR_UNSUPPORTED = 2
GDR_ERR_MISALIGNED = 3
GDR_ERR_WORKSPACE_TOO_SMALL = 4
GDR_ERR_HIP = 5

GDR_BF16, GDR_FP32 = 0, 1
GATE_NONE, GATE_SCALAR, GATE_CHANNEL = 0, 1, 2
ERASE_THEN_DECAY, DECAY_THEN_ERASE = 0, 1

EXPORTED = ("gdr_abi_version", "gdr_status_string", "gdr_chunk_fwd_workspace_bytes",
            "gdr_chunk_fwd", "gdr_chunk_fwd_marked", "gdr_chunk_fwd_noalloc", "gdr_decode_step",
            "gdr_chunk_bwd_workspace_bytes", "gdr_chunk_bwd", "gdr_mfma_probe", "gdr_mfma_probe_flop")
NOALLOC_SCRATCH_BYTES = 64 << 20  # GDR_NOALLOC_SCRATCH_BYTES


class GdrProblem(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_int32),
        ("io_dtype", ctypes.c_int32),
        ("batch", ctypes.c_int64),
        ("heads", ctypes.c_int64),
        ("seqlen", ctypes.c_int64),
        ("dk", ctypes.c_int64),
        ("dv", ctypes.c_int64),
        ("chunk", ctypes.c_int32),
        ("alpha_kind", ctypes.c_int32),
        ("b_kind", ctypes.c_int32),
        ("w_kind", ctypes.c_int32),
        ("order", ctypes.c_int32),
        ("qk_heads", ctypes.c_int32),
    ]


def make_problem(batch, heads, seqlen, dk, dv, io_dtype=GDR_BF16, alpha_kind=GATE_NONE,
                 b_kind=GATE_NONE, w_kind=GATE_NONE, order=ERASE_THEN_DECAY, chunk=64, qk_heads=0):
    return GdrProblem(ctypes.sizeof(GdrProblem), io_dtype, batch, heads, seqlen, dk, dv, chunk,
                      alpha_kind, b_kind, w_kind, order, qk_heads)


class GdrError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s" % (where, status_string(status)))


_lib = None


def lib():
    """The loaded library.  Raises if it has not been built: there is no fallback path."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libgdr.so is not built (%s); run `python -m "
                               "gated_delta_rule_71_amd.buildlib` first" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        pp = ctypes.POINTER(GdrProblem)
        L.gdr_abi_version.restype = ctypes.c_int
        L.gdr_abi_version.argtypes = []
        L.gdr_status_string.restype = ctypes.c_char_p
        L.gdr_status_string.argtypes = [ctypes.c_int]
        L.gdr_chunk_fwd_workspace_bytes.restype = sz
        L.gdr_chunk_fwd_workspace_bytes.argtypes = [pp]
        L.gdr_chunk_fwd.restype = ctypes.c_int
        L.gdr_chunk_fwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.gdr_chunk_fwd_marked.restype = ctypes.c_int
        L.gdr_chunk_fwd_marked.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp]
        L.gdr_chunk_fwd_noalloc.restype = ctypes.c_int
        L.gdr_chunk_fwd_noalloc.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.gdr_decode_step.restype = ctypes.c_int
        L.gdr_decode_step.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.gdr_chunk_bwd_workspace_bytes.restype = sz
        L.gdr_chunk_bwd_workspace_bytes.argtypes = [pp]
        L.gdr_chunk_bwd.restype = ctypes.c_int
        L.gdr_chunk_bwd.argtypes = [pp] + [vp] * 17 + [sz, vp]
        L.gdr_mfma_probe.restype = ctypes.c_int
        L.gdr_mfma_probe.argtypes = [ctypes.c_int64, ctypes.c_int32, vp, vp]
        L.gdr_mfma_probe_flop.restype = ctypes.c_int64
        L.gdr_mfma_probe_flop.argtypes = [ctypes.c_int64, ctypes.c_int32]
        _lib = L
    return _lib


def status_string(status):
    return lib().gdr_status_string(int(status)).decode()


def abi_version():
    return lib().gdr_abi_version()


def workspace_bytes(problem):
    return lib().gdr_chunk_fwd_workspace_bytes(ctypes.byref(problem))


def chunk_fwd_raw(problem, q, k, v, la, b, w, S0, o, S_T, ws, ws_bytes, stream):
    """Direct call with integer device addresses (0 = NULL).  Returns the status."""
    return lib().gdr_chunk_fwd(ctypes.byref(problem), q or None, k or None, v or None, la or None,
                               b or None, w or None, S0 or None, o or None, S_T or None,
                               ws or None, ws_bytes, stream or None)


def chunk_fwd_marked_raw(problem, q, k, v, la, b, w, S0, o, S_T, ws, ws_bytes, stream, event):
    """chunk_fwd_raw that also records the HIP event `event` (raw handle) between the
    chunk-local and the per-state kernel.  Returns the status."""
    return lib().gdr_chunk_fwd_marked(ctypes.byref(problem), q or None, k or None, v or None,
                                      la or None, b or None, w or None, S0 or None, o or None,
                                      S_T or None, ws or None, ws_bytes, stream or None,
                                      event or None)


def chunk_fwd_noalloc_raw(problem, q, k, v, la, b, w, S0, o, S_T, stream):
    """gdr_chunk_fwd_noalloc with integer device addresses (0 = NULL).  Returns the status."""
    return lib().gdr_chunk_fwd_noalloc(ctypes.byref(problem), q or None, k or None, v or None,
                                       la or None, b or None, w or None, S0 or None, o or None,
                                       S_T or None, stream or None)


def decode_step_raw(problem, q, k, v, la, b, w, S, o, stream):
    return lib().gdr_decode_step(ctypes.byref(problem), q or None, k or None, v or None,
                                 la or None, b or None, w or None, S or None, o or None,
                                 stream or None)


def bwd_workspace_bytes(problem):
    return lib().gdr_chunk_bwd_workspace_bytes(ctypes.byref(problem))


def chunk_bwd_raw(problem, q, k, v, la, b, w, S0, dO, dS_T, dq, dk, dv, dla, db, dw, dS0, ws,
                  ws_bytes, stream):
    """gdr_chunk_bwd with integer device addresses (0 = NULL).  Returns the status."""
    n = lambda x: x or None
    return lib().gdr_chunk_bwd(ctypes.byref(problem), n(q), n(k), n(v), n(la), n(b), n(w), n(S0),
                               n(dO), n(dS_T), n(dq), n(dk), n(dv), n(dla), n(db), n(dw), n(dS0),
                               n(ws), ws_bytes, n(stream))


def mfma_probe_raw(iters, blocks, out, stream):
    return lib().gdr_mfma_probe(int(iters), int(blocks), out, stream)


def mfma_probe_flop(iters, blocks):
    return lib().gdr_mfma_probe_flop(int(iters), int(blocks))
