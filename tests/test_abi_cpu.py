"""The C ABI without a GPU: the library loads, exports what include/gdr.h declares, and
rejects bad arguments with the documented status before any HIP call."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_71_amd import _native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A = 0x10000  # fake, 16-byte-aligned device addresses: never dereferenced by a rejected call


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "gdr.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = N.lib()
    names = declared_symbols()
    assert set(names) == set(N.EXPORTED)
    for name in names:
        assert hasattr(lib, name), name


def test_struct_layout_matches_header():
    # two int32, five int64, six int32 -> 4+4 + 40 + 24 = 72 bytes, 8-byte aligned
    assert ctypes.sizeof(N.GdrProblem) == 72


def test_version_and_status_strings():
    assert N.abi_version() == 2
    for s in range(6):
        assert N.status_string(s).startswith("GDR_")
    assert "unknown" in N.status_string(99)


def prob(**kw):
    base = dict(batch=2, heads=3, seqlen=70, dk=128, dv=128, io_dtype=N.GDR_BF16,
                alpha_kind=N.GATE_CHANNEL, b_kind=N.GATE_CHANNEL, w_kind=N.GATE_CHANNEL)
    base.update(kw)
    return N.make_problem(**base)


def call(p, **ptrs):
    a = dict(q=A, k=A * 2, v=A * 3, la=A * 4, b=A * 5, w=A * 6, S0=A * 7, o=A * 8, S_T=A * 9)
    a.update(ptrs)
    return N.chunk_fwd_raw(p, a["q"], a["k"], a["v"], a["la"], a["b"], a["w"], a["S0"], a["o"],
                           a["S_T"], 0, 0, 0)


def big_apart():
    # addresses far enough apart that no two tensors of prob() overlap
    step = 1 << 32
    return dict(q=step, k=2 * step, v=3 * step, la=4 * step, b=5 * step, w=6 * step, S0=7 * step,
                o=8 * step, S_T=9 * step)


@pytest.mark.parametrize("field,value,status", [
    ("struct_size", 8, N.GDR_ERR_INVALID_ARGUMENT),
    ("qk_heads", 2, N.GDR_ERR_INVALID_ARGUMENT),   # 3 value heads are not a multiple of 2
    ("qk_heads", -1, N.GDR_ERR_INVALID_ARGUMENT),
    ("io_dtype", 7, N.GDR_ERR_INVALID_ARGUMENT),
    ("alpha_kind", 3, N.GDR_ERR_INVALID_ARGUMENT),
    ("order", 2, N.GDR_ERR_INVALID_ARGUMENT),
    ("batch", -1, N.GDR_ERR_INVALID_ARGUMENT),
    ("seqlen", -5, N.GDR_ERR_INVALID_ARGUMENT),
    ("dk", 96, N.GDR_ERR_UNSUPPORTED),
    ("dk", 256, N.GDR_ERR_UNSUPPORTED),  # per-channel decay after the erase does not fit at dk 256
    ("io_dtype_dk256", None, N.GDR_ERR_UNSUPPORTED),  # fp32 at dk 256
    ("dk", 0, N.GDR_ERR_INVALID_ARGUMENT),
    ("dv", 40, N.GDR_ERR_UNSUPPORTED),
    ("dv", 512, N.GDR_ERR_UNSUPPORTED),
    ("chunk", 32, N.GDR_ERR_UNSUPPORTED),
])
def test_bad_problem_fields(field, value, status):
    p = prob()
    if field == "io_dtype_dk256":
        p.io_dtype, p.dk, p.alpha_kind = N.GDR_FP32, 256, N.GATE_SCALAR
    else:
        setattr(p, field, value)
    assert call(p, **big_apart()) == status


def test_null_and_misaligned_pointers():
    ok = big_apart()
    for name in ("q", "k", "v", "o", "la", "b", "w"):
        bad = dict(ok)
        bad[name] = 0
        assert call(prob(), **bad) == N.GDR_ERR_INVALID_ARGUMENT, name
    for name in ("q", "k", "v", "o", "la", "b", "w", "S0", "S_T"):
        bad = dict(ok)
        bad[name] = ok[name] + 2
        assert call(prob(), **bad) == N.GDR_ERR_MISALIGNED, name


def test_gate_pointer_ignored_when_kind_none():
    # kind NONE: a NULL gate is fine; the call then fails only on the overlap check below
    p = prob(alpha_kind=N.GATE_NONE, b_kind=N.GATE_NONE, w_kind=N.GATE_NONE)
    ptrs = big_apart()
    ptrs.update(la=0, b=0, w=0, o=ptrs["q"])  # o overlapping q must be rejected
    assert call(p, **ptrs) == N.GDR_ERR_INVALID_ARGUMENT


def test_overlaps_rejected():
    ptrs = big_apart()
    ptrs["o"] = ptrs["v"] + 64  # partial overlap with v
    assert call(prob(), **ptrs) == N.GDR_ERR_INVALID_ARGUMENT
    ptrs = big_apart()
    ptrs["S_T"] = ptrs["S0"] + 1024  # partial overlap of the states
    assert call(prob(), **ptrs) == N.GDR_ERR_INVALID_ARGUMENT


def test_marked_entry_validates_like_the_plain_one():
    # the timing-marker variant shares every check; the (fake) event is never recorded here
    ev = 1 << 40
    cases = [(prob(), big_apart()), (prob(dk=96), big_apart()), (prob(batch=0), big_apart()),
             (prob(), dict(big_apart(), q=0)), (prob(), dict(big_apart(), o=big_apart()["v"] + 64))]
    for p, ptrs in cases:
        a = dict(q=A, k=A * 2, v=A * 3, la=A * 4, b=A * 5, w=A * 6, S0=A * 7, o=A * 8, S_T=A * 9)
        a.update(ptrs)
        plain = call(p, **ptrs)
        marked = N.chunk_fwd_marked_raw(p, a["q"], a["k"], a["v"], a["la"], a["b"], a["w"],
                                        a["S0"], a["o"], a["S_T"], 0, 0, 0, ev)
        assert marked == plain
    assert plain == N.GDR_ERR_INVALID_ARGUMENT


def test_empty_problem_is_a_no_op():
    # nothing to do: returns OK without touching the (fake) pointers or the GPU
    assert call(prob(batch=0), **big_apart()) == N.GDR_OK
    assert call(prob(heads=0), **big_apart()) == N.GDR_OK


def test_workspace_query_and_decode_validation():
    # per-channel decay (either order): the chunk's affine map A' (dk x dk), Q' (64 x dk), D^T
    # (dv x dk), Z' (64 x dv) in bf16, e^{G_n} (dk + 4 fp32) and a flag per 64-token chunk of every
    # (batch, head), each array rounded up to 256 bytes
    r = lambda n: (n + 255) // 256 * 256
    ch = 2 * 3 * 2
    two = r(ch * 128 * 128 * 2) + r(ch * 64 * 128 * 2) + r(ch * 128 * 128 * 2) + \
        r(ch * 64 * 128 * 2) + r(ch * 132 * 4) + r(ch * 4)
    assert N.workspace_bytes(prob()) == two
    assert N.workspace_bytes(prob(order=N.DECAY_THEN_ERASE)) == two
    # scalar decay in bf16: W (64 x dk), U (64 x dv), -M (64 x 64), all bf16, and 132 fp32 gate
    # exponentials per 64-token chunk of every (batch, head), each array rounded up to 256 bytes
    sp = prob(alpha_kind=N.GATE_SCALAR, b_kind=N.GATE_SCALAR, w_kind=N.GATE_SCALAR)
    chunks = 2 * 3 * 2  # batch 2, heads 3, ceil(70 / 64) = 2
    r = lambda n: (n + 255) // 256 * 256
    need = r(chunks * 64 * 128 * 2) + r(chunks * 64 * 128 * 2) + r(chunks * 64 * 64 * 2) + \
        r(chunks * 132 * 4)
    assert N.workspace_bytes(sp) == need
    assert N.workspace_bytes(prob(alpha_kind=N.GATE_SCALAR, b_kind=N.GATE_SCALAR, w_kind=N.GATE_SCALAR,
                                  io_dtype=N.GDR_FP32, dk=32, dv=32)) == 0
    a = big_apart()
    args = [a[n] for n in ("q", "k", "v", "la", "b", "w", "S0", "o", "S_T")]
    ws = 10 * (1 << 32)
    assert N.chunk_fwd_raw(sp, *args, ws, need - 1, 0) == N.GDR_ERR_WORKSPACE_TOO_SMALL
    assert N.chunk_fwd_raw(sp, *args, 0, need, 0) == N.GDR_ERR_INVALID_ARGUMENT
    assert N.chunk_fwd_raw(sp, *args, ws + 8, need, 0) == N.GDR_ERR_MISALIGNED
    p = prob(seqlen=2)
    step = 1 << 32
    rc = N.decode_step_raw(p, step, 2 * step, 3 * step, 4 * step, 5 * step, 6 * step, 7 * step,
                           8 * step, 0)
    assert rc == N.GDR_ERR_INVALID_ARGUMENT  # decode needs seqlen == 1
    p = prob(seqlen=1)
    rc = N.decode_step_raw(p, step, 2 * step, 3 * step, 4 * step, 5 * step, 6 * step, 0, 8 * step, 0)
    assert rc == N.GDR_ERR_INVALID_ARGUMENT  # NULL state


def test_python_binding_rejects_host_tensors():
    import torch
    import gated_delta_rule_71_amd as gdr
    q = torch.zeros(1, 4, 1, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        gdr.chunk_fwd(q, q, q)
    with pytest.raises(TypeError):
        gdr.chunk_fwd(q.float(), q, q)


def bwd_ptrs():
    step = 1 << 32
    names = ("q", "k", "v", "la", "b", "w", "S0", "dO", "dS_T", "dq", "dk", "dv", "dla", "db", "dw",
             "dS0")
    return {n: (i + 1) * step for i, n in enumerate(names)}


def bwd_call(p, ws=0, ws_bytes=0, **over):
    a = bwd_ptrs()
    a.update(over)
    return N.chunk_bwd_raw(p, *[a[n] for n in ("q", "k", "v", "la", "b", "w", "S0", "dO", "dS_T", "dq",
                                                "dk", "dv", "dla", "db", "dw", "dS0")], ws, ws_bytes, 0)


def test_backward_workspace_and_validation():
    sp = prob(alpha_kind=N.GATE_SCALAR, b_kind=N.GATE_SCALAR, w_kind=N.GATE_SCALAR)
    # the per-channel forward's chunk map, four bf16 dk x dv checkpoints and Q'^T dO per 64-token chunk of
    # every (batch, head), each array rounded up to 256 bytes
    r = lambda n: (n + 255) // 256 * 256
    ch = 2 * 3 * 2
    need = r(ch * 128 * 128 * 2) + r(ch * 64 * 128 * 2) + r(ch * 128 * 128 * 2) + \
        r(ch * 64 * 128 * 2) + r(ch * 132 * 4) + r(ch * 4) + 5 * r(ch * 128 * 128 * 2)
    assert N.bwd_workspace_bytes(sp) == need
    # grouped q / k heads: dq and dk per value head as well (bf16 [B, T, H, dk] each)
    gp = prob(alpha_kind=N.GATE_SCALAR, heads=4, qk_heads=2)
    chg = 2 * 4 * 2
    assert N.bwd_workspace_bytes(gp) == (
        r(chg * 128 * 128 * 2) + r(chg * 64 * 128 * 2) + r(chg * 128 * 128 * 2) + r(chg * 64 * 128 * 2) +
        r(chg * 132 * 4) + r(chg * 4) + 5 * r(chg * 128 * 128 * 2) + 2 * r(2 * 70 * 4 * 128 * 2))
    # d_v = 256: the chunk-local adjoint runs per 128-column half, with partial dq, dk (per value
    # head) and per-token gate gradients (three arrays of [B, T, H, dk] bf16) per half
    wp = prob(alpha_kind=N.GATE_SCALAR, b_kind=N.GATE_SCALAR, w_kind=N.GATE_SCALAR, dv=256)
    rows = 2 * 70 * 3
    assert N.bwd_workspace_bytes(wp) == (
        r(ch * 128 * 128 * 2) + r(ch * 64 * 128 * 2) + r(ch * 256 * 128 * 2) + r(ch * 64 * 256 * 2) +
        r(ch * 132 * 4) + r(ch * 4) + 5 * r(ch * 128 * 256 * 2) + 2 * 2 * r(rows * 128 * 2) +
        3 * 2 * r(rows * 128 * 2))
    # outside the backward's scope: per-channel decay, fp32, dv > 256, dk = 16
    for p in (prob(), prob(alpha_kind=N.GATE_SCALAR, io_dtype=N.GDR_FP32),
              prob(alpha_kind=N.GATE_SCALAR, dv=512), prob(alpha_kind=N.GATE_SCALAR, dk=16)):
        assert N.bwd_workspace_bytes(p) == 0
        assert bwd_call(p) == N.GDR_ERR_UNSUPPORTED
    ws = 20 * (1 << 32)
    assert bwd_call(sp, ws, need - 1) == N.GDR_ERR_WORKSPACE_TOO_SMALL
    assert bwd_call(sp, 0, need) == N.GDR_ERR_INVALID_ARGUMENT
    assert bwd_call(sp, ws + 8, need) == N.GDR_ERR_MISALIGNED
    for name in ("q", "dO", "dq", "dk", "dv", "dla", "db", "dw"):
        assert bwd_call(sp, ws, need, **{name: 0}) == N.GDR_ERR_INVALID_ARGUMENT, name
    for name in ("dO", "dS_T", "dq", "dla", "dS0"):
        assert bwd_call(sp, ws, need, **{name: bwd_ptrs()[name] + 4}) == N.GDR_ERR_MISALIGNED, name
    # an output over an input, or over another output
    assert bwd_call(sp, ws, need, dq=bwd_ptrs()["k"] + 64) == N.GDR_ERR_INVALID_ARGUMENT
    assert bwd_call(sp, ws, need, dk=bwd_ptrs()["dq"] + 64) == N.GDR_ERR_INVALID_ARGUMENT
    assert bwd_call(sp, ws, need, dS0=bwd_ptrs()["dS_T"]) == N.GDR_ERR_INVALID_ARGUMENT
    # nothing to do
    assert bwd_call(prob(alpha_kind=N.GATE_SCALAR, batch=0)) == N.GDR_OK
