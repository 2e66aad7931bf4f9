"""Benchmark: chunkwise prefill of the Gated DeltaNet-2 workload (B=1, H=16, T=32768, d_k=d_v=128,
chunk 64, per-channel decay, erase gate b and write gate w, bf16 inputs, fp32 state with a nonzero
S0) as the headline, the KDA and Gated DeltaNet prefills beside it, and the Gated DeltaNet-2 decode
step (256 x 32 states, 1000 steps), on one MI355X, through the C ABI.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gdn2|kda|gdn|mamba2|gla|gdn_gqa|gdn_d256]
                    [--also kda,gdn] [--decode-steps N] [--no-cpu-baseline] [--no-decode]

Prints ONE JSON line.  `value` is prefill tokens/s (B*T / time per call) of the headline workload
with inputs resident in HBM; a step is one gdr_chunk_fwd call over the whole batch.  Two input sets
alternate between calls so that the 256 MB Infinity Cache cannot serve a call from the previous
one.  `roofline` is for one prefill call (all of its kernel launches): algorithmic HBM bytes per
call (inputs read once, o and S_T written once, S0 read once) divided by the mean call time from
HIP events on the launch stream, against MI355X's 8 TB/s; `flops` gives the same call against the
2.5166 PFLOP/s dense bf16 matrix-core peak (algorithmic FLOP of the chunk form, triangular products
at half).  `phases` splits the call with an event recorded after its first launch
(gdr_chunk_fwd_marked).  `traffic` is the measured HBM bytes per call from
profiles/hbm_counters.txt when that file was recorded on the current kernel sources, else null.
`workloads` holds the same figures for the other prefill workloads (`--also`).  `decode` reports
state GB/s for the decode workload (the state is read and written once per step), and under
`copy_reference` the rate of torch's copy kernel over the same bytes; `mfma_calibration` the bf16
matrix-core rate of a register-only loop (gdr_mfma_probe), the reachable side of the 2.5166 PFLOP/s
figure.  `cpu_baseline` times the
fp64 oracle on the host: the whole headline workload on the host threads it may use, and one state
of it on one thread; its outputs also give `parity`, the headline call's errors against the oracle
on the same inputs (max |o - o_ref| and the largest per-state relative Frobenius error of S_T).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2516.6
METRIC = "prefill tokens/s + %bf16 MFMA peak; decode state GB/s + %HBM peak"


def flops_per_head_token(d, C, channel_two_factor, erase=True):
    """Algorithmic FLOP of the chunk form per (head, token); triangular products count half.
    Rank-one form: 6d^2 + 5Cd + C^2/3; per-channel decay applied after the erase:
    8d^2 + 9Cd + C^2/3; no erase gate (Gram, its product with the values, K^T X and Q S):
    4d^2 + 2Cd."""
    if not erase:
        return 4 * d * d + 2 * C * d
    if channel_two_factor:
        return 8 * d * d + 9 * C * d + C * C / 3.0
    return 6 * d * d + 5 * C * d + C * C / 3.0


def prefill_chunk(wl):
    """Chunk length the library's kernels use for this workload: 32 in the segment kernel (bf16,
    d_k = d_v = 128, per-channel decay with per-channel or scalar erase and write gates, or scalar
    decay with scalar gates), 64 elsewhere."""
    gates = ((wl.alpha == "channel" and wl.b == "channel" and wl.w == "channel") or
             (wl.alpha in ("channel", "scalar") and wl.b == "scalar" and wl.w == "scalar"))
    seg = wl.dtype == "bf16" and wl.DK == 128 and wl.DV == 128 and gates
    return 32 if seg else 64


def prefill_bytes(wl):
    """Minimal HBM bytes of one prefill call: every input read once, o and S_T written once."""
    es = 2 if wl.dtype == "bf16" else 4
    rows = wl.B * wl.T * wl.H
    qk_rows = wl.B * wl.T * (wl.HK or wl.H)
    gate = {"none": 0, "scalar": 1, "channel": wl.DK}
    n = qk_rows * 2 * wl.DK * es + rows * 2 * wl.DV * es  # q, k; v, o
    n += rows * gate[wl.alpha] * es
    if wl.shared_beta:
        n += rows * es if wl.b != "none" else 0
    else:
        n += rows * gate[wl.b] * es
        n += rows * {"none": 0, "scalar": 1, "channel": wl.DV}[wl.w] * es
    state = wl.B * wl.H * wl.DK * wl.DV * 4
    n += state * (2 if wl.s0_std > 0 else 1)  # S0 read (if any) and S_T written
    return n


def backward_bytes(wl):
    """Minimal HBM bytes of one backward call: the forward's inputs and do read once, every input
    gradient written once, S0 read (if any) and dS0 written (dS_T is not passed here)."""
    es = 2
    rows = wl.B * wl.T * wl.H
    qk_rows = wl.B * wl.T * (wl.HK or wl.H)
    gate = {"none": 0, "scalar": 1, "channel": wl.DK}
    wgate = {"none": 0, "scalar": 1, "channel": wl.DV}
    per_row = wl.DV + gate[wl.alpha] + gate[wl.b] + wgate[wl.w]
    if wl.shared_beta and wl.b != "none":
        per_row -= gate[wl.b]  # one buffer passed as both b and w
    n = (rows * (2 * per_row + wl.DV) + qk_rows * 4 * wl.DK) * es  # inputs, their gradients; do
    state = wl.B * wl.H * wl.DK * wl.DV * 4
    return n + state * (2 if wl.s0_std > 0 else 1)


def backward_path(wl):
    """Which backward gdr_chunk_bwd runs for the workload: the chunkwise adjoint for bf16 with a
    scalar or no decay at d_k in {32, 64, 128} and d_v up to 256, or a per-channel decay at
    d_k = 128 with d_v 64 or 128; the token adjoint for every other problem."""
    if wl.dtype == "bf16":
        if wl.alpha == "channel" and wl.DK == 128 and wl.DV in (64, 128):
            return "chunkwise"
        if wl.alpha != "channel" and wl.DV <= 256 and wl.DK in (32, 64, 128):
            return "chunkwise"
    return "token"


def decode_bytes(wl):
    es = 2
    n_state = wl.B * wl.H
    state = n_state * wl.DK * wl.DV * 4
    io = n_state * (wl.DK * 4 + wl.DV * 3) * es  # q, k, log alpha, b; v, w, o
    return 2 * state + io


def kernel_source_digest():
    """SHA-256 over the kernel sources and the build script: HBM counter figures recorded for
    other sources no longer describe the kernels that run.  The C ABI's argument validation
    (gdr_api.hip) launches nothing and is left out."""
    import hashlib
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "gated_delta_rule_71_amd")
    files = sorted(os.path.join("csrc", f) for f in os.listdir(os.path.join(pkg, "csrc"))
                   if f != "gdr_api.hip")
    for rel in files + ["buildlib.py"]:
        h.update(rel.encode())
        with open(os.path.join(pkg, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(key):
    """HBM bytes per launch for `key` ("prefill:<workload>" for a whole call, "prefill_prep:" and
    "prefill_state:" for its two kernels, "backward:<workload>" for a gdr_chunk_bwd call, or
    "decode:<workload>") from the
    committed rocprofv3 counter summary, scaled by the calibration copy; None when the summary
    is absent, has no such entry, or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "hbm_counters.txt")
    try:
        lines = open(path).read().splitlines()
    except OSError:
        return None
    digest, found = None, None
    for line in lines:
        f = line.split()
        if len(f) == 2 and f[0] == "source_sha256":
            digest = f[1]
        elif len(f) >= 3 and f[0] == "traffic" and f[1] == key:
            found = float(f[2])
    if digest != kernel_source_digest():
        return None
    return found


def time_prefill(wl, steps, warmup, dev):
    import torch
    import gated_delta_rule_71_amd as gdr
    import synth
    sets = []
    for s in range(2):
        x = synth.make_prefill(wl, seed=wl.seed + 17 * s)
        sets.append({n: (None if t is None else t.to(dev)) for n, t in x.items()})
    outs = [torch.empty((wl.B, wl.T, wl.H, wl.DV), dtype=sets[0]["q"].dtype, device=dev)
            for _ in range(2)]
    S_T = [torch.empty((wl.B, wl.H, wl.DK, wl.DV), dtype=torch.float32, device=dev) for _ in range(2)]

    need = gdr.workspace_bytes(sets[0]["q"], sets[0]["v"], sets[0]["log_alpha"], sets[0]["b"],
                               sets[0]["w"])
    ws = torch.empty((max(1, need),), dtype=torch.uint8, device=dev)

    def call(i, mark=None):
        g = sets[i % 2]
        gdr.chunk_fwd(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"], g["S0"],
                      out=outs[i % 2], final_state=S_T[i % 2], workspace=ws, phase_event=mark)

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    mids = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for e in mids:
        e.record(stream)  # creates the HIP events before the timed region
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        call(i, mids[i])
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))  # ms, one call each
    prep = [s.elapsed_time(m) for s, m in zip(starts, mids)]       # chunk-local kernel
    state = [m.elapsed_time(e) for m, e in zip(mids, ends)]        # per-state kernel
    mean = sum(per) / len(per)
    call(0)  # set 0's outputs for the parity check
    torch.cuda.synchronize()
    return dict(wall_s=wall, mean_ms=mean, median_ms=per[len(per) // 2], p10_ms=per[len(per) // 10],
                p90_ms=per[(9 * len(per)) // 10], prep_ms=sum(prep) / len(prep),
                state_ms=sum(state) / len(state), workspace_bytes=need,
                o=outs[0], S_T=S_T[0])


def time_decode(wl, n_steps, dev):
    import torch
    import gated_delta_rule_71_amd as gdr
    import synth
    S = synth.make_decode_state(wl, dev)
    st = synth.make_decode_steps(wl, n_steps, dev)
    o = torch.empty((wl.B, 1, wl.H, wl.DV), dtype=torch.bfloat16, device=dev)

    def call(i):
        gdr.decode_step(st["q"][i], st["k"][i], st["v"][i], st["log_alpha"][i], st["b"][i],
                        st["w"][i], S, out=o)

    for i in range(min(20, n_steps)):
        call(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n_steps):
        call(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n_steps
    del st
    return ms


def time_mfma_probe(dev, blocks=1024, iters=20000):
    """TFLOP/s of the library's register-only bf16 matrix-core loop (gdr_mfma_probe): the dense
    rate the GPU sustains, beside the 2.5166 PFLOP/s vendor figure the roofline uses.  Four
    512-thread workgroups per CU; checks the probe's exact result."""
    import torch
    import gated_delta_rule_71_amd as gdr
    gdr.mfma_probe(100, blocks, dev)  # warm-up
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    out, flop = gdr.mfma_probe(iters, blocks, dev)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    if not bool((out == 4.0 * iters).all()):
        raise RuntimeError("gdr_mfma_probe returned a wrong result")
    tf = flop / (ms * 1e-3) / 1e12
    return {"TFLOP/s": tf, "frac_of_peak": tf / PEAK_BF16_TFLOPS, "ms": ms, "flop": flop,
            "kernel": "gdr_mfma_probe: 8 independent bf16 16x16x32 MFMA chains per wave, register "
                      "operands, %d workgroups of 512 threads, %d steps" % (blocks, iters)}


def time_copy(nbytes, reps, dev):
    """GB/s (read + write) of torch's device-to-device copy of an fp32 tensor of `nbytes`: the
    rate a plain streaming kernel reaches on this GPU, beside the decode step's."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2 * nbytes / (ms * 1e-3) / 1e9


def time_backward(wl, steps, warmup, dev):
    """gdr_chunk_bwd on the workload's inputs with a seeded output gradient (dS_T = None), the
    workspace allocated once; mean of `steps` calls between HIP events on the launch stream."""
    import torch
    import gated_delta_rule_71_amd as gdr
    import synth
    x = synth.make_prefill(wl)
    g = {n: (None if t is None else t.to(dev)) for n, t in x.items()}
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed + 101)
    do = torch.randn((wl.B, wl.T, wl.H, wl.DV), generator=gen, device=dev).to(torch.bfloat16)
    prob = gdr.make_problem(wl.B, wl.H, wl.T, wl.DK, wl.DV, gdr._native.GDR_BF16,
                            {"none": 0, "scalar": 1, "channel": 2}[wl.alpha],
                            {"none": 0, "scalar": 1, "channel": 2}[wl.b],
                            {"none": 0, "scalar": 1, "channel": 2}[wl.w], 0,
                            qk_heads=0 if wl.HK in (0, wl.H) else wl.HK)
    need = gdr._native.bwd_workspace_bytes(prob)
    ws = torch.empty((need,), dtype=torch.uint8, device=dev)
    run = lambda: gdr.chunk_bwd(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"], g["S0"], do,
                                None, workspace=ws)
    for _ in range(max(1, warmup)):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nb = backward_bytes(wl)
    gbs = nb / (ms * 1e-3) / 1e9
    return {"ms": ms, "tokens_per_s": wl.B * wl.T / (ms * 1e-3), "workspace_bytes": need,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS, "algorithmic_bytes": nb,
                         "traffic": recorded_traffic("backward:" + wl.name),
                         "scope": ("one gdr_chunk_bwd call: chunk maps, two chains, chunk-local adjoint"
                                   if backward_path(wl) == "chunkwise" else
                                   "one gdr_chunk_bwd call: the token adjoint (forward checkpoints, "
                                   "reverse walk, column-block sums)")}}


def time_hooks(wl, dev, positions=64, reps=5):
    """State decomposition ("How Linear Attention Remembers", Analytical Framework): C_i^(t) of
    `positions` evenly spaced positions at the last token, batch row 0 of the workload, one
    hooks.contributions call (positions x T tokens x H heads of recurrence)."""
    import torch
    import synth
    from gated_delta_rule_71_amd import hooks
    x = synth.make_prefill(wl.with_(B=1))
    g = {n: (None if t is None else t.to(dev)) for n, t in x.items()}
    pos = [int(round(i * (wl.T - 1) / (positions - 1))) for i in range(positions)]
    run = lambda: hooks.contributions(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"],
                                      positions=pos, t=wl.T - 1)
    run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"what": "C_i^(t) for %d positions at t = T-1, one sequence of the %s workload"
                    % (positions, wl.name),
            "positions": positions, "ms_per_call": ms,
            "head_tokens_per_s": positions * wl.T * wl.H / (ms * 1e-3),
            "contributions_per_s": positions * wl.H / (ms * 1e-3)}


def host_cpu():
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model or "host"


def cpu_baseline(wl, pf):
    """The fp64 oracle, as it stands, on the host: the whole workload on as many threads as this
    process may use (at most 16, the host share of one GPU), and one (batch, head) state of it on
    one thread.  Its outputs on input set 0 check the GPU call's outputs (`parity`)."""
    import numpy as np
    import oracle
    import synth
    host_cores = len(os.sched_getaffinity(0))
    threads = min(host_cores, 16)
    x = synth.expand_heads(synth.make_prefill(wl), wl.H)
    t0 = time.perf_counter()
    o_ref, S_ref = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], x["S0"],
                                  n_threads=threads)
    dt = time.perf_counter() - t0
    one = {n: (None if t is None else (t[:1, :1] if n == "S0" else t[:1, :, :1])) for n, t in x.items()}
    t1 = time.perf_counter()
    oracle.forward(one["q"], one["k"], one["v"], one["log_alpha"], one["b"], one["w"], one["S0"],
                   n_threads=1)
    dt1 = time.perf_counter() - t1
    o = pf["o"].float().cpu().numpy().astype(np.float64)
    S = pf["S_T"].cpu().numpy().astype(np.float64)
    n = wl.B * wl.H
    rel = (np.linalg.norm((S - S_ref).reshape(n, -1), axis=1) /
           np.linalg.norm(S_ref.reshape(n, -1), axis=1)).max()
    parity = {"max_abs_o": float(np.abs(o - o_ref).max()), "max_rel_frobenius_S_T": float(rel),
              "tolerance": {"o": 2e-2, "S_T": 1e-2}, "states": n, "tokens": wl.B * wl.T,
              "reference": "fp64 oracle on the same (bf16-rounded) inputs"}
    base = {"value": wl.B * wl.T / dt, "unit": "tokens/s", "cores": threads, "host_cores": host_cores,
            "kind": "oracle",
            "sample": "whole %s workload (B=%d, H=%d, T=%d), fp64 recurrence on %d threads, %.1f s wall "
                      "on %s" % (wl.name, wl.B, wl.H, wl.T, threads, dt, host_cpu()),
            "one_core": {"value": wl.T / dt1, "unit": "tokens/s of one state (head-tokens/s)",
                         "sample": "one state of %s (T=%d), 1 thread, %.1f s wall" % (wl.name, wl.T, dt1)}}
    return base, parity


def prefill_report(wl, pf):
    """Throughput and rooflines of one prefill call of workload `wl` from time_prefill's result."""
    two = wl.alpha == "channel"  # erase-then-decay with a per-channel decay: two key families
    sec = pf["mean_ms"] * 1e-3
    chunk = prefill_chunk(wl)
    flops = flops_per_head_token(wl.DK, chunk, two, wl.b != "none") * wl.B * wl.T * wl.H
    nbytes = prefill_bytes(wl)
    gbs = nbytes / sec / 1e9
    tf = flops / sec / 1e12
    return {
        "tokens_per_s": wl.B * wl.T / sec,
        "ms": pf["mean_ms"],
        "kernel_ms": {"mean": pf["mean_ms"], "median": pf["median_ms"], "p10": pf["p10_ms"],
                      "p90": pf["p90_ms"]},
        "config": {"workload": wl.name, "batch": wl.B, "heads": wl.H, "qk_heads": wl.HK or wl.H,
                   "seq_len": wl.T, "d_k": wl.DK, "d_v": wl.DV, "chunk": chunk, "state": "fp32",
                   "decay": wl.alpha, "erase_gate": wl.b, "write_gate": wl.w, "seed": wl.seed,
                   "S0": "N(0, %g^2)" % wl.s0_std if wl.s0_std > 0 else "zero"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS, "traffic": recorded_traffic("prefill:" + wl.name),
                     "algorithmic_bytes": nbytes,
                     "scope": "one gdr_chunk_fwd call (all of its kernel launches)"},
        "flops": {"achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS,
                  "algorithmic_flop": flops},
        "phases": {"first_launch_ms": pf["prep_ms"], "rest_ms": pf["state_ms"],
                   "traffic_first": recorded_traffic("prefill_prep:" + wl.name),
                   "traffic_rest": recorded_traffic("prefill_state:" + wl.name)},
        "workspace_bytes": pf["workspace_bytes"],
    }


def device_identity(dev):
    import torch
    p = torch.cuda.get_device_properties(dev)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "cus": p.multi_processor_count,
            "hbm_bytes": p.total_memory, "hip": torch.version.hip, "torch": torch.__version__}


def progress(msg):
    print("bench: " + msg, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # untimed calls before each timed loop: at least ~50 ms of GPU work, so that the timed calls
    # run at the clocks the GPU holds under load (the first few milliseconds after idle run slower)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="gdn2",
                    choices=["gdn2", "kda", "gdn", "mamba2", "gla", "gdn_gqa", "gdn_d256"])
    ap.add_argument("--also", default="kda,gdn",
                    help="comma-separated prefill workloads timed beside the headline one ('' for none)")
    ap.add_argument("--decode-steps", type=int, default=None)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip timing gdr_chunk_bwd on the timed prefill workloads")
    ap.add_argument("--hooks", action="store_true",
                    help="also time the state-decomposition hook (64 positions, one sequence)")
    ap.add_argument("--no-calibration", action="store_true",
                    help="skip the register-only matrix-core probe (mfma_calibration)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 1 GiB device copy (read 1 GiB, write 1 GiB): the "
                         "reference dispatch that scales rocprofv3 FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the recurrence runs per (batch, head) state with no "
              "communication, and the library has no multi-GPU path (--gpus %d requested)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            torch.mul(src, 1.0, out=dst)  # one elementwise kernel: reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst
    wl = synth.WORKLOADS[args.workload]
    pf = time_prefill(wl, args.steps, args.warmup, dev)
    rep = prefill_report(wl, pf)
    progress("%s prefill %.4f ms" % (wl.name, pf["mean_ms"]))
    out = {
        "metric": METRIC,
        "value": rep["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pf["wall_s"] * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes of the %s workload)" % wl.name,
        "config": rep["config"],
        "kernel_ms": rep["kernel_ms"],
        "mfma_frac": rep["flops"]["frac"],
        "tflops": rep["flops"]["achieved"],
        "roofline": rep["roofline"],
        "flops": rep["flops"],
        "phases": rep["phases"],
        "workspace_bytes": rep["workspace_bytes"],
        "device": device_identity(dev),
    }
    if not args.no_calibration:
        out["mfma_calibration"] = time_mfma_probe(dev)
        progress("mfma probe %.1f TFLOP/s" % out["mfma_calibration"]["TFLOP/s"])
    extra = [n for n in args.also.split(",") if n and n != wl.name]
    if extra:
        out["workloads"] = {}
        for name in extra:
            w2 = synth.WORKLOADS[name]
            p2 = time_prefill(w2, args.steps, args.warmup, dev)
            r2 = prefill_report(w2, p2)
            progress("%s prefill %.4f ms" % (name, p2["mean_ms"]))
            del p2
            out["workloads"][name] = r2
    if not args.no_decode:
        dw = synth.WORKLOADS["decode"]
        n = args.decode_steps or dw.steps
        ms = time_decode(dw, n, dev)
        progress("decode %.1f us per step" % (ms * 1e3))
        db = decode_bytes(dw)
        gbs = db / (ms * 1e-3) / 1e9
        out["decode"] = {"workload": "decode", "batch": dw.B, "heads": dw.H, "d_k": dw.DK,
                         "d_v": dw.DV, "steps": n, "us_per_step": ms * 1e3,
                         "states_per_s": dw.B * dw.H / (ms * 1e-3), "value": gbs, "unit": "GB/s",
                         "hbm_frac": gbs / PEAK_HBM_GBS, "bytes_per_step": db,
                         "traffic": recorded_traffic("decode:decode")}
        # the same bytes through torch's copy kernel: what a plain streaming kernel reaches
        cgbs = time_copy(dw.B * dw.H * dw.DK * dw.DV * 4, 20, dev)
        out["decode"]["copy_reference"] = {"GB/s": cgbs, "bytes": 2 * dw.B * dw.H * dw.DK * dw.DV * 4,
                                           "decode_over_copy": gbs / cgbs}
    if not args.no_backward:
        # every timed prefill workload; the first under "backward".  The token adjoint is tens of
        # times slower than the chunkwise one: a few calls of it suffice
        covered = [wl] + [synth.WORKLOADS[n] for n in extra]
        for i, bw in enumerate(covered):
            tok = backward_path(bw) == "token"
            r = time_backward(bw, min(args.steps, 3) if tok else args.steps, 1 if tok else args.warmup, dev)
            r["path"] = backward_path(bw)
            r["workload"] = bw.name
            progress("%s backward %.4f ms" % (bw.name, r["ms"]))
            if i == 0:
                out["backward"] = r
            else:
                out.setdefault("backward_workloads", {})[bw.name] = r
    if args.hooks:
        out["hooks"] = time_hooks(wl, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"], out["parity"] = cpu_baseline(wl, pf)
        progress("oracle done: parity %s" % json.dumps(out["parity"]))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
