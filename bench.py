#!/usr/bin/env python3
"""Benchmark of the KDA forward hot path on one MI355X.

Prints ONE JSON line.  `value` is prefill throughput on the 8K-token workload
(H=32, T=8192, d_k=d_v=128, chunk 64, bf16): one step = the gate and the
prefill over one batch of seeded synthetic inputs already resident in HBM, as
one kda_prefill_gated call (the gate computed in the prefill's decay stage;
three input sets are rotated so the 256 MB last-level cache cannot hold a
step's working set).  `unfused` times the same work as kda_gate + kda_prefill.
The decode leg (B=256, H=32, 1000 consecutive in-place steps) is reported
under "decode" (one kda_decode_step_gated call per step; `unfused` times
kda_gate + kda_decode_step), and verify/commit (B=256, K=4) under
"speculative".  Every duration is the mean over back-to-back calls bracketed
by two HIP events on the stream the library launches on (an event between
calls would serialise them).  `roofline` covers the prefill call (algorithmic
bytes per call); each roofline also carries the fraction of a plain 1 GiB
device copy measured on the same device, and the prefill's matrix-core rate
is also given against a plain bf16 GEMM measured there.  `cpu_baseline` is the fp64 oracle
timed on this host on a bounded sample; `verified` compares the timed run's
output with that oracle pass (whole workload, normwise max relative error).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--decode-steps D]
                  [--no-cpu] [--copy-calib] [--spin-up SECONDS]

Before the W warmup steps the prefill step runs untimed for --spin-up seconds
(0.5 by default) so that the timed steps see the GPU's steady clocks.

Two more legs time the million-token workloads: `prefill_1m` (one sequence,
H=8, T=2^20, z shifted by +3) and `varlen_64` (64 packed sequences, ~1.03M
tokens, H=32, initial states N(0, 0.01)), each one kda_prefill_gated call on
seeded inputs drawn on the device (the same distributions as the tests'), with
its HBM roofline and an oracle check on sampled heads and sequences.
`f32_prefill` times the 8K shape with fp32 tensors (the token-serial path,
segments with warm-up windows) and checks two heads against the oracle.
`measured_roofs` holds the device's own streaming bandwidth (read, write, copy
and in-place kernels) and bf16 matrix-core issue rate (libkda_roofs), against
which every roofline also reports a fraction.  Decode and commit also report
against the same in-place update over their own 512 MiB working set, part of
which the 256 MB last-level cache keeps between launches; the decode leg times
one more step over a 4 GiB state (B=2048), past that cache, for comparison
with the 4 GiB roof.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s (H=32,d=128,T=8K) + decode tok/s (B=256); % of roofline"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
SPIN_UP_S = 0.5  # untimed full steps before the warmup steps


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_sequence_gate_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def load_traffic(kind: str):
    """HBM bytes per call from committed rocprofv3 --pmc runs, if they were
    taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", f"{kind}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("source_hash") != kernel_source_hash():
        return None
    return d.get("bytes_per_call")


def prefill_algo(T: int, H: int, dk: int, dv: int, chunk: int = 64, N: int = 1, with_init: bool = False):
    """Algorithmic HBM bytes and flops of one prefill call (bf16 tokens, fp32 state).

    bytes: q, k, g, v, beta read once, o written once, the N final states
    written (and the N initial states read, with_init).
    flops: per token and head, C*(3*dk + 2*dv) + 6*dk*dv for the chunkwise form
    with triangular intra-chunk products (2 flops per multiply-add)."""
    tok = T * H
    states = N * H * dk * dv * 4
    nbytes = tok * (3 * dk + dv + 1) * 2 + tok * dv * 2 + states * (2 if with_init else 1)
    flops = tok * (chunk * (3 * dk + 2 * dv) + 6 * dk * dv)
    return nbytes, flops


def decode_algo(B: int, H: int, dk: int, dv: int):
    """State read + write (fp32) plus q, k, g, v, beta in and o out (bf16)."""
    bh = B * H
    nbytes = bh * dk * dv * 4 * 2 + bh * (3 * dk + dv + 1) * 2 + bh * dv * 2
    flops = bh * (7 * dk * dv)  # decay 1, two column sums 2+2, rank-1 update 2
    return nbytes, flops


def spec_algo(B: int, K: int, H: int, dk: int, dv: int, commit: bool):
    """verify: state read once, K draft tokens in, K outputs out; commit (all K
    accepted): state read and written once, K tokens in (no q, no output)."""
    bh = B * H
    state = bh * dk * dv * 4 * (2 if commit else 1)
    tok = bh * K * ((2 * dk + dv + 1) * 2 if commit else (3 * dk + dv + 1) * 2 + dv * 2)
    return state + tok


def backward_algo(T: int, H: int, dk: int, dv: int, interval: int = 64):
    """q, k, g, v, beta and dO read (bf16), dq, dk, dg, dv, dbeta written (fp32),
    the forward's checkpoints read once (one state per 64 tokens), the final
    state's gradient read and the initial state's written (fp32)."""
    tok = T * H
    return (tok * (3 * dk + 2 * dv + 1) * 2 + tok * (3 * dk + dv + 1) * 4 + (T // interval) * H * dk * dv * 4
            + 2 * H * dk * dv * 4)


CPU_SHARE = 16  # CPU threads the baseline uses at most: one GPU's share of the host


def host_cpu() -> dict:
    """What the CPU baseline ran on: the machine's logical CPUs, the ones this
    process may use, and the model name."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        allowed = len(os.sched_getaffinity(0))
    except AttributeError:
        allowed = os.cpu_count()
    return {"logical_cpus": os.cpu_count(), "allowed_cpus": allowed, "model": model}


def cpu_baseline(wl, seconds: float = 12.0):
    """The fp64 oracle on this host over the whole 8K workload (every head,
    every token), repeated until at least `seconds` have passed; tokens/s of
    the full problem.  The oracle is compiled here for this host (gcc -O3
    -march=native, OpenMP) and runs one thread per head, up to the host share
    of CPUs.  Also returns the first pass's (o, S): the oracle's result for
    input set 0 (bf16-rounded inputs, as the GPU holds them; g from the gate
    in fp64, unrounded, as the fused gate keeps it), against which the timed
    run's output is checked."""
    import tempfile
    import oracle
    import synth
    cpu = host_cpu()
    threads = max(1, min(wl.H, CPU_SHARE, cpu["allowed_cpus"] or 1))
    out = os.path.join(tempfile.mkdtemp(prefix="kda_oracle_"), "liboracle_native.so")
    oracle.build(out=out, native=True)
    lib = oracle.load(out)
    x = synth.prefill_inputs(wl)
    for n in ("q", "k", "v", "z", "beta"):
        x[n] = oracle.round_bf16(x[n], lib=lib)
    g = oracle.gate(x["z"], x["A"], lib=lib)  # the fused gate keeps g in fp32
    reps, first, t0 = 0, None, time.perf_counter()
    while True:
        res = oracle.prefill(x["q"], x["k"], x["v"], g, x["beta"], threads=threads, lib=lib)
        first = first or res
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            break
    return ({"value": round(reps * wl.T_total / dt, 1), "unit": "tokens/s", "cores": threads,
             "threads": threads, "kind": "oracle", "build": "gcc -O3 -march=native -fopenmp, built on this host",
             "host": cpu,
             "sample": f"fp64 token-serial oracle on the whole 8K workload ({wl.H} heads x "
                       f"{wl.T_total} tokens, one head per thread), {reps} passes in {dt:.1f} s"}, first)


def max_rel_err(got, want) -> float:
    """Normwise max relative error, max|got - want| / max|want|."""
    import numpy as np
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    return float(np.max(np.abs(got - want)) / max(float(np.max(np.abs(want))), 1e-300))


def measured_roofs(torch, dev, stream) -> dict:
    """Streaming read, write and copy bandwidth over 4 GiB and the bf16
    matrix-core issue rate, measured with libkda_roofs on this device."""
    import ctypes
    from linear_attention_sequence_gate_amd import build as kbuild
    L = ctypes.CDLL(kbuild.ROOFS_LIB)
    P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    L.kda_roof_stream.argtypes = [I, P, P, I64, P, I64, I, I, P, ctypes.POINTER(ctypes.c_float)]
    L.kda_roof_mfma.argtypes = [I, I, P, P, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double)]
    nbytes = 4 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.fill_(0)
    sink = torch.empty(32768 * 256, dtype=torch.int32, device=dev)
    ms = ctypes.c_float(0.0)
    out = {}
    # (mode, name, bytes moved per launch, workgroups: 0 = one vector per thread);
    # the shapes are the fastest of a sweep of grid-stride widths, one to sixteen
    # vectors per thread and streaming or plain stores on MI355X
    for mode, name, moved, wgs in ((0, "hbm_read_gbs", nbytes, 8192), (1, "hbm_write_gbs", nbytes, 32768),
                                   (2, "hbm_copy_gbs", 2 * nbytes, 0), (3, "hbm_inplace_gbs", 2 * nbytes, 0)):
        rc = L.kda_roof_stream(mode, src.data_ptr(), dst.data_ptr(), nbytes, sink.data_ptr(), sink.numel(), wgs, 5,
                               stream.cuda_stream, ctypes.byref(ms))
        if rc != 0:
            raise RuntimeError(f"kda_roof_stream mode {mode}: {rc}")
        out[name] = round(moved / (ms.value * 1e-3) / 1e9, 1)
    # in place in the decode step's access pattern (64 KB fp32 states, all 16
    # loads of a lane in flight, streaming stores), the delay between each
    # workgroup's loads and stores swept (it spreads their read and write
    # bursts apart): over 4 GiB, and over 512 MiB, the size of the decode
    # workload's state, which the 256 MB last-level cache partly holds from
    # one launch to the next
    L.kda_roof_state_inplace.argtypes = [P, I64, I, I, P, ctypes.POINTER(ctypes.c_float)]
    for size, name, reps in ((nbytes, "hbm_inplace_state_gbs", 5), (512 << 20, "inplace_state_512mib_gbs", 50)):
        best, best_delay = 0.0, 0
        for delay in (0, 16, 20, 24, 28, 32):
            rc = L.kda_roof_state_inplace(dst.data_ptr(), size, delay, reps, stream.cuda_stream, ctypes.byref(ms))
            if rc != 0:
                raise RuntimeError(f"kda_roof_state_inplace: {rc}")
            gbs = 2 * size / (ms.value * 1e-3) / 1e9
            if gbs > best:
                best, best_delay = gbs, delay
        out[name] = round(best, 1)
        out[name.replace("_gbs", "_delay")] = best_delay
    out["hbm_rw_gbs"] = max(out["hbm_copy_gbs"], out["hbm_inplace_gbs"], out["hbm_inplace_state_gbs"])
    del src, dst
    fsink = torch.empty(256 * 8 * 256, dtype=torch.float32, device=dev)
    fl = ctypes.c_double(0.0)
    rc = L.kda_roof_mfma(256 * 8, 4096, fsink.data_ptr(), stream.cuda_stream, ctypes.byref(ms), ctypes.byref(fl))
    if rc != 0:
        raise RuntimeError(f"kda_roof_mfma: {rc}")
    out["mfma_bf16_tflops"] = round(fl.value / (ms.value * 1e-3) / 1e12, 1)
    out["how"] = ("libkda_roofs over 4 GiB, 16-byte vectors, mean of 5 launches: read grid-stride over 8192 "
                  "workgroups of 256, write grid-stride over 32768, copy and in-place update one vector per "
                  "thread, in-place update of 64 KB fp32 states in the decode step's access pattern with "
                  "streaming stores, best over a 0-32 round delay between loads and stores (read + write "
                  "bytes; hbm_rw_gbs is the largest of the three); the same state update over 512 MiB, the "
                  "decode workload's own working set (inplace_state_512mib_gbs, mean of 50); 2048 "
                  "workgroups of 4 waves, each issuing 4096 x 8 independent v_mfma_f32_16x16x32_bf16")
    return out


def device_inputs(torch, wl, dev, seed):
    """The workload's token tensors drawn on the device (seeded torch
    generator, the distributions of the seeded host generator): q, k ~ N(0,1)
    L2-normalised per (token, head), v ~ N(0,1), z ~ N(shift, 1),
    beta = sigmoid(N(0,1)), all rounded once to bf16; drawn in windows so the
    fp32 temporaries stay small."""
    gen = torch.Generator(device=dev).manual_seed(seed)
    T, H = wl.T_total, wl.H
    out = {n: torch.empty((T, H, wl.dv if n == "v" else wl.dk), dtype=torch.bfloat16, device=dev)
           for n in ("q", "k", "v", "z")}
    out["beta"] = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    step = 1 << 16
    for t0 in range(0, T, step):
        t1 = min(T, t0 + step)
        for n in ("q", "k"):
            x = torch.randn((t1 - t0, H, wl.dk), generator=gen, device=dev)
            out[n][t0:t1] = (x / x.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
        out["v"][t0:t1] = torch.randn((t1 - t0, H, wl.dv), generator=gen, device=dev).to(torch.bfloat16)
        out["z"][t0:t1] = (torch.randn((t1 - t0, H, wl.dk), generator=gen, device=dev) + wl.z_shift).to(
            torch.bfloat16)
        out["beta"][t0:t1] = torch.sigmoid(torch.randn((t1 - t0, H), generator=gen, device=dev)).to(torch.bfloat16)
    return out


def big_leg(kda, torch, synth, wl, dev, stream, timed_loop, rw_gbs, roof_ms, steps=5):
    """One million-token workload: one kda_prefill_gated call per step, timed
    over `steps` back-to-back calls, with its HBM roofline and an oracle check
    of sampled outputs and final states the fp64 oracle computes exactly."""
    import numpy as np
    import oracle
    T, H, dk, dv, N = wl.T_total, wl.H, wl.dk, wl.dv, wl.N
    x = device_inputs(torch, wl, dev, wl.seed)
    A = torch.from_numpy(synth.gate_A(wl)).to(dev)
    cu = torch.from_numpy(wl.cu_seqlens).to(dev) if N > 1 else None
    S0 = torch.from_numpy(synth.initial_state(wl)).to(dev) if wl.state_std > 0 else None
    o = torch.empty((T, H, dv), dtype=torch.bfloat16, device=dev)
    S = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    ws = torch.empty(max(kda.kda_prefill_workspace_size(T, N, H, dk, dv), 1), dtype=torch.uint8, device=dev)

    def call(i):
        kda.kda_prefill_gated(x["q"], x["k"], x["v"], x["z"], A, x["beta"], cu_seqlens=cu, initial_state=S0,
                              final_state=S, o=o, workspace=ws)

    for i in range(2):
        call(i)
    ms = timed_loop(call, steps)
    nbytes, flops = prefill_algo(T, H, dk, dv, N=N, with_init=S0 is not None)
    ach = nbytes / (ms * 1e-3) / 1e9
    # oracle check on samples: outputs from the sequence start (exact from the
    # known initial state) and whole short sequences with their final states
    hx = lambda t: t.float().cpu().numpy()
    Ah = synth.gate_A(wl)
    heads = [0, H // 2 + 1]
    errs = {}
    cuh = wl.cu_seqlens
    picks = [0] if N == 1 else [int(n) for n in np.argsort(np.asarray(wl.seqlens))[:2]]
    for n in picks:
        a = int(cuh[n])
        b = min(int(cuh[n + 1]), a + 8192)
        xs = {k_: hx(x[k_][a:b][:, heads]) for k_ in ("q", "k", "v", "z")}
        xs["beta"] = hx(x["beta"][a:b][:, heads])
        g = oracle.gate(xs["z"], Ah[heads])
        s0 = None if S0 is None else S0[n:n + 1][:, heads].cpu().numpy()
        o_ref, S_ref = oracle.prefill(xs["q"], xs["k"], xs["v"], g, xs["beta"], S0=s0)
        errs[f"seq{n}_heads{heads}_o_tokens_{b - a}"] = max_rel_err(hx(o[a:b][:, heads]), o_ref)
        if b == int(cuh[n + 1]):
            errs[f"seq{n}_heads{heads}_final_state"] = max_rel_err(S[n, heads].cpu().numpy(), S_ref[0])
    del x, ws
    return {"value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "ms_per_call": round(ms, 4), "steps": steps,
            "config": {"workload": wl.name, "N": N, "H": H, "T": T, "d_k": dk, "d_v": dv, "z_shift": wl.z_shift,
                       "initial_state": S0 is not None, "inputs": "drawn on the device, seeded"},
            "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(ach / HBM_PEAK_GBS, 4), "frac_of_measured_rw": round(ach / rw_gbs, 4) if rw_gbs else None,
                         "binding_roof_ms": roof_ms, "algorithmic_bytes_per_call": nbytes,
                         "mfma_tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                         "traffic": load_traffic(wl.name), "kernel": "kda_prefill_gated"},
            "verified": {"against": "fp64 oracle on sampled heads and sequences (exact from their initial state)",
                         "max_rel_err": errs, "tolerance": 2e-2}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--spin-up", type=float, default=SPIN_UP_S,
                    help="seconds of untimed steps before the warmup steps (clock ramp)")
    ap.add_argument("--no-big", action="store_true", help="skip the million-token legs")
    ap.add_argument("--legs", default="decode,speculative,backward,f32,roofs,big",
                    help="comma-separated legs to run beside the 8K prefill (default: all)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    legs = set(x for x in args.legs.split(",") if x)
    if args.no_big:
        legs.discard("big")
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the KDA path here is built and measured on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import synth
    import linear_attention_sequence_gate_amd as kda

    kda.lib()
    dev = "cuda"
    stream = torch.cuda.current_stream()

    # ------------------------------------------------------------ prefill leg
    wl = synth.PREFILL_8K
    T, H, dk, dv = wl.T_total, wl.H, wl.dk, wl.dv
    A = torch.from_numpy(synth.gate_A(wl)).to(dev)
    sets = []
    for si in range(3):
        x = {n: synth.token_rows(wl, n, 0, T, set_index=si) for n in ("q", "k", "v", "z", "beta")}
        d = {n: torch.from_numpy(x[n]).to(dev).to(torch.bfloat16) for n in x}
        d["g"] = torch.empty_like(d["z"])
        d["o"] = torch.empty((T, H, dv), dtype=torch.bfloat16, device=dev)
        d["S"] = torch.empty((1, H, dk, dv), dtype=torch.float32, device=dev)
        sets.append(d)
    wbytes = kda.kda_prefill_workspace_size(T, 1, H, dk, dv)
    ws = torch.empty(max(wbytes, 1), dtype=torch.uint8, device=dev)

    def step(i):  # one call: the gate fused into the prefill's decay stage
        d = sets[i % 3]
        kda.kda_prefill_gated(d["q"], d["k"], d["v"], d["z"], A, d["beta"], final_state=d["S"], o=d["o"],
                              workspace=ws)

    def prefill(i):  # the unfused prefill, on g from a separate kda_gate
        d = sets[i % 3]
        kda.kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], final_state=d["S"], o=d["o"],
                        workspace=ws)

    def step_unfused(i):
        d = sets[i % 3]
        kda.kda_gate(d["z"], A, g=d["g"])
        prefill(i)

    def timed_loop(fn, n):
        """Mean ms per call of n back-to-back calls fn(i), bracketed by two events
        on the stream the library launches on (no event between calls)."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # bring the GPU to its steady clocks first (untimed): a fresh device runs
    # the first few hundred microsecond-scale launches at ramping clocks.  The
    # clock starts after a first call has finished, which also loads the
    # library's kernels (that can take longer than the whole spin-up).
    step(0)
    torch.cuda.synchronize()
    # the checksum every later run must reproduce, taken on the host: a device-side
    # reduction here allocates and slowed the next hundred or so calls
    ref_sum = float(sets[0]["o"].cpu().float().abs().sum())
    spin_end = time.perf_counter() + args.spin_up
    i = 0
    while time.perf_counter() < spin_end:
        for _ in range(20):
            step(i)
            i += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms_step = timed_loop(step, args.steps)  # the timed region: K whole steps
    wall = time.perf_counter() - t0
    total_ms = ms_step * args.steps
    # the timed runs produce the verified run's result (no caching, same inputs)
    step(0)
    torch.cuda.synchronize()
    o_host = sets[0]["o"].cpu().float()
    assert abs(float(o_host.abs().sum()) - ref_sum) <= 1e-6 * max(ref_sum, 1.0)
    o_timed = o_host.numpy()
    S_timed = sets[0]["S"].cpu().numpy()
    # the same work as separate launches: kda_gate (g through HBM) then kda_prefill
    for i in range(args.warmup):
        step_unfused(i)
    unfused_ms = timed_loop(step_unfused, args.steps)
    prefill_ms = timed_loop(prefill, args.steps)
    unfused = {"ms_per_step": round(unfused_ms, 4), "kda_prefill_ms_per_call": round(prefill_ms, 4),
               "value": round(T / (unfused_ms * 1e-3), 1)}

    # the roofline's unit is the step's one call, kda_prefill_gated
    p_bytes, p_flops = prefill_algo(T, H, dk, dv)
    achieved = p_bytes / (ms_step * 1e-3) / 1e9
    traffic = load_traffic("prefill_8k")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "kda_prefill_gated: prefill_warm_kernel (segments with warm-up windows, gate in the "
                          "decay stage) + the flag-gated exact passes, which end at once here",
                "algorithmic_bytes_per_call": p_bytes, "ms_per_call": round(ms_step, 4),
                "mfma_tflops": round(p_flops / (ms_step * 1e-3) / 1e12, 1),
                "mfma_frac": round(p_flops / (ms_step * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)}

    # prefill with state checkpoints every 512 tokens (prefix-cache emission)
    n_ck = kda.kda_checkpoint_count(None, T, 512)
    ck = torch.empty((n_ck, H, dk, dv), dtype=torch.float32, device=dev)
    def prefill_ckpt(i):
        d = sets[i % 3]
        kda.kda_prefill_gated(d["q"], d["k"], d["v"], d["z"], A, d["beta"], final_state=d["S"], o=d["o"],
                              workspace=ws, interval=512, ckpt=ck)

    for i in range(args.warmup):
        prefill_ckpt(i)
    ck_ms = timed_loop(prefill_ckpt, args.steps)
    ckpt_leg = {"interval": 512, "checkpoints_per_call": n_ck * H, "ms_per_call": round(ck_ms, 4),
                "overhead_vs_plain": round(ck_ms / ms_step - 1.0, 4),
                "checkpoint_bytes_per_call": n_ck * H * dk * dv * 4}

    decode = spec = backward = None
    roofs, big = {}, {}
    rw_gbs = None
    if "decode" in legs:
        # ------------------------------------------------------------- decode leg
        dwl = synth.DECODE_B256
        B = dwl.N
        dA = torch.from_numpy(synth.gate_A(dwl)).to(dev)
        dsets = []
        for si in range(8):
            x = {n: synth.token_rows(dwl, n, 0, B, set_index=si) for n in ("q", "k", "v", "z", "beta")}
            d = {n: torch.from_numpy(x[n]).to(dev).to(torch.bfloat16) for n in x}
            d["g"] = torch.empty_like(d["z"])
            dsets.append(d)
        state = torch.from_numpy(synth.initial_state(dwl)).to(dev)
        dout = torch.empty((B, dwl.H, dwl.dv), dtype=torch.bfloat16, device=dev)

        def dstep(i):  # one call: the gate fused into the decode step
            d = dsets[i % 8]
            kda.kda_decode_step_gated(d["q"], d["k"], d["v"], d["z"], dA, d["beta"], state, o=dout)

        def dstep_unfused(i):
            d = dsets[i % 8]
            kda.kda_gate(d["z"], dA, g=d["g"])
            kda.kda_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state, o=dout)

        for i in range(16):
            dstep(i)
        d_total_ms = timed_loop(dstep, args.decode_steps) * args.decode_steps
        d_kernel_ms = d_total_ms / args.decode_steps  # the step is the one launch
        for i in range(16):
            dstep_unfused(i)
        d_unfused_ms = timed_loop(dstep_unfused, args.decode_steps)
        # the same step over a 4 GiB state (B = 2048), far past the 256 MB
        # last-level cache, which holds part of the 512 MiB state above from
        # one step to the next: its rate is compared with the 4 GiB
        # state-update roof
        B4 = 2048
        g4 = torch.Generator(device=dev).manual_seed(dwl.seed + 1)
        x4 = {}
        for n in ("q", "k", "v", "z"):
            t = torch.randn((B4, dwl.H, dwl.dk), generator=g4, device=dev)
            x4[n] = (t / t.norm(dim=-1, keepdim=True) if n in ("q", "k") else t).to(torch.bfloat16)
        b4 = torch.sigmoid(torch.randn((B4, dwl.H), generator=g4, device=dev)).to(torch.bfloat16)
        s4 = torch.randn((B4, dwl.H, dwl.dk, dwl.dv), generator=g4, device=dev) * 0.05
        o4 = torch.empty((B4, dwl.H, dwl.dv), dtype=torch.bfloat16, device=dev)

        def dstep4(i):
            kda.kda_decode_step_gated(x4["q"], x4["k"], x4["v"], x4["z"], dA, b4, s4, o=o4)

        for i in range(3):
            dstep4(i)
        d4_ms = timed_loop(dstep4, 20)
        d4_bytes, _ = decode_algo(B4, dwl.H, dwl.dk, dwl.dv)
        del x4, b4, s4, o4
        d_bytes, d_flops = decode_algo(B, dwl.H, dwl.dk, dwl.dv)
        d_ach = d_bytes / (d_kernel_ms * 1e-3) / 1e9
        decode = {"value": round(B * args.decode_steps / (d_total_ms * 1e-3), 1), "unit": "tokens/s",
                  "steps": args.decode_steps, "ms_per_step": round(d_total_ms / args.decode_steps, 4),
                  "config": {"workload": "decode_b256", "B": B, "H": dwl.H, "d_k": dwl.dk,
                             "d_v": dwl.dv, "input_sets": 8},
                  "roofline": {"bound": "hbm", "achieved": round(d_ach, 1), "peak": HBM_PEAK_GBS,
                               "unit": "GB/s", "frac": round(d_ach / HBM_PEAK_GBS, 4),
                               "traffic": load_traffic("decode_b256"),
                               "kernel": "step_wave_kernel (kda_decode_step_gated)",
                               "algorithmic_bytes_per_call": d_bytes,
                               "ms_per_call": round(d_kernel_ms, 4)},
                  "unfused": {"ms_per_step": round(d_unfused_ms, 4),
                              "value": round(B / (d_unfused_ms * 1e-3), 1)},
                  "state_4gib": {"B": B4, "ms_per_call": round(d4_ms, 4), "algorithmic_bytes_per_call": d4_bytes,
                                 "achieved_gbs": round(d4_bytes / (d4_ms * 1e-3) / 1e9, 1)}}

    if "speculative" in legs:
        # ------------------------------------------- speculative decode leg (K = 4)
        swl = synth.VERIFY_B256_K4
        K = swl.seqlens[0]
        SB = swl.N
        sA = torch.from_numpy(synth.gate_A(swl)).to(dev)
        ssets = []
        for si in range(4):
            x = {n: synth.token_rows(swl, n, 0, SB * K, set_index=si) for n in ("q", "k", "v", "z", "beta")}
            d = {n: torch.from_numpy(x[n]).to(dev).to(torch.bfloat16) for n in x}
            d["g"] = kda.kda_gate(d["z"], sA)
            d = {n: t.reshape((SB, K) + tuple(t.shape[1:])) for n, t in d.items()}
            ssets.append(d)
        sstate = torch.from_numpy(synth.initial_state(swl.with_(seqlens=(1,) * SB))).to(dev)
        sout = torch.empty((SB, K, swl.H, swl.dv), dtype=torch.bfloat16, device=dev)
        n_all = torch.full((SB,), K, dtype=torch.int32, device=dev)
        spec_iters = 200
        for i in range(5):
            d = ssets[i % 4]
            kda.kda_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], sstate, o=sout)
            kda.kda_commit(d["k"], d["v"], d["g"], d["beta"], n_all, sstate)
        torch.cuda.synchronize()

        def vcall(i):
            d = ssets[i % 4]
            kda.kda_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], sstate, o=sout)

        def ccall(i):
            d = ssets[i % 4]
            kda.kda_commit(d["k"], d["v"], d["g"], d["beta"], n_all, sstate)

        v_ms = timed_loop(vcall, spec_iters)
        c_ms = timed_loop(ccall, spec_iters)
        vb = spec_algo(SB, K, swl.H, swl.dk, swl.dv, False)
        cb = spec_algo(SB, K, swl.H, swl.dk, swl.dv, True)
        spec = {"value": round(SB * K / ((v_ms + c_ms) * 1e-3), 1), "unit": "draft tokens/s (verify + commit)",
                "config": {"workload": "verify_b256_k4", "B": SB, "K": K, "H": swl.H, "d_k": swl.dk,
                           "d_v": swl.dv, "n_accept": K, "input_sets": 4},
                "verify": {"ms_per_call": round(v_ms, 4),
                           "roofline": {"bound": "hbm", "achieved": round(vb / (v_ms * 1e-3) / 1e9, 1),
                                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                        "frac": round(vb / (v_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                        "traffic": load_traffic("verify_b256_k4"), "kernel": "verify_wave_kernel",
                                        "algorithmic_bytes_per_call": vb}},
                "commit": {"ms_per_call": round(c_ms, 4),
                           "roofline": {"bound": "hbm", "achieved": round(cb / (c_ms * 1e-3) / 1e9, 1),
                                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                        "frac": round(cb / (c_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                        "traffic": load_traffic("commit_b256_k4"), "kernel": "step_wave_kernel (commit)",
                                        "algorithmic_bytes_per_call": cb}}}

    if "backward" in legs:
        # ------------------------------------------- backward leg (8K workload)
        # the forward's interval-64 checkpoints and g come from untimed calls; one
        # kda_backward call (summary, scan and full pass) is timed per step
        bsets = sets[0]
        bg = torch.empty_like(bsets["z"])
        kda.kda_gate(bsets["z"], A, g=bg)
        _, _, bck = kda.kda_prefill_ckpt(bsets["q"], bsets["k"], bsets["v"], bg, bsets["beta"], 64)
        gen = torch.Generator(device=dev).manual_seed(7)
        bdo = torch.randn((T, H, dv), device=dev, generator=gen).to(torch.bfloat16)
        bdfin = torch.randn((1, H, dk, dv), device=dev, generator=gen)
        bws = torch.empty(kda.lib().kda_backward_workspace_size(T, 1, H, dk, dv), dtype=torch.uint8, device=dev)

        def bcall(i):
            kda.kda_backward(bsets["q"], bsets["k"], bsets["v"], bg, bsets["beta"], d_o=bdo, d_final_state=bdfin,
                             ckpt=bck, interval=64, workspace=bws)

        bcall(0)
        b_ms = timed_loop(bcall, 3)
        b_bytes = backward_algo(T, H, dk, dv)
        backward = {"value": round(T / (b_ms * 1e-3), 1), "unit": "tokens/s", "ms_per_call": round(b_ms, 3),
                    "config": {"workload": "prefill_8k backward (dq, dk, dv, dg, dbeta, dS0) from interval-64 "
                                           "checkpoints", "H": H, "T": T, "d_k": dk, "d_v": dv},
                    "roofline": {"bound": "hbm", "achieved": round(b_bytes / (b_ms * 1e-3) / 1e9, 1),
                                 "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": round(b_bytes / (b_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 5),
                                 "kernel": "bwd_chunk_summary_kernel (windows) + flag-gated summary and scan + bwd_chunk_full_kernel",
                                 "traffic": load_traffic("backward_8k"),
                                 "algorithmic_bytes_per_call": b_bytes}}
        del bws, bck

    if "roofs" in legs:
        # the device's own roofs: streaming read / write / copy / in-place kernels over 4 GiB
        # (far past the 256 MB last-level cache) and back-to-back 16x16x32 bf16
        # matrix-core instructions on every SIMD (libkda_roofs)
        roofs = measured_roofs(torch, dev, stream)
        rw_gbs = roofs["hbm_rw_gbs"]
        for r in (roofline, decode and decode["roofline"], spec and spec["verify"]["roofline"],
                  spec and spec["commit"]["roofline"], backward and backward["roofline"]):
            if r is None:
                continue
            r["measured_rw_gbs"] = round(rw_gbs, 1)
            r["frac_of_measured_rw"] = round(r["achieved"] / rw_gbs, 4)
        # decode and commit update a 512 MiB state in place: against the same
        # update over the same working set (part of it cache-resident), and
        # decode over 4 GiB against the 4 GiB state update
        same = roofs["inplace_state_512mib_gbs"]
        for r in (decode and decode["roofline"], spec and spec["commit"]["roofline"]):
            if r is not None:
                r["measured_rw_same_working_set_gbs"] = same
                r["frac_of_measured_rw_same_working_set"] = round(r["achieved"] / same, 4)
        if decode is not None:
            d4 = decode["state_4gib"]
            d4["measured_state_rw_gbs"] = roofs["hbm_inplace_state_gbs"]
            d4["frac_of_measured_state_rw"] = round(d4["achieved_gbs"] / roofs["hbm_inplace_state_gbs"], 4)
            d4["frac"] = round(d4["achieved_gbs"] / HBM_PEAK_GBS, 4)
        roofline["measured_mfma_bf16_tflops"] = roofs["mfma_bf16_tflops"]
        roofline["mfma_frac_of_measured_mfma"] = round(roofline["mfma_tflops"] / roofs["mfma_bf16_tflops"], 4)
        # a plain 8192^3 bf16 GEMM through the vendor library, for reference
        ga = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
        gb = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
        gc = torch.empty(8192, 8192, device=dev, dtype=torch.bfloat16)
        for _ in range(3):
            torch.mm(ga, gb, out=gc)
        gemm_ms = timed_loop(lambda i: torch.mm(ga, gb, out=gc), 10)
        gemm_tflops = 2.0 * 8192 ** 3 / (gemm_ms * 1e-3) / 1e12
        del ga, gb, gc
        roofs["vendor_gemm_bf16_tflops"] = round(gemm_tflops, 1)

    f32 = None
    if "f32" in legs:
        # ------------------------------------------- fp32 tensors at the 8K shape
        # (d_k = d_v = 128 in fp32: the token-serial path, segments with warm-up
        # windows), one kda_prefill_gated call per step; two heads against the oracle
        import numpy as np
        import oracle
        fw = synth.PREFILL_8K.with_(dtype="f32")
        fx = {n: torch.from_numpy(synth.token_rows(fw, n, 0, T)).to(dev) for n in ("q", "k", "v", "z", "beta")}
        fA = torch.from_numpy(synth.gate_A(fw)).to(dev)
        fo = torch.empty((T, H, dv), dtype=torch.float32, device=dev)
        fS = torch.empty((1, H, dk, dv), dtype=torch.float32, device=dev)
        fws = torch.empty(kda.kda_prefill_workspace_size(T, 1, H, dk, dv, dtype=kda.KDA_F32), dtype=torch.uint8,
                          device=dev)

        def fcall(i):
            kda.kda_prefill_gated(fx["q"], fx["k"], fx["v"], fx["z"], fA, fx["beta"], final_state=fS, o=fo,
                                  workspace=fws)

        for i in range(2):
            fcall(i)
        f_ms = timed_loop(fcall, 10)
        heads = [1, H - 2]
        hx = {n: fx[n][:, heads].cpu().numpy() for n in fx}
        fo_ref, fS_ref = oracle.prefill(hx["q"], hx["k"], hx["v"], oracle.gate(hx["z"], synth.gate_A(fw)[heads]),
                                        hx["beta"])
        f_bytes = T * H * ((3 * dk + dv + 1) * 4 + dv * 4) + H * dk * dv * 4
        f32 = {"value": round(T / (f_ms * 1e-3), 1), "unit": "tokens/s", "ms_per_call": round(f_ms, 4),
               "config": {"workload": "prefill_8k shape with fp32 tensors (token-serial path)", "H": H, "T": T,
                          "d_k": dk, "d_v": dv},
               "achieved_gbs": round(f_bytes / (f_ms * 1e-3) / 1e9, 1), "bound": "latency (token-serial VALU chain)",
               "verified": {"against": f"fp64 oracle, heads {heads}, whole sequence",
                            "o_max_rel_err": max_rel_err(fo[:, heads].cpu().numpy(), fo_ref),
                            "final_state_max_rel_err": max_rel_err(fS[0, heads].cpu().numpy(), fS_ref[0]),
                            "tolerance": 1e-4}}
        del fx, fo, fws

    # ------------------------------------------- million-token workloads
    if "big" in legs:
        big["prefill_1m"] = big_leg(kda, torch, synth, synth.PREFILL_1M, dev, stream, timed_loop, rw_gbs, 1.34)
        big["varlen_64"] = big_leg(kda, torch, synth, synth.VARLEN_64, dev, stream, timed_loop, rw_gbs, 5.1)

    if args.copy_calib:  # plain copy of known size, for the HBM counter calibration
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    cpu, verified = None, None
    if not args.no_cpu:
        cpu, (o_ref, S_ref) = cpu_baseline(wl)
        verified = {"against": "fp64 oracle on input set 0 (bf16-rounded inputs), whole workload",
                    "o_max_rel_err": max_rel_err(o_timed, o_ref),
                    "final_state_max_rel_err": max_rel_err(S_timed, S_ref), "tolerance": 2e-2}
    tok_s = T * args.steps / (total_ms * 1e-3)
    out = {"metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": "prefill_8k: gate + chunked prefill in one kda_prefill_gated call, "
                                  "B=1 H=32 T=8192 d_k=d_v=128 chunk=64, zero initial state",
                      "B": 1, "H": H, "T": T, "d_k": dk, "d_v": dv, "chunk": 64, "input_sets": 3},
           "roofline": roofline, "cpu_baseline": cpu, "verified": verified, "unfused": unfused,
           "checkpoints": ckpt_leg,
           "decode": decode,
           "speculative": spec, "backward": backward, "f32_prefill": f32, "million_token": big,
           "measured_roofs": roofs,
           "wall_s": round(wall, 3), "source_hash": kernel_source_hash()}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
