"""GPU parity at full size on the three large workloads, every output and state
against the fp64 oracle:
  - prefill_1m (H=8, T=2^20, z shifted by +3): every head, all 2^20 outputs and
    the final state;
  - varlen_64 (64 sequences, ~1.03M tokens, H=32, initial states N(0, 0.01)):
    every sequence x head, outputs and final states;
  - decode_b256 (B=256, H=32, 1000 consecutive in-place steps over 8 input
    sets): all 8192 states after the last step and the last step's outputs.
The oracle runs token-serially in fp64 on the host, streamed window by window
with its state carried across windows, and compares each window as it goes.
The 1000 decode steps of a state are replayed as one 1000-token oracle prefill
(T decode steps equal a T-token prefill: a pin of the oracle).  The oracle is
compiled for the host the tests run on.  varlen_64 runs the fused gate
(kda_prefill_gated, the benchmark's call) at full size; kda_gate + kda_prefill
run the same block kernels and are checked whole on prefill_1m and at smaller
sizes elsewhere.

The error measure is the normwise max relative error, max|x - y| / max|y|,
taken per head (prefill_1m), per (sequence, head) (varlen_64) and per (b, h)
state (decode), so a head or sequence with small values cannot hide behind the
others; every one must meet the bf16 bar."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import TOL, announce, dev, dev_stream, host, native_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    import torch
    import linear_attention_sequence_gate_amd as m
    assert torch.cuda.is_available()
    m.lib()
    return m


def gpu_prefill(kda, xs, A, gated, **kw):
    """kda_gate + kda_prefill, or the fused kda_prefill_gated, on device tensors."""
    if gated:
        return kda.kda_prefill_gated(xs["q"], xs["k"], xs["v"], xs["z"], A, xs["beta"], **kw)
    g = kda.kda_gate(xs["z"], A)
    del xs["z"]
    return kda.kda_prefill(xs["q"], xs["k"], xs["v"], g, xs["beta"], **kw)


class NormwiseMax:
    """Running max|x - y| and max|y| per unit, over windows of one unit's values."""

    def __init__(self, shape):
        self.num = np.zeros(shape)
        self.den = np.zeros(shape)

    def add(self, got, want, axis):
        d = np.abs(np.asarray(got, np.float64) - want)
        assert np.all(np.isfinite(got)), "non-finite values from the GPU"
        self.num = np.maximum(self.num, d.max(axis=axis))
        self.den = np.maximum(self.den, np.abs(want).max(axis=axis))

    def err(self):
        return self.num / np.maximum(self.den, 1e-300)


def stream_sequence(wl, o, gated, a, b, S0, window, o_acc, idx):
    """The oracle over tokens [a, b) of the packed input, `window` tokens at a
    time, each window's outputs compared with the GPU's as it goes (per head,
    into o_acc[idx]).  Returns the oracle's final state [H, dk, dv]."""
    A = synth.gate_A(wl)
    S = S0[None]
    for w0 in range(a, b, window):
        w1 = min(b, w0 + window)
        x = {n: synth.token_rows(wl, n, w0, w1) for n in ("q", "k", "v", "z", "beta")}
        lib = native_oracle()
        g = oracle.gate(x["z"], A, round_bf16=not gated, lib=lib)  # the fused gate keeps g in fp32
        o_ref, S = oracle.prefill(x["q"], x["k"], x["v"], g, x["beta"], S0=S, lib=lib)
        num, den = o_acc
        got = host(o[w0:w1])
        sub = NormwiseMax(wl.H)
        sub.add(got, o_ref, axis=(0, 2))
        num[idx] = np.maximum(num[idx], sub.num)
        den[idx] = np.maximum(den[idx], sub.den)
    return S[0]


def report(name, err, tol):
    flat = err.ravel()
    worst = np.unravel_index(np.argmax(err), err.shape)
    print(f"  {name}: max {flat.max():.3e} at {tuple(int(i) for i in worst)}, median {np.median(flat):.3e}, "
          f"{flat.size} units, {int(np.sum(flat >= tol))} at or above {tol}")
    assert flat.max() < tol, f"{name}: worst {flat.max():.3e}"


@pytest.mark.parametrize("gated", [False, True])
def test_prefill_1m_every_head(kda, gated):
    import torch
    wl = synth.PREFILL_1M
    T, H = wl.T_total, wl.H
    announce(f"prefill_1m full size, every head: H={H} T={T} gated={gated}")
    xs = {n: dev_stream(wl, n) for n in ("q", "k", "v", "z", "beta")}
    o, S = gpu_prefill(kda, xs, dev(synth.gate_A(wl)), gated)
    del xs
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(S).all()
    num, den = np.zeros((1, H)), np.zeros((1, H))
    S_ref = stream_sequence(wl, o, gated, 0, T, np.zeros((H, wl.dk, wl.dv)), 1 << 16, (num, den), 0)
    report("o per head", num[0] / den[0], TOL["bf16"])
    es = NormwiseMax(H)
    es.add(host(S[0]), S_ref, axis=(1, 2))
    report("final state per head", es.err(), TOL["bf16"])


@pytest.mark.parametrize("gated", [True])
def test_varlen_64_every_sequence(kda, gated):
    import torch
    wl = synth.VARLEN_64
    T, H, N = wl.T_total, wl.H, wl.N
    cu = wl.cu_seqlens
    announce(f"varlen_64 full size, every sequence x head: N={N} H={H} T={T} gated={gated}")
    xs = {n: dev_stream(wl, n, rows=1 << 14) for n in ("q", "k", "v", "z", "beta")}
    S0 = synth.initial_state(wl)
    o, S = gpu_prefill(kda, xs, dev(synth.gate_A(wl)), gated, cu_seqlens=torch.from_numpy(cu).cuda(),
                       initial_state=dev(S0))
    del xs
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(S).all()
    num, den = np.zeros((N, H)), np.zeros((N, H))
    es = NormwiseMax((N, H))
    S_gpu = host(S)
    for n in range(N):
        S_ref = stream_sequence(wl, o, gated, int(cu[n]), int(cu[n + 1]), S0[n], 1 << 16, (num, den), n)
        es.num[n] = np.abs(S_gpu[n] - S_ref).max(axis=(1, 2))
        es.den[n] = np.abs(S_ref).max(axis=(1, 2))
    report("o per (sequence, head)", num / den, TOL["bf16"])
    report("final state per (sequence, head)", es.err(), TOL["bf16"])


def _decode_sets(wl, nsets, B):
    return [{n: synth.token_rows(wl, n, 0, B, set_index=s) for n in ("q", "k", "v", "z", "beta")}
            for s in range(nsets)]


@pytest.mark.parametrize("gated", [False, True])
def test_decode_1000_steps_every_state(kda, gated):
    """1000 consecutive in-place steps at B=256, H=32, inputs cycling through 8
    seeded sets; every (b, h) state and its last output against 1000-token
    oracle prefills (32 sequences at a time)."""
    import torch
    wl = synth.DECODE_B256
    B, H, dk, dv = wl.N, wl.H, wl.dk, wl.dv
    steps, nsets = 1000, 8
    announce(f"decode B=256 H=32, 1000 steps, every state, gated={gated}")
    A = synth.gate_A(wl)
    S0 = synth.initial_state(wl)
    sets = _decode_sets(wl, nsets, B)
    Ad = dev(A)
    dsets = []
    for x in sets:
        d = {n: dev(x[n], "bf16") for n in ("q", "k", "v", "z", "beta")}
        d["g"] = kda.kda_gate(d["z"], Ad)
        dsets.append(d)
    St = dev(S0)
    o = torch.empty((B, H, dv), dtype=torch.bfloat16, device="cuda")
    for t in range(steps):
        d = dsets[t % nsets]
        if gated:
            kda.kda_decode_step_gated(d["q"], d["k"], d["v"], d["z"], Ad, d["beta"], St, o=o)
        else:
            kda.kda_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], St, o=o)
    torch.cuda.synchronize()
    S_gpu, o_gpu = host(St), host(o)
    # the oracle's inputs: token t of every sequence comes from set t % 8
    stack = {n: np.stack([x[n] for x in sets]) for n in ("q", "k", "v", "z", "beta")}  # [8, B, H, ...]
    order = np.arange(steps) % nsets
    eo, es = NormwiseMax((B, H)), NormwiseMax((B, H))
    nb = 32
    for b0 in range(0, B, nb):
        b1 = b0 + nb

        def packed(name):  # [nb * steps, H, ...]: sequence b holds steps 0..999 of state b
            x = stack[name][order][:, b0:b1]  # [steps, nb, H, ...]
            return np.ascontiguousarray(np.swapaxes(x, 0, 1)).reshape((nb * steps,) + x.shape[2:])

        x = {n: packed(n) for n in ("q", "k", "v", "z", "beta")}
        lib = native_oracle()
        g = oracle.gate(x["z"], A, round_bf16=not gated, lib=lib)
        cu = np.arange(0, nb * steps + 1, steps, dtype=np.int64)
        o_ref, S_ref = oracle.prefill(x["q"], x["k"], x["v"], g, x["beta"], cu=cu, S0=S0[b0:b1], lib=lib)
        last = o_ref[cu[1:] - 1]  # [nb, H, dv]: each sequence's last output
        es.num[b0:b1] = np.abs(S_gpu[b0:b1] - S_ref).max(axis=(2, 3))
        es.den[b0:b1] = np.abs(S_ref).max(axis=(2, 3))
        eo.num[b0:b1] = np.abs(o_gpu[b0:b1] - last).max(axis=2)
        eo.den[b0:b1] = np.abs(last).max(axis=2)
    report("state per (b, h) after 1000 steps", es.err(), TOL["bf16"])
    report("last output per (b, h)", eo.err(), TOL["bf16"])
