"""GPU parity of the prefill's warm-up pass: every segment of a long sequence
takes its incoming state from a window of tokens before it, run from a zero
state beside the window's transition M; when the computed M is exactly zero
the segment runs on, else its chain is flagged and the exact summary / scan /
output passes redo it.  Outputs, final states and checkpoints against the fp64
oracle, with the path each chain took read from the call's workspace."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import TOL, announce, dev, host, relerr

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    import torch
    import linear_attention_sequence_gate_amd as m
    assert torch.cuda.is_available()
    m.lib()
    return m


def inputs(wl, g_shift_heads=None):
    """Seeded inputs and the oracle's g (rounded to the storage dtype, as
    kda_gate returns it).  g_shift_heads: heads whose g comes from z - 4 (weak
    decay: their warm-up transition does not vanish)."""
    x = synth.prefill_inputs(wl)
    z = x["z"].copy()
    if g_shift_heads:
        z[:, g_shift_heads] -= 4.0
    g = oracle.gate(z, x["A"], round_bf16=(wl.dtype == "bf16"))
    S0 = synth.initial_state(wl) if wl.state_std > 0 else None
    return x, g, S0


def run(kda, wl, x, g, S0, seg=0, warm=-1, interval=0):
    d = {n: dev(x[n], wl.dtype) for n in ("q", "k", "v", "beta")}
    o, S, ck, ws = kda.kda_test_prefill(d["q"], d["k"], d["v"], dev(g, wl.dtype), d["beta"],
                                        initial_state=None if S0 is None else dev(S0), seg_chunks=seg,
                                        warm_tokens=warm, interval=interval)
    flags = kda.test_prefill_flags(ws, wl.T_total, 1, wl.H, wl.dk, wl.dv, 1 if wl.dtype == "bf16" else 0,
                                   seg, warm)
    return o, S, ck, flags


def nseg_of(T, L):
    return max(1, -(-T // (64 * L)))


def check(o, S, wl, x, g, S0):
    o_ref, S_ref = oracle.prefill(x["q"], x["k"], x["v"], g, x["beta"], S0=S0)
    eo, es = relerr(host(o), o_ref), relerr(host(S), S_ref)
    print(f"  o {eo:.3e}  S {es:.3e}")
    tol = TOL[wl.dtype]
    assert eo < tol and es < tol


@pytest.mark.parametrize("T", [2048, 2000, 4160])
def test_warm_outputs(kda, T):
    """Strong decay (the workloads' gate): every window's transition vanishes,
    so no chain is redone.  Lengths with a partial last chunk and more than two
    segments."""
    wl = synth.PREFILL_8K.with_(H=4, seqlens=(T,), state_std=0.1)
    announce(f"warm-up pass T={T} H={wl.H}")
    x, g, S0 = inputs(wl)
    o, S, _, flags = run(kda, wl, x, g, S0, seg=16)
    n = nseg_of(T, 16)
    assert n >= 2
    assert int(flags[:n].sum()) == 0, f"warm-up fell back: {host(flags[:n])}"
    check(o, S, wl, x, g, S0)


def test_warm_weak_decay_falls_back(kda):
    """z shifted by -4 on every head: the windows' transitions stay non-zero,
    every chain is flagged and redone by the exact passes."""
    wl = synth.PREFILL_8K.with_(H=4, seqlens=(2048,), state_std=0.1)
    announce("warm-up pass, weak decay: exact passes")
    x, g, S0 = inputs(wl, g_shift_heads=[0, 1, 2, 3])
    o, S, _, flags = run(kda, wl, x, g, S0, seg=8)
    n = nseg_of(2048, 8)
    assert np.all(host(flags[1:n]).sum(axis=0) > 0), "expected every chain flagged"
    check(o, S, wl, x, g, S0)


def test_warm_mixed_heads(kda):
    """Heads 1 and 3 decay weakly: only their chains are redone; heads 0 and 2
    keep the warm-up pass's results.  Every head against the oracle."""
    wl = synth.PREFILL_8K.with_(H=4, seqlens=(3000,), state_std=0.1)
    announce("warm-up pass, mixed heads")
    x, g, S0 = inputs(wl, g_shift_heads=[1, 3])
    o, S, _, flags = run(kda, wl, x, g, S0, seg=8)
    n = nseg_of(3000, 8)
    per_head = host(flags[:n]).sum(axis=0)
    assert per_head[0] == 0 and per_head[2] == 0, per_head
    assert per_head[1] > 0 and per_head[3] > 0, per_head
    check(o, S, wl, x, g, S0)


@pytest.mark.parametrize("warm", [32, 64, 96, 256])
def test_warm_window_lengths(kda, warm):
    """Windows from one block to four chunks (a 32-token window is too short
    for some chains: those are redone); segments of two chunks, so windows
    also reach back past the previous segment and to the sequence start."""
    wl = synth.PREFILL_8K.with_(H=4, dk=64, dv=64, seqlens=(1500,), state_std=0.1)
    announce(f"warm-up window {warm}")
    x, g, S0 = inputs(wl)
    o, S, _, flags = run(kda, wl, x, g, S0, seg=2, warm=warm)
    print(f"  chains redone: {int((host(flags[:nseg_of(1500, 2)]).sum(axis=0) > 0).sum())} of {wl.H}")
    check(o, S, wl, x, g, S0)


def test_warm_matches_exact_passes(kda):
    """The warm-up pass and the exact passes alone (warm = 0) both land on the
    oracle and agree with each other to the bf16 bar."""
    wl = synth.PREFILL_8K.with_(H=4, seqlens=(2048,), state_std=0.1)
    announce("warm-up pass against the exact passes")
    x, g, S0 = inputs(wl)
    o1, S1, _, _ = run(kda, wl, x, g, S0, seg=4)
    o2, S2, _, flags = run(kda, wl, x, g, S0, seg=4, warm=0)
    assert flags is None
    check(o1, S1, wl, x, g, S0)
    check(o2, S2, wl, x, g, S0)
    assert relerr(host(o1), host(o2)) < TOL["bf16"]


def test_warm_f32(kda):
    """fp32 tensors (d_k = d_v = 32) through the warm-up pass."""
    wl = synth.TINY_F32.with_(H=2, seqlens=(2048,), state_std=0.1)
    announce("warm-up pass, fp32")
    x, g, S0 = inputs(wl)
    o, S, _, flags = run(kda, wl, x, g, S0, seg=8)
    assert int(flags[:nseg_of(2048, 8)].sum()) == 0
    check(o, S, wl, x, g, S0)


@pytest.mark.parametrize("interval", [64, 512, 384])
def test_warm_checkpoints(kda, interval):
    """Checkpoints come from the segments' own blocks, never from the warm-up
    windows: every row against the oracle state at that token."""
    wl = synth.PREFILL_8K.with_(H=4, seqlens=(2048,), state_std=0.1)
    announce(f"warm-up pass, checkpoints every {interval}")
    x, g, S0 = inputs(wl)
    o, S, ck, flags = run(kda, wl, x, g, S0, seg=4, interval=interval)
    assert int(flags[:nseg_of(2048, 4)].sum()) == 0
    T = wl.T_total
    rows = []
    Sr = S0
    for j in range(T // interval):
        r = slice(j * interval, (j + 1) * interval)
        _, Sr = oracle.prefill(x["q"][r], x["k"][r], x["v"][r], g[r], x["beta"][r], S0=Sr)
        rows.append(Sr[0])
    e = relerr(host(ck), np.array(rows))
    print(f"  {len(rows)} checkpoints {e:.3e}")
    assert e < TOL["bf16"]
    check(o, S, wl, x, g, S0)


def test_warm_in_place_state_and_gate(kda):
    """initial_state == final_state (in place) through the fused gate."""
    import torch
    wl = synth.PREFILL_8K.with_(H=4, seqlens=(2048,), state_std=0.1)
    announce("warm-up pass, in-place state, fused gate")
    x = synth.prefill_inputs(wl)
    S0 = synth.initial_state(wl)
    d = {n: dev(x[n], wl.dtype) for n in ("q", "k", "v", "z", "beta")}
    st = dev(S0)
    o, _ = kda.kda_prefill_gated(d["q"], d["k"], d["v"], d["z"], dev(x["A"]), d["beta"],
                                 initial_state=st, final_state=st)
    torch.cuda.synchronize()
    g = oracle.gate(x["z"], x["A"])  # the fused gate keeps g in fp32
    o_ref, S_ref = oracle.prefill(x["q"], x["k"], x["v"], g, x["beta"], S0=S0)
    assert relerr(host(o), o_ref) < TOL["bf16"] and relerr(host(st), S_ref) < TOL["bf16"]


@pytest.mark.parametrize("weak", [False, True])
def test_two_streams(kda, weak):
    """Two calls in flight on two user streams, each with its own workspace:
    each result equals the same call run alone (the library keeps nothing
    between calls)."""
    import torch
    wl = synth.PREFILL_8K.with_(H=4, seqlens=(2048,), state_std=0.1)
    announce(f"two calls on two streams, weak={weak}")
    x, g, S0 = inputs(wl, g_shift_heads=[0, 2] if weak else None)
    d = {n: dev(x[n], wl.dtype) for n in ("q", "k", "v", "beta")}
    gd = dev(g, wl.dtype)
    o_ref, S_ref = kda.kda_prefill(d["q"], d["k"], d["v"], gd, d["beta"], initial_state=dev(S0))
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for st in (s1, s2):
        with torch.cuda.stream(st):
            outs.append(kda.kda_prefill(d["q"], d["k"], d["v"], gd, d["beta"], initial_state=dev(S0),
                                        stream=st))
    torch.cuda.synchronize()
    for o, S in outs:
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref)


@pytest.mark.parametrize("weak", [False, True])
def test_graph_replay(kda, weak):
    """The whole call (warm-up pass, then the flag-gated exact passes; with
    weak decay on two heads they do run) captured into a HIP graph and replayed
    three times, with eager work and synchronisation between replays: every
    replay equals the eager call."""
    import torch
    wl = synth.PREFILL_8K.with_(H=4, seqlens=(2048,), state_std=0.1)
    announce(f"graph capture and replay, weak={weak}")
    x, g, S0 = inputs(wl, g_shift_heads=[1, 2] if weak else None)
    d = {n: dev(x[n], wl.dtype) for n in ("q", "k", "v", "beta")}
    gd = dev(g, wl.dtype)
    T, H = wl.T_total, wl.H
    init = dev(S0)
    o_ref, S_ref = kda.kda_prefill(d["q"], d["k"], d["v"], gd, d["beta"], initial_state=init)
    o = torch.empty_like(o_ref)
    S = torch.empty_like(S_ref)
    ws = torch.empty(kda.lib().kda_prefill_workspace_size(T, 1, H, wl.dk, wl.dv, 64, 1), dtype=torch.uint8,
                     device="cuda")
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):  # warm up on the capture stream
        kda.kda_prefill(d["q"], d["k"], d["v"], gd, d["beta"], initial_state=init, final_state=S, o=o,
                        workspace=ws, stream=st)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        kda.kda_prefill(d["q"], d["k"], d["v"], gd, d["beta"], initial_state=init, final_state=S, o=o,
                        workspace=ws, stream=st)
    for _ in range(3):
        o.zero_()
        S.zero_()
        ws.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 32)])
def test_serial_windows(kda, dk, dv):
    """The fp32 token-serial path cut into segments of 4 chunks with the
    default 128-token windows: under the workloads' gate no window is
    flagged; heads 1 and 2 with g from z - 4 are flagged and rerun whole."""
    wl = synth.TINY_F32.with_(H=3, dk=dk, dv=dv, seqlens=(2000,), state_std=0.1)
    announce(f"serial windows dk={dk} dv={dv}")
    x, g, S0 = inputs(wl)
    o, S, _, flags = run(kda, wl, x, g, S0, seg=4)
    n = nseg_of(2000, 4)
    assert int(host(flags[:n]).sum()) == 0, f"a window fell back: {host(flags[:n])}"
    check(o, S, wl, x, g, S0)
    x, g, S0 = inputs(wl, g_shift_heads=[1, 2])
    o, S, _, flags = run(kda, wl, x, g, S0, seg=4)
    per_head = host(flags[:n]).sum(axis=0)
    assert per_head[0] == 0 and per_head[1] > 0 and per_head[2] > 0, per_head
    check(o, S, wl, x, g, S0)


@pytest.mark.parametrize("warm", [0, 32])
def test_serial_short_or_no_windows(kda, warm):
    """warm = 0 flags every segment after the first (the chains rerun whole);
    a 32-token window falls back on the slower decay of z - 2 somewhere."""
    wl = synth.TINY_F32.with_(H=2, dk=64, dv=64, seqlens=(1100,), state_std=0.1, z_shift=-2.0)
    announce(f"serial windows of {warm} tokens")
    x, g, S0 = inputs(wl)
    o, S, _, _ = run(kda, wl, x, g, S0, seg=4, warm=warm)
    check(o, S, wl, x, g, S0)


@pytest.mark.parametrize("interval", [64, 192])
def test_serial_checkpoints_across_segments(kda, interval):
    """checkpoints written by every segment of the windowed serial path, at
    positions counted from the sequence start"""
    wl = synth.TINY_F32.with_(H=2, dk=128, dv=64, seqlens=(1500,), state_std=0.1)
    announce(f"serial checkpoints interval={interval}")
    x, g, S0 = inputs(wl)
    o, S, ck, flags = run(kda, wl, x, g, S0, seg=4, interval=interval)
    assert int(host(flags[:nseg_of(1500, 4)]).sum()) == 0
    check(o, S, wl, x, g, S0)
    St = S0
    for j in range(1500 // interval):
        r = slice(j * interval, (j + 1) * interval)
        _, St = oracle.prefill(x["q"][r], x["k"][r], x["v"][r], g[r], x["beta"][r], S0=St)
        e = relerr(host(ck[j]), St[0])
        assert e < TOL["f32"], f"checkpoint {j}: {e:.3e}"


@pytest.mark.parametrize("dk,dv,dtype", [(128, 128, "bf16"), (64, 64, "bf16"), (128, 128, "f32")])
def test_in_place_with_some_windows_failing(kda, dk, dv, dtype):
    """initial_state is final_state with segments of 4 chunks, where tokens
    256..767 decay weakly (g from z - 4): the windows inside them fail and the
    chain is composed exactly, while the last segment's window holds and that
    segment writes the final state early.  The exact composition must still
    start from the initial state, not from the final state written over it."""
    import torch
    wl = synth.PREFILL_8K.with_(H=2, dk=dk, dv=dv, dtype=dtype, seqlens=(2048,), state_std=0.1)
    announce(f"in place, windows failing in the middle, dk={dk} dv={dv} {dtype}")
    x = synth.prefill_inputs(wl)
    z = x["z"].copy()
    z[256:768] -= 4.0
    g = oracle.gate(z, x["A"], round_bf16=(dtype == "bf16"))
    S0 = synth.initial_state(wl)
    d = {n: dev(x[n], dtype) for n in ("q", "k", "v", "beta")}
    st = dev(S0)
    o, S, _, ws = kda.kda_test_prefill(d["q"], d["k"], d["v"], dev(g, dtype), d["beta"], initial_state=st,
                                       final_state=st, seg_chunks=4)
    torch.cuda.synchronize()
    flags = kda.test_prefill_flags(ws, wl.T_total, 1, wl.H, dk, dv, 1 if dtype == "bf16" else 0, 4, -1)
    per_seg = host(flags[:nseg_of(2048, 4)]).sum(axis=1)
    assert per_seg[2] > 0 and per_seg[-1] == 0, per_seg  # windows fail inside the weak part, hold at the end
    o_ref, S_ref = oracle.prefill(x["q"], x["k"], x["v"], g, x["beta"], S0=S0)
    eo, es = relerr(host(o), o_ref), relerr(host(st), S_ref)
    print(f"  o {eo:.3e}  S {es:.3e}")
    assert eo < TOL[dtype] and es < TOL[dtype]


@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("f32", 128)])
def test_in_place_packed_with_some_windows_failing(kda, dtype, dk):
    """The same over packed sequences (weak decay in the middle of the first
    one only), through cu_seqlens: each sequence's initial state is copied
    before any last segment writes its final state over it."""
    import torch
    wl = synth.VARLEN_64.with_(H=2, dk=dk, dv=dk, dtype=dtype, seqlens=(2048, 700, 0, 1300), state_std=0.1)
    announce(f"in place, packed, windows failing in the first sequence, {dtype}")
    x = synth.prefill_inputs(wl)
    z = x["z"].copy()
    z[256:768] -= 4.0
    g = oracle.gate(z, x["A"], round_bf16=(dtype == "bf16"))
    S0 = synth.initial_state(wl)
    d = {n: dev(x[n], dtype) for n in ("q", "k", "v", "beta")}
    st = dev(S0)
    cu = torch.from_numpy(wl.cu_seqlens).cuda()
    o, _, _, _ = kda.kda_test_prefill(d["q"], d["k"], d["v"], dev(g, dtype), d["beta"], cu_seqlens=cu,
                                      initial_state=st, final_state=st, seg_chunks=4)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.prefill(x["q"], x["k"], x["v"], g, x["beta"], cu=wl.cu_seqlens, S0=S0)
    eo, es = relerr(host(o), o_ref), relerr(host(st), S_ref)
    print(f"  o {eo:.3e}  S {es:.3e}")
    assert eo < TOL[dtype] and es < TOL[dtype]
