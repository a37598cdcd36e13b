"""GPU parity of the prefill's head split: one sequence whose first tokens run
as a prefill of their own on a second stream while the summary pass of the
rest runs, the rest's scan starting from the head's final state.  Outputs,
final states and checkpoints against the fp64 oracle, on shapes where the
split is taken (and, with a checkpoint interval that does not divide the
head, where it is not)."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import TOL, announce, dev, host, relerr
from tests.test_gpu_prefill import SegEnv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    import torch
    import linear_attention_sequence_gate_amd as m
    assert torch.cuda.is_available()
    m.lib()
    return m


def inputs(wl):
    x = synth.prefill_inputs(wl)
    g = oracle.gate(x["z"], x["A"], round_bf16=(wl.dtype == "bf16"))
    S0 = synth.initial_state(wl) if wl.state_std > 0 else None
    return x, g, S0


def reference(wl, x, g, S0):
    return oracle.prefill(x["q"], x["k"], x["v"], g, x["beta"], S0=S0)


@pytest.mark.parametrize("T", [2048, 2000, 4160])
def test_split_outputs(kda, T):
    """Lengths with a partial last chunk and with more than two segments."""
    wl = synth.PREFILL_8K.with_(H=4, seqlens=(T,), state_std=0.1)
    announce(f"head split T={T} H={wl.H}")
    x, g, S0 = inputs(wl)
    d = {n: dev(x[n], wl.dtype) for n in ("q", "k", "v", "beta")}
    o, S = kda.kda_prefill(d["q"], d["k"], d["v"], dev(g, wl.dtype), d["beta"], initial_state=dev(S0))
    o_ref, S_ref = reference(wl, x, g, S0)
    eo, es = relerr(host(o), o_ref), relerr(host(S), S_ref)
    print(f"  o {eo:.3e}  S {es:.3e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


def test_split_f32(kda):
    """The fp32 prefill (d_k = 32) takes the split too."""
    wl = synth.TINY_F32.with_(H=2, seqlens=(2048,), state_std=0.1)
    announce("head split, fp32, d_k = d_v = 32")
    x = synth.prefill_inputs(wl)
    g = oracle.gate(x["z"], x["A"])
    S0 = synth.initial_state(wl)
    d = {n: dev(x[n], "f32") for n in ("q", "k", "v", "beta")}
    o, S = kda.kda_prefill(d["q"], d["k"], d["v"], dev(g), d["beta"], initial_state=dev(S0))
    o_ref, S_ref = reference(wl, x, g, S0)
    eo, es = relerr(host(o), o_ref), relerr(host(S), S_ref)
    print(f"  o {eo:.3e}  S {es:.3e}")
    assert eo < TOL["f32"] and es < TOL["f32"]


def test_split_matches_unsplit_run(kda):
    """The same call with the split switched off (a forced segment length)
    lands on the oracle too, and both agree to the bf16 bar."""
    import torch
    wl = synth.PREFILL_8K.with_(H=4, seqlens=(2048,), state_std=0.1)
    x, g, S0 = inputs(wl)
    d = {n: dev(x[n], wl.dtype) for n in ("q", "k", "v", "beta")}
    gd = dev(g, wl.dtype)
    o1, S1 = kda.kda_prefill(d["q"], d["k"], d["v"], gd, d["beta"], initial_state=dev(S0))
    with SegEnv(16):
        o2, S2 = kda.kda_prefill(d["q"], d["k"], d["v"], gd, d["beta"], initial_state=dev(S0))
    torch.cuda.synchronize()
    o_ref, S_ref = reference(wl, x, g, S0)
    for o, S in ((o1, S1), (o2, S2)):
        assert relerr(host(o), o_ref) < TOL["bf16"] and relerr(host(S), S_ref) < TOL["bf16"]
    assert relerr(host(o1), host(o2)) < TOL["bf16"]


@pytest.mark.parametrize("interval", [64, 512, 384])
def test_split_checkpoints(kda, interval):
    """Checkpoint rows on both sides of the head's end (64, 512), and an
    interval that does not divide the head (384: no split)."""
    wl = synth.PREFILL_8K.with_(H=4, seqlens=(2048,), state_std=0.1)
    announce(f"head split, checkpoints every {interval}")
    x, g, S0 = inputs(wl)
    d = {n: dev(x[n], wl.dtype) for n in ("q", "k", "v", "beta")}
    o, S, ck = kda.kda_prefill_ckpt(d["q"], d["k"], d["v"], dev(g, wl.dtype), d["beta"], interval,
                                    initial_state=dev(S0))
    T = wl.T_total
    rows = []
    Sr = S0
    for j in range(T // interval):
        r = slice(j * interval, (j + 1) * interval)
        _, Sr = oracle.prefill(x["q"][r], x["k"][r], x["v"][r], g[r], x["beta"][r], S0=Sr)
        rows.append(Sr[0])
    e = relerr(host(ck), np.array(rows))
    o_ref, S_ref = reference(wl, x, g, S0)
    print(f"  {len(rows)} checkpoints {e:.3e}")
    assert e < TOL["bf16"]
    assert relerr(host(o), o_ref) < TOL["bf16"] and relerr(host(S), S_ref) < TOL["bf16"]


def test_split_in_place_state_and_gate(kda):
    """initial_state == final_state (in place) through the fused gate."""
    import torch
    wl = synth.PREFILL_8K.with_(H=4, seqlens=(2048,), state_std=0.1)
    announce("head split, in-place state, fused gate")
    x = synth.prefill_inputs(wl)
    S0 = synth.initial_state(wl)
    d = {n: dev(x[n], wl.dtype) for n in ("q", "k", "v", "z", "beta")}
    st = dev(S0)
    o, _ = kda.kda_prefill_gated(d["q"], d["k"], d["v"], d["z"], dev(x["A"]), d["beta"],
                                 initial_state=st, final_state=st)
    torch.cuda.synchronize()
    g = oracle.gate(x["z"], x["A"])  # the fused gate keeps g in fp32
    o_ref, S_ref = reference(wl, x, g, S0)
    assert relerr(host(o), o_ref) < TOL["bf16"] and relerr(host(st), S_ref) < TOL["bf16"]


def test_split_two_streams(kda):
    """Two calls in flight on two user streams share the library's second
    stream and events: each result equals the same call run alone."""
    import torch
    wl = synth.PREFILL_8K.with_(H=4, seqlens=(2048,), state_std=0.1)
    announce("head split, two calls on two streams")
    x, g, S0 = inputs(wl)
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


def test_split_graph_replay(kda):
    """The split call captured into a HIP graph (the second stream joins the
    capture through the fork and join events) and replayed three times, with
    eager work and synchronisation between replays: every replay equals the
    eager call."""
    import torch
    wl = synth.PREFILL_8K.with_(H=4, seqlens=(2048,), state_std=0.1)
    announce("head split, graph capture and replay")
    x, g, S0 = inputs(wl)
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
    with torch.cuda.stream(st):  # warm up on the capture stream (creates the library's second stream)
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
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
