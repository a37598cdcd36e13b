"""GPU self-consistency of the KDA path, beside the oracle parity tests:
bitwise determinism on repeat, prefill chaining through the final state,
packed varlen against per-sequence runs, segment parallelism on and off, and
T decode steps against a T-token prefill.  Each comparison between two GPU
runs that take different routes is held to the bf16 parity tolerance, and
every route is also checked against the fp64 oracle."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import TOL, announce, dev, gated_prefill, host, relerr

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    import torch
    import linear_attention_sequence_gate_amd as m
    assert torch.cuda.is_available()
    m.lib()
    return m


def _inputs(wl):
    x = synth.prefill_inputs(wl)
    d = {n: dev(x[n], wl.dtype) for n in ("q", "k", "v", "z", "beta")}
    d["A"] = dev(x["A"])
    return x, d


def _gated(kda, d, rows=None, cu=None, S0=None, seg=None):
    import torch
    sl = (lambda t: t) if rows is None else (lambda t: t[rows[0]:rows[1]].contiguous())
    o, S = gated_prefill(kda, sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["z"]), d["A"], sl(d["beta"]), seg=seg,
                         cu_seqlens=cu, initial_state=S0)
    torch.cuda.synchronize()
    return o, S


def test_determinism(kda):
    """Same inputs, same launch configuration: bit-identical outputs and states
    (no atomics anywhere on the path)."""
    import torch
    wl = synth.PREFILL_8K.with_(H=8, seqlens=(3000,), state_std=0.1)
    announce("consistency: determinism (prefill, decode, verify)")
    x, d = _inputs(wl)
    S0 = dev(synth.initial_state(wl))
    o1, S1 = _gated(kda, d, S0=S0, seg=4)
    o2, S2 = _gated(kda, d, S0=S0, seg=4)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    B = 16
    st1 = S0.repeat(B, 1, 1, 1).contiguous()
    st2 = st1.clone()
    q, k, v, z, b = (d[n][:B] for n in ("q", "k", "v", "z", "beta"))
    oa = kda.kda_decode_step_gated(q, k, v, z, d["A"], b, st1)
    ob = kda.kda_decode_step_gated(q, k, v, z, d["A"], b, st2)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob) and torch.equal(st1, st2)


def test_chaining_through_the_final_state(kda):
    """prefill(T1) -> its final state -> prefill(T2) equals prefill(T1 + T2):
    the state hand-off of a prefix cache, with T1 off the chunk grid."""
    wl = synth.PREFILL_8K.with_(H=4, seqlens=(1700,), state_std=0.1, z_shift=-3.0)
    announce("consistency: chaining 1111 + 589 tokens")
    x, d = _inputs(wl)
    S0 = dev(synth.initial_state(wl))
    T, T1 = wl.T_total, 1111
    o_all, S_all = _gated(kda, d, S0=S0, seg=3)
    o_a, S_a = _gated(kda, d, rows=(0, T1), S0=S0, seg=3)
    o_b, S_b = _gated(kda, d, rows=(T1, T), S0=S_a, seg=3)
    o_cat = np.concatenate([host(o_a), host(o_b)])
    assert relerr(o_cat, host(o_all)) < TOL["bf16"]
    assert relerr(host(S_b), host(S_all)) < TOL["bf16"]
    g = oracle.gate(x["z"], x["A"])
    o_ref, S_ref = oracle.prefill(x["q"], x["k"], x["v"], g, x["beta"], S0=synth.initial_state(wl))
    assert relerr(o_cat, o_ref) < TOL["bf16"] and relerr(host(S_b), S_ref) < TOL["bf16"]


def test_varlen_packed_against_separate_runs(kda):
    """Packed sequences leave no trace in each other: each sequence run alone
    (its own launch, its own segment plan) gives the packed run's outputs and
    final state."""
    import torch
    wl = synth.VARLEN_64.with_(H=3, seqlens=(700, 0, 64, 129, 1000, 5), state_std=0.1)
    announce(f"consistency: varlen packed vs separate, lens={wl.seqlens}")
    x, d = _inputs(wl)
    S0 = synth.initial_state(wl)
    cu = wl.cu_seqlens
    o_p, S_p = _gated(kda, d, cu=torch.from_numpy(cu).cuda(), S0=dev(S0), seg=2)
    for n in range(wl.N):
        a, b = int(cu[n]), int(cu[n + 1])
        if b == a:
            assert torch.equal(S_p[n], dev(S0[n]))  # an empty sequence hands its state through
            continue
        o_n, S_n = _gated(kda, d, rows=(a, b), S0=dev(S0[n:n + 1]), seg=1)
        assert relerr(host(o_p[a:b]), host(o_n)) < TOL["bf16"], f"sequence {n}"
        assert relerr(host(S_p[n]), host(S_n[0])) < TOL["bf16"], f"sequence {n}"


@pytest.mark.parametrize("seg", [1, 2, 5])
def test_segments_on_and_off(kda, seg):
    """The segment summary / scan / rerun route against one segment per sequence."""
    wl = synth.PREFILL_8K.with_(H=4, seqlens=(2000,), state_std=0.1, z_shift=-3.0)
    announce(f"consistency: segments of {seg} chunks vs none")
    x, d = _inputs(wl)
    S0 = dev(synth.initial_state(wl))
    o1, S1 = _gated(kda, d, S0=S0, seg=1000)  # one segment: no summary pass, no scan
    o2, S2 = _gated(kda, d, S0=S0, seg=seg)
    assert relerr(host(o2), host(o1)) < TOL["bf16"] and relerr(host(S2), host(S1)) < TOL["bf16"]


def test_decode_steps_against_prefill(kda):
    """T in-place decode steps from a state give the T-token prefill from it."""
    import torch
    wl = synth.PREFILL_8K.with_(H=4, dk=64, dv=64, seqlens=(40,), state_std=0.1, z_shift=-2.0)
    announce("consistency: 40 decode steps vs a 40-token prefill")
    x, d = _inputs(wl)
    S0 = dev(synth.initial_state(wl))
    o_p, S_p = _gated(kda, d, S0=S0)
    st = S0.clone()
    outs = []
    for t in range(wl.T_total):
        r = lambda n: d[n][t:t + 1].contiguous()
        outs.append(kda.kda_decode_step_gated(r("q"), r("k"), r("v"), r("z"), d["A"], r("beta"), st))
    torch.cuda.synchronize()
    o_d = np.concatenate([host(o) for o in outs])
    assert relerr(o_d, host(o_p)) < TOL["bf16"] and relerr(host(st), host(S_p)) < TOL["bf16"]
