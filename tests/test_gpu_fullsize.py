"""GPU parity at the full sizes of the two million-token workloads, in the
default launch configuration (the planner's own segment length).

The oracle cannot run a million tokens of every head in seconds, so it checks
samples it can compute exactly:
  - prefill_1m (z shifted by +3, so every channel decays hard): windows of the
    output and the final state for sampled heads, from an oracle started at
    zero state W tokens earlier.  Every step applies Diag(alpha_t) and then the
    delta-rule factor (I - beta k k^T), whose 2-norm is at most 1 (beta in
    [0, 1], |k| = 1), so whatever the state held W tokens back is damped by at
    least prod_t max_c alpha_t,c = exp(sum_t max_c g_t,c).  The test computes
    that bound from the actual gate values and requires it below e^-60.
  - varlen_64: whole sequences (outputs and final states) for the three
    shortest sequences on every head, and the longest sequence on two heads.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import TOL, announce, dev, dev_stream, host, relerr

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    import torch
    import linear_attention_sequence_gate_amd as m
    assert torch.cuda.is_available()
    m.lib()
    return m


def oracle_rows(wl, t0, t1, heads, gated=False):
    """Oracle inputs for rows [t0, t1) of `heads`.  The separate gate returns g
    rounded to bf16; the gate fused into kda_prefill_gated keeps it in fp32."""
    x = {n: synth.token_rows(wl, n, t0, t1)[:, heads] for n in ("q", "k", "v", "z", "beta")}
    g = oracle.gate(x["z"], synth.gate_A(wl)[heads], round_bf16=not gated)
    return x, g


def gpu_prefill(kda, xs, A, gated, **kw):
    """kda_gate + kda_prefill, or the fused kda_prefill_gated, on device tensors."""
    if gated:
        return kda.kda_prefill_gated(xs["q"], xs["k"], xs["v"], xs["z"], A, xs["beta"], **kw)
    g = kda.kda_gate(xs["z"], A)
    del xs["z"]
    return kda.kda_prefill(xs["q"], xs["k"], xs["v"], g, xs["beta"], **kw)


@pytest.mark.parametrize("gated", [False, True])
def test_prefill_1m_windows(kda, gated):
    import torch
    wl = synth.PREFILL_1M
    T = wl.T_total
    announce(f"prefill_1m full size: H={wl.H} T={T} gated={gated}")
    xs = {n: dev_stream(wl, n) for n in ("q", "k", "v", "z", "beta")}
    o, S = gpu_prefill(kda, xs, dev(synth.gate_A(wl)), gated)
    del xs
    torch.cuda.synchronize()
    seg = 256 * 64  # the planner's segment length for this shape (tokens)
    heads = [2, 6]
    W = 512
    windows = [(0, 256), (3 * T // 4 + 5000, 3 * T // 4 + 5256), (32 * seg - 37, 32 * seg + 219), (T - 256, T)]
    for a, b in windows:
        s0 = max(0, a - W)
        x, gw = oracle_rows(wl, s0, b, heads, gated)
        if s0 > 0:  # damping of the state the window starts without
            damp = float(np.max(np.sum(np.max(gw[: a - s0], axis=2), axis=0)))
            assert damp < -60.0, f"warm-up too short: log damping {damp:.1f}"
        o_ref, S_ref = oracle.prefill(x["q"], x["k"], x["v"], gw, x["beta"])
        got = host(o[a:b, heads])
        e = relerr(got, o_ref[a - s0:])
        print(f"  window [{a}, {b}) heads {heads}: o err {e:.3e}")
        assert e < TOL["bf16"]
        if b == T:
            es = relerr(host(S[0, heads]), S_ref[0])
            print(f"  final state heads {heads}: err {es:.3e}")
            assert es < TOL["bf16"]
    assert torch.isfinite(o).all() and torch.isfinite(S).all()


@pytest.mark.parametrize("gated", [False, True])
def test_varlen_64_sampled_sequences(kda, gated):
    import torch
    wl = synth.VARLEN_64
    T = wl.T_total
    cu = wl.cu_seqlens
    lens = np.asarray(wl.seqlens)
    announce(f"varlen_64 full size: N={wl.N} H={wl.H} T={T} gated={gated}")
    xs = {n: dev_stream(wl, n, rows=1 << 14) for n in ("q", "k", "v", "z", "beta")}
    S0 = synth.initial_state(wl)
    o, S = gpu_prefill(kda, xs, dev(synth.gate_A(wl)), gated, cu_seqlens=torch.from_numpy(cu).cuda(),
                       initial_state=dev(S0))
    del xs
    torch.cuda.synchronize()
    order = np.argsort(lens)
    cases = [(int(n), list(range(wl.H))) for n in order[:3]] + [(int(order[-1]), [5, 21])]
    for n, heads in cases:
        a, b = int(cu[n]), int(cu[n + 1])
        x, gw = oracle_rows(wl, a, b, heads, gated)
        o_ref, S_ref = oracle.prefill(x["q"], x["k"], x["v"], gw, x["beta"], S0=S0[n:n + 1][:, heads])
        eo = relerr(host(o[a:b, heads]), o_ref)
        es = relerr(host(S[n, heads]), S_ref[0])
        print(f"  sequence {n} (len {b - a}) heads {len(heads)}: o err {eo:.3e} state err {es:.3e}")
        assert eo < TOL["bf16"] and es < TOL["bf16"]
    assert torch.isfinite(o).all() and torch.isfinite(S).all()
