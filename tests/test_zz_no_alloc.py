"""kda_prefill_gated_noalloc (the prefill whose workspace is the library's
static scratch) against kda_prefill_gated with a caller workspace: two calls in
a row on one GPU, the second smaller and taking the exact passes for two heads
(weak decay), so both the warm-up flags and the fallback's summaries live in
the scratch.  Each result must equal the workspace call's bit for bit (same
kernels, same plan) and meet the oracle's bf16 bar."""
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


def one_call(kda, wl, weak_heads=()):
    import torch
    x = synth.prefill_inputs(wl)
    if weak_heads:
        x["z"][:, list(weak_heads)] -= 4.0
        x["z"] = synth.bf16_round(x["z"])
    S0 = synth.initial_state(wl)
    d = {n: dev(x[n], wl.dtype) for n in ("q", "k", "v", "z", "beta")}
    A = dev(x["A"])
    cu = torch.from_numpy(wl.cu_seqlens).cuda() if wl.N > 1 else None
    T, H = wl.T_total, wl.H
    o_ref, S_ref = kda.kda_prefill_gated(d["q"], d["k"], d["v"], d["z"], A, d["beta"], cu_seqlens=cu,
                                         initial_state=dev(S0))
    o = torch.empty((T, H, wl.dv), dtype=torch.bfloat16, device="cuda")
    S = torch.empty((wl.N, H, wl.dk, wl.dv), dtype=torch.float32, device="cuda")
    kda.kda_prefill_gated_noalloc(d["q"], d["k"], d["v"], d["z"], A, d["beta"], o, final_state=S, cu_seqlens=cu,
                                  initial_state=dev(S0))
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    g = oracle.gate(x["z"], x["A"])
    o_or, S_or = oracle.prefill(x["q"], x["k"], x["v"], g, x["beta"], cu=wl.cu_seqlens, S0=S0)
    eo, es = relerr(host(o), o_or), relerr(host(S), S_or)
    print(f"  o {eo:.3e}  S {es:.3e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


def test_noalloc_two_calls(kda):
    wl1 = synth.PREFILL_8K.with_(H=16, seqlens=(4096,), state_std=0.1)
    announce("noalloc call 1: H=16 T=4096")
    need1 = kda.kda_prefill_workspace_size(wl1.T_total, 1, wl1.H, 128, 128)
    assert 0 < need1 <= (64 << 20)  # within the static scratch (KDA_NOALLOC_SCRATCH_BYTES)
    one_call(kda, wl1)
    wl2 = synth.VARLEN_64.with_(H=4, seqlens=(1500, 700, 33), state_std=0.1)
    announce("noalloc call 2: smaller, varlen, weak decay on heads 1 and 3")
    one_call(kda, wl2, weak_heads=(1, 3))
