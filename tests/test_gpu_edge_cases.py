"""GPU edge cases of the boundary and the planner's extreme shapes, against
the fp64 oracle where there is arithmetic:
  - zero tokens (one sequence, and three empty packed sequences): the final
    state is the initial state bit for bit, or zero without one, for the plain
    and the fused-gate prefill; the backward then passes d_final_state through
    to d_initial_state;
  - 520 heads over 300 tokens (more (sequence, head) items than compute units:
    one segment per sequence, no warm-up windows);
  - one head over 20,000 tokens (the planner's one-sequence split at few
    heads: 79 segments of 256 tokens, 78 of them with a warm-up window)."""
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


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("N", [1, 3])
@pytest.mark.parametrize("with_init", [False, True])
def test_zero_tokens(kda, gated, N, with_init):
    import torch
    H, dk, dv = 4, 64, 128
    announce(f"zero tokens: N={N} gated={gated} initial state={with_init}")
    e = lambda d: torch.empty((0, H, d), dtype=torch.bfloat16, device="cuda")
    q, k, z, v = e(dk), e(dk), e(dk), e(dv)
    beta = torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    cu = torch.zeros(N + 1, dtype=torch.int32, device="cuda") if N > 1 else None
    rng = np.random.default_rng(3)
    S0 = rng.standard_normal((N, H, dk, dv)).astype(np.float32) if with_init else None
    init = dev(S0) if with_init else None
    fin = torch.full((N, H, dk, dv), float("nan"), dtype=torch.float32, device="cuda")
    if gated:
        A = dev(np.zeros(H, np.float32))
        o, S = kda.kda_prefill_gated(q, k, v, z, A, beta, cu_seqlens=cu, initial_state=init, final_state=fin)
    else:
        o, S = kda.kda_prefill(q, k, v, z, beta, cu_seqlens=cu, initial_state=init, final_state=fin)
    torch.cuda.synchronize()
    assert o.shape == (0, H, dv)
    got = S.cpu().numpy()
    want = S0 if with_init else np.zeros((N, H, dk, dv), np.float32)
    assert np.array_equal(got, want)


def test_backward_zero_tokens(kda):
    import torch
    H, dk, dv = 2, 64, 64
    announce("backward, zero tokens")
    e = lambda d: torch.empty((0, H, d), dtype=torch.bfloat16, device="cuda")
    rng = np.random.default_rng(4)
    dfin = dev(rng.standard_normal((1, H, dk, dv)).astype(np.float32))
    d_o = torch.empty((0, H, dv), dtype=torch.bfloat16, device="cuda")
    beta = torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    out = kda.kda_backward(e(dk), e(dk), e(dv), e(dk), beta, d_o=d_o, d_final_state=dfin)
    torch.cuda.synchronize()
    assert np.array_equal(out["d_initial_state"].cpu().numpy(), dfin.cpu().numpy())


def run_vs_oracle(kda, wl, tag):
    import torch
    x = synth.prefill_inputs(wl)
    S0 = synth.initial_state(wl)
    dt = wl.dtype
    o, S = kda.kda_prefill_gated(dev(x["q"], dt), dev(x["k"], dt), dev(x["v"], dt), dev(x["z"], dt), dev(x["A"]),
                                 dev(x["beta"], dt), initial_state=dev(S0))
    torch.cuda.synchronize()
    g = oracle.gate(x["z"], x["A"])
    o_ref, S_ref = oracle.prefill(x["q"], x["k"], x["v"], g, x["beta"], S0=S0)
    eo, es = relerr(host(o), o_ref), relerr(host(S), S_ref)
    print(f"  {tag}: o err {eo:.3e}  state err {es:.3e}")
    assert eo < TOL[dt] and es < TOL[dt]


def test_many_heads(kda):
    wl = synth.PREFILL_8K.with_(H=520, dk=64, dv=64, seqlens=(300,), state_std=0.1)
    announce("520 heads x 300 tokens")
    assert "prefill_warm_kernel" in kda.describe_prefill_plan(300, 520, 64, 64)
    run_vs_oracle(kda, wl, "520 heads")


def test_one_head_long(kda):
    wl = synth.PREFILL_8K.with_(H=1, seqlens=(20000,), state_std=0.1)
    announce("1 head x 20000 tokens")
    plan = kda.describe_prefill_plan(20000, 1, 128, 128)
    assert "segments: 4 chunks of 64 tokens (256 tokens) each" in plan, plan
    run_vs_oracle(kda, wl, "1 head, 20000 tokens")
