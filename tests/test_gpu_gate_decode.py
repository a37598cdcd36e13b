"""GPU parity: kda_gate and kda_decode_step against the fp64 oracle."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import TOL, announce, dev, dev_unaligned, host, relerr

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    import torch
    import linear_attention_sequence_gate_amd as m
    assert torch.cuda.is_available()
    m.lib()
    return m


def _bf16_ulps(got, want):
    """distance in bf16 units of the last place between bf16-exact values"""
    g = np.asarray(got, np.float32).view(np.int32) >> 16
    w = np.asarray(want, np.float32).view(np.int32) >> 16
    return np.abs(g.astype(np.int64) - w.astype(np.int64))


@pytest.mark.parametrize("wl,T", [(synth.TINY_F32, 256), (synth.PREFILL_8K, 2048)],
                         ids=["f32", "bf16"])
def test_gate_parity(kda, wl, T):
    announce(f"gate {wl.name} T={T}")
    z = synth.token_rows(wl, "z", 0, T)
    A = synth.gate_A(wl)
    g = host(kda.kda_gate(dev(z, wl.dtype), dev(A)))
    if wl.dtype == "bf16":
        ref = oracle.gate(z, A, round_bf16=True)
        ulps = _bf16_ulps(g.astype(np.float32), ref.astype(np.float32))
        assert ulps.max() <= 1, f"max {ulps.max()} bf16 ulps"
        assert np.mean(ulps > 0) < 1e-3, f"{np.mean(ulps > 0):.2e} of values off by one ulp"
    else:
        ref = oracle.gate(z, A)
        err = np.max(np.abs(g - ref) / np.maximum(np.abs(ref), 1e-30))
        assert err < 1e-5, f"elementwise relative error {err:.2e}"
    assert g.min() >= -5.0 and g.max() <= 0.0


def test_gate_inplace_and_unaligned(kda):
    import torch
    wl = synth.PREFILL_8K.with_(H=3, dk=36)
    announce("gate in place, d_k=36 (scalar path)")
    z = synth.token_rows(wl, "z", 0, 77)
    A = synth.gate_A(wl)
    zt = dev(z, "bf16")
    out = kda.kda_gate(zt, dev(A), g=zt)
    assert out.data_ptr() == zt.data_ptr()
    ref = oracle.gate(z, A, round_bf16=True)
    assert _bf16_ulps(host(zt).astype(np.float32), ref.astype(np.float32)).max() <= 1
    # sub-tensor starting 2 elements in: not 16-byte aligned
    big = dev(np.concatenate([np.zeros(2, np.float32), z.ravel()]), "bf16")
    zs = big[2:].view(77, 3, 36)
    g2 = torch.empty_like(zs)
    kda.kda_gate(zs, dev(A), g=g2)
    assert _bf16_ulps(host(g2).astype(np.float32), ref.astype(np.float32)).max() <= 1


def _decode_inputs(wl, set_index, B):
    d = {n: synth.token_rows(wl, n, 0, B, set_index=set_index) for n in ("q", "k", "v", "z", "beta")}
    return d


def _decode(kda, gated, q, k, v, z, A, beta, St, o=None):
    """kda_gate + kda_decode_step, or the fused kda_decode_step_gated."""
    if gated:
        return kda.kda_decode_step_gated(q, k, v, z, A, beta, St, o=o)
    return kda.kda_decode_step(q, k, v, kda.kda_gate(z, A), beta, St, o=o)


def _oracle_g(x, A, gated, dtype="bf16"):
    """The oracle's g: rounded to the storage dtype for the separate gate, fp32
    (unrounded) for the fused one."""
    return oracle.gate(x["z"], A, round_bf16=(dtype == "bf16" and not gated))


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("unaligned", [False, True])  # one-wave slice kernel / workgroup-per-state kernel
@pytest.mark.parametrize("dk,dv,dtype", [(128, 128, "bf16"), (64, 32, "bf16"), (32, 128, "bf16"),
                                         (32, 32, "f32"), (128, 64, "f32")])
def test_decode_small(kda, dk, dv, dtype, unaligned, gated):
    import torch
    wl = synth.DECODE_B256.with_(H=3, dk=dk, dv=dv, dtype=dtype, seqlens=(1,) * 5)
    announce(f"decode small dk={dk} dv={dv} {dtype} unaligned={unaligned} gated={gated}")
    B = 5
    x = _decode_inputs(wl, 0, B)
    A = synth.gate_A(wl)
    S0 = synth.initial_state(wl)
    St = dev(S0)
    q = dev(x["q"], dtype)
    if unaligned:
        q = dev_unaligned(q)
    o = _decode(kda, gated, q, dev(x["k"], dtype), dev(x["v"], dtype), dev(x["z"], dtype), dev(A),
                dev(x["beta"], dtype), St)
    gr = _oracle_g(x, A, gated, dtype)
    o_ref, S_ref = oracle.decode_step(x["q"], x["k"], x["v"], gr, x["beta"], S0)
    tol = TOL[dtype]
    assert relerr(host(o), o_ref) < tol
    assert relerr(host(St), S_ref) < tol


@pytest.mark.parametrize("gated", [False, True])
def test_decode_full_one_step(kda, gated):
    """B=256, H=32, d=128: one step, every output and every state entry."""
    wl = synth.DECODE_B256
    B = wl.N
    announce(f"decode B=256 H=32 one step gated={gated}")
    x = _decode_inputs(wl, 0, B)
    A = synth.gate_A(wl)
    S0 = synth.initial_state(wl)
    St = dev(S0)
    o = _decode(kda, gated, dev(x["q"], "bf16"), dev(x["k"], "bf16"), dev(x["v"], "bf16"), dev(x["z"], "bf16"),
                dev(A), dev(x["beta"], "bf16"), St)
    gr = _oracle_g(x, A, gated)
    o_ref, S_ref = oracle.decode_step(x["q"], x["k"], x["v"], gr, x["beta"], S0)
    e_o, e_s = relerr(host(o), o_ref), relerr(host(St), S_ref)
    print(f"decode 1 step: o err {e_o:.2e}, state err {e_s:.2e}")
    assert e_o < TOL["bf16"] and e_s < TOL["bf16"]


@pytest.mark.parametrize("gated", [False, True])
def test_decode_full_1000_steps_sampled(kda, gated):
    """1000 consecutive in-place steps at B=256, H=32 (inputs cycle through 8
    seeded sets); 64 sampled (b, h) states and their last outputs are replayed
    by the oracle over all 1000 steps."""
    import torch
    wl = synth.DECODE_B256
    B, H = wl.N, wl.H
    steps, nsets = 1000, 8
    announce(f"decode B=256 H=32 1000 steps gated={gated}")
    A = synth.gate_A(wl)
    S0 = synth.initial_state(wl)
    sets = [_decode_inputs(wl, s, B) for s in range(nsets)]
    dsets = []
    for x in sets:
        d = {n: dev(x[n], "bf16") for n in ("q", "k", "v", "z", "beta")}
        d["g"] = kda.kda_gate(d["z"], dev(A))
        dsets.append(d)
    St = dev(S0)
    Ad = dev(A)
    o = torch.empty((B, H, wl.dv), dtype=torch.bfloat16, device="cuda")
    for t in range(steps):
        d = dsets[t % nsets]
        if gated:
            kda.kda_decode_step_gated(d["q"], d["k"], d["v"], d["z"], Ad, d["beta"], St, o=o)
        else:
            kda.kda_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], St, o=o)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    units = rng.choice(B * H, size=64, replace=False)
    bs, hs = units // H, units % H
    S = S0[bs, hs][None].astype(np.float64)  # [1, 64, dk, dv] as 64 "heads" of one batch row
    gr = [_oracle_g(x, A, gated) for x in sets]
    for t in range(steps):
        x = sets[t % nsets]
        pick = lambda a: a[bs, hs][None]
        o_ref, S = oracle.decode_step(pick(x["q"]), pick(x["k"]), pick(x["v"]), pick(gr[t % nsets]),
                                      pick(x["beta"]), S)
    e_o = relerr(host(o)[bs, hs], o_ref[0])
    e_s = relerr(host(St)[bs, hs], S[0])
    print(f"decode 1000 steps: o err {e_o:.2e}, state err {e_s:.2e}")
    assert e_o < TOL["bf16"] and e_s < TOL["bf16"]
