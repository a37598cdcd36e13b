"""GPU parity of kda_verify / kda_commit (speculative multi-token decode with
replay) against the fp64 oracle: verify of K draft tokens from a state equals
a K-token prefill from that state (outputs); commit of n accepted tokens
equals an n-token prefill (state)."""
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


def inputs(wl, B, K):
    """Draft tokens [B, K, ...] as the packed rows of a workload of B sequences of K tokens."""
    x = synth.prefill_inputs(wl.with_(seqlens=(K,) * B))
    g = oracle.gate(x["z"], x["A"], round_bf16=(wl.dtype == "bf16"))
    S0 = synth.initial_state(wl.with_(seqlens=(K,) * B))
    return x, g, S0


def to_dev(kda, wl, x, B, K):
    import torch
    dt = wl.dtype
    shp = lambda a: a.reshape((B, K) + a.shape[1:])
    t = {n: dev(shp(x[n]), dt) for n in ("q", "k", "v", "beta")}
    t["g"] = kda.kda_gate(dev(shp(x["z"]), dt).reshape(B * K, wl.H, wl.dk), dev(x["A"])).reshape(B, K, wl.H, wl.dk)
    return t


def oracle_run(x, g, S0, lens, K):
    """Prefill over the first lens[b] of each sequence's K tokens."""
    B = len(lens)
    idx = np.concatenate([np.arange(b * K, b * K + n) for b, n in enumerate(lens)]).astype(np.int64)
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    return oracle.prefill(x["q"][idx], x["k"][idx], x["v"][idx], g[idx], x["beta"][idx], cu=cu, S0=S0)


CASES = [(32, 32, "bf16"), (64, 128, "bf16"), (128, 64, "bf16"), (128, 128, "bf16"), (32, 32, "f32"),
         (32, 64, "f32")]


@pytest.mark.parametrize("K,unaligned", [(3, False), (5, False), (12, False), (5, True)])
@pytest.mark.parametrize("dk,dv,dtype", CASES)
def test_verify_and_commit_small(kda, dk, dv, dtype, K, unaligned):
    """unaligned: token tensors off a 16-byte boundary, which the
    workgroup-per-state kernels take instead of the one-wave slice kernels."""
    import torch
    B = 6
    wl = synth.VERIFY_B256_K4.with_(H=3, dk=dk, dv=dv, dtype=dtype)
    announce(f"verify/commit B={B} K={K} H=3 dk={dk} dv={dv} {dtype} unaligned={unaligned}")
    x, g, S0 = inputs(wl, B, K)
    t = to_dev(kda, wl, x, B, K)
    if unaligned:
        t = {n: dev_unaligned(a) for n, a in t.items()}
    state = dev(S0)
    before = state.clone()
    o = kda.kda_verify(t["q"], t["k"], t["v"], t["g"], t["beta"], state)
    torch.cuda.synchronize()
    assert torch.equal(state, before), "verify modified the state"
    o_ref, _ = oracle_run(x, g, S0, [K] * B, K)
    e = relerr(host(o).reshape(B * K, 3, dv), o_ref)
    print(f"  verify o err {e:.3e}")
    assert e < TOL[dtype]
    n = np.array([0, 1, K, 2, K - 1, 3], dtype=np.int32)
    kda.kda_commit(t["k"], t["v"], t["g"], t["beta"], torch.from_numpy(n).cuda(), state)
    torch.cuda.synchronize()
    got = host(state)
    assert np.array_equal(got[0], host(before)[0]), "n_accept = 0 must leave the state untouched"
    _, S_ref = oracle_run(x, g, S0, list(n), K)
    es = relerr(got, S_ref)
    print(f"  commit state err {es:.3e}")
    assert es < TOL[dtype]


OTHER_SHAPES = [(dk, dv, dt) for dt in ("bf16", "f32") for dk in (32, 64, 128) for dv in (32, 64, 128)
                if (dk, dv, dt) not in CASES]


@pytest.mark.parametrize("dk,dv,dtype", OTHER_SHAPES)
def test_verify_and_commit_other_shapes(kda, dk, dv, dtype):
    """The remaining head shapes and dtypes the step kernels are built for (the
    verify kernel stages 1 to 8 tokens per group, over 64 to 256 threads,
    depending on the shape), with K = 9 drafts."""
    import torch
    B, K, H = 4, 9, 2
    wl = synth.VERIFY_B256_K4.with_(H=H, dk=dk, dv=dv, dtype=dtype)
    announce(f"verify/commit B={B} K={K} H={H} dk={dk} dv={dv} {dtype}")
    x, g, S0 = inputs(wl, B, K)
    t = to_dev(kda, wl, x, B, K)
    state = dev(S0)
    o = kda.kda_verify(t["q"], t["k"], t["v"], t["g"], t["beta"], state)
    n = np.array([K, 0, 5, 1], dtype=np.int32)
    kda.kda_commit(t["k"], t["v"], t["g"], t["beta"], torch.from_numpy(n).cuda(), state)
    torch.cuda.synchronize()
    o_ref, _ = oracle_run(x, g, S0, [K] * B, K)
    _, S_ref = oracle_run(x, g, S0, list(n), K)
    eo, es = relerr(host(o).reshape(B * K, H, dv), o_ref), relerr(host(state), S_ref)
    print(f"  verify o {eo:.3e}  commit state {es:.3e}")
    assert eo < TOL[dtype] and es < TOL[dtype]


def test_verify_commit_match_decode_steps(kda):
    """verify's outputs and commit's state equal the same tokens fed one by one
    to kda_decode_step (the same arithmetic per token)."""
    import torch
    B, K = 16, 4
    wl = synth.VERIFY_B256_K4.with_(H=4)
    x, g, S0 = inputs(wl, B, K)
    t = to_dev(kda, wl, x, B, K)
    state = dev(S0)
    o = kda.kda_verify(t["q"], t["k"], t["v"], t["g"], t["beta"], state)
    s2 = dev(S0)
    outs = []
    for i in range(K):
        sl = lambda a: a[:, i].contiguous()
        outs.append(kda.kda_decode_step(sl(t["q"]), sl(t["k"]), sl(t["v"]), sl(t["g"]), sl(t["beta"]), s2))
    n = torch.full((B,), K, dtype=torch.int32, device="cuda")
    kda.kda_commit(t["k"], t["v"], t["g"], t["beta"], n, state)
    torch.cuda.synchronize()
    od = torch.stack(outs, dim=1)
    assert relerr(host(o), host(od)) < 1e-6
    assert relerr(host(state), host(s2)) < 1e-6


@pytest.mark.parametrize("K", [17, 64])
def test_long_drafts_match_decode_steps_and_oracle(kda, K):
    """Drafts of several LDS token groups (up to the K = 64 maximum; 17 ends in
    a one-token group): verify's outputs and commit's state equal K decode
    steps and meet the oracle's bar."""
    import torch
    B = 3
    wl = synth.VERIFY_B256_K4.with_(H=4)
    announce(f"verify/commit B={B} K={K} H=4 d=128 bf16 against decode steps")
    x, g, S0 = inputs(wl, B, K)
    t = to_dev(kda, wl, x, B, K)
    state = dev(S0)
    o = kda.kda_verify(t["q"], t["k"], t["v"], t["g"], t["beta"], state)
    s2 = dev(S0)
    outs = []
    for i in range(K):
        sl = lambda a: a[:, i].contiguous()
        outs.append(kda.kda_decode_step(sl(t["q"]), sl(t["k"]), sl(t["v"]), sl(t["g"]), sl(t["beta"]), s2))
    n = torch.full((B,), K, dtype=torch.int32, device="cuda")
    kda.kda_commit(t["k"], t["v"], t["g"], t["beta"], n, state)
    torch.cuda.synchronize()
    assert torch.equal(o, torch.stack(outs, dim=1)), "verify differs from the decode steps"
    assert torch.equal(state, s2), "commit differs from the decode steps"
    o_ref, S_ref = oracle_run(x, g, S0, [K] * B, K)
    eo, es = relerr(host(o).reshape(B * K, 4, wl.dv), o_ref), relerr(host(state), S_ref)
    print(f"  o {eo:.3e}  state {es:.3e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


def test_verify_commit_full_sampled(kda):
    """The decode workload's shape (B=256, H=32, d=128) with K=4 draft tokens;
    sampled sequences against the oracle."""
    import torch
    wl = synth.VERIFY_B256_K4
    B, K = 256, 4
    announce(f"verify/commit full size B={B} K={K} H={wl.H}")
    x, g, S0 = inputs(wl, B, K)
    t = to_dev(kda, wl, x, B, K)
    state = dev(S0)
    o = kda.kda_verify(t["q"], t["k"], t["v"], t["g"], t["beta"], state)
    rng = np.random.default_rng(7)
    n = rng.integers(0, K + 1, size=B).astype(np.int32)
    kda.kda_commit(t["k"], t["v"], t["g"], t["beta"], torch.from_numpy(n).cuda(), state)
    torch.cuda.synchronize()
    oh, sh = host(o), host(state)
    for b in [0, 1, 77, 128, 255]:
        rows = slice(b * K, (b + 1) * K)
        sub = {k_: x[k_][rows] for k_ in ("q", "k", "v", "beta")}
        o_ref, _ = oracle.prefill(sub["q"], sub["k"], sub["v"], g[rows], sub["beta"], S0=S0[b:b + 1])
        nb = int(n[b])
        _, S_ref = oracle.prefill(sub["q"][:nb], sub["k"][:nb], sub["v"][:nb], g[rows][:nb], sub["beta"][:nb],
                                  S0=S0[b:b + 1])
        eo, es = relerr(oh[b], o_ref), relerr(sh[b:b + 1], S_ref)
        print(f"  seq {b} n_accept {nb}: o err {eo:.3e} state err {es:.3e}")
        assert eo < TOL["bf16"] and es < TOL["bf16"]
