"""GPU parity of kda_prefill_ckpt: the state checkpoints every `interval`
tokens of each sequence equal the fp64 oracle's states at those positions
(the oracle run window by window, each window starting from the previous
window's final state); outputs and final states equal plain kda_prefill."""
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


def oracle_ckpts(wl, x, g, S0, interval):
    cu = wl.cu_seqlens
    out = []
    for n in range(wl.N):
        S = (S0[n:n + 1] if S0 is not None else np.zeros((1, wl.H, wl.dk, wl.dv)))
        a = int(cu[n])
        for j in range(int(cu[n + 1] - cu[n]) // interval):
            r = slice(a + j * interval, a + (j + 1) * interval)
            _, S = oracle.prefill(x["q"][r], x["k"][r], x["v"][r], g[r], x["beta"][r], S0=S)
            out.append(S[0])
    return np.array(out) if out else np.zeros((0, wl.H, wl.dk, wl.dv))


def check(kda, wl, interval, seg=None):
    import torch
    announce(f"ckpt {wl.name} H={wl.H} dk={wl.dk} dv={wl.dv} {wl.dtype} lens={list(wl.seqlens)[:10]} "
             f"interval={interval} seg={seg}")
    dt = wl.dtype
    x = synth.prefill_inputs(wl)
    S0 = synth.initial_state(wl) if wl.state_std > 0 else None
    g_dev = kda.kda_gate(dev(x["z"], dt), dev(x["A"]))
    cu = torch.from_numpy(wl.cu_seqlens).cuda() if wl.N > 1 else None
    args = [dev(x[n], dt) for n in ("q", "k", "v")] + [g_dev, dev(x["beta"], dt)]
    with SegEnv(seg):
        o, S, ck = kda.kda_prefill_ckpt(*args, interval=interval, cu_seqlens=cu,
                                        cu_seqlens_host=wl.cu_seqlens if wl.N > 1 else None,
                                        initial_state=None if S0 is None else dev(S0))
        o2, S2 = kda.kda_prefill(*args, cu_seqlens=cu, initial_state=None if S0 is None else dev(S0))
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(S, S2), "checkpointing changed the outputs"
    g = oracle.gate(x["z"], x["A"], round_bf16=(dt == "bf16"))
    ref = oracle_ckpts(wl, x, g, S0, interval)
    assert ck.shape[0] == ref.shape[0]
    if ref.shape[0]:
        e = relerr(host(ck), ref)
        print(f"  {ref.shape[0]} checkpoints: err {e:.3e}")
        assert e < TOL[dt]


@pytest.mark.parametrize("interval", [64, 512])
def test_ckpt_varlen(kda, interval):
    wl = synth.VARLEN_64.with_(H=3, dk=64, dv=64, seqlens=(0, 1, 63, 64, 65, 512, 513, 1024, 1100),
                               state_std=0.1)
    check(kda, wl, interval)


def test_ckpt_segmented(kda):
    """checkpoints written by the output pass of every segment of a long sequence"""
    wl = synth.VARLEN_64.with_(H=2, seqlens=(3000, 700), state_std=0.1)
    check(kda, wl, 128, seg=3)


def test_ckpt_f32(kda):
    check(kda, synth.TINY_F32.with_(seqlens=(256, 130), state_std=0.1), 64)


def test_ckpt_8k(kda):
    check(kda, synth.PREFILL_8K, 512)
