"""GPU parity of kda_prefill_ckpt: the state checkpoints every `interval`
tokens of each sequence equal the fp64 oracle's states at those positions
(the oracle run window by window, each window starting from the previous
window's final state); outputs and final states equal plain kda_prefill."""
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


def check(kda, wl, interval, seg=None, warm=-1):
    import torch
    announce(f"ckpt {wl.name} H={wl.H} dk={wl.dk} dv={wl.dv} {wl.dtype} lens={list(wl.seqlens)[:10]} "
             f"interval={interval} seg={seg} warm={warm}")
    dt = wl.dtype
    x = synth.prefill_inputs(wl)
    S0 = synth.initial_state(wl) if wl.state_std > 0 else None
    g_dev = kda.kda_gate(dev(x["z"], dt), dev(x["A"]))
    cu = torch.from_numpy(wl.cu_seqlens).cuda() if wl.N > 1 else None
    args = [dev(x[n], dt) for n in ("q", "k", "v")] + [g_dev, dev(x["beta"], dt)]
    init = None if S0 is None else dev(S0)
    if seg is None:
        o, S, ck = kda.kda_prefill_ckpt(*args, interval=interval, cu_seqlens=cu,
                                        cu_seqlens_host=wl.cu_seqlens if wl.N > 1 else None, initial_state=init)
        o2, S2 = kda.kda_prefill(*args, cu_seqlens=cu, initial_state=init)
    else:  # a forced segment length, through the test entry point
        hcu = wl.cu_seqlens if wl.N > 1 else None
        o, S, ck, _ = kda.kda_test_prefill(*args, interval=interval, cu_seqlens=cu, cu_seqlens_host=hcu,
                                           initial_state=init, seg_chunks=seg, warm_tokens=warm)
        o2, S2, _, _ = kda.kda_test_prefill(*args, cu_seqlens=cu, initial_state=init, seg_chunks=seg,
                                            warm_tokens=warm)
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


@pytest.mark.parametrize("warm", [-1, 0])
@pytest.mark.parametrize("zshift", [0.0, -3.0])
def test_ckpt_segmented(kda, warm, zshift):
    """checkpoints written by every segment of long sequences, after a warm-up
    window (weak decay: the exact passes write them) or the exact passes alone"""
    wl = synth.VARLEN_64.with_(H=2, seqlens=(3000, 700), state_std=0.1, z_shift=zshift)
    check(kda, wl, 128, seg=3, warm=warm)


def test_ckpt_f32(kda):
    check(kda, synth.TINY_F32.with_(seqlens=(256, 130), state_std=0.1), 64)


@pytest.mark.parametrize("interval", [64, 192])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 32)])
def test_ckpt_f32_serial(kda, dk, dv, interval):
    """checkpoints of the token-serial fp32 kernel over packed sequences"""
    wl = synth.TINY_F32.with_(H=2, dk=dk, dv=dv, seqlens=(0, 63, 64, 65, 400, 130), state_std=0.1)
    check(kda, wl, interval)


def test_ckpt_8k(kda):
    check(kda, synth.PREFILL_8K, 512)


@pytest.mark.parametrize("dk,dv,dtype,seg,warm", [(128, 128, "bf16", 0, -1), (64, 64, "bf16", 3, 0),
                                                  (64, 64, "bf16", 3, -1), (128, 64, "f32", 4, -1)])
def test_ckpt_capacity_short(kda, dk, dv, dtype, seg, warm):
    """A checkpoint buffer three rows short of kda_checkpoint_count: the rows it
    holds equal a full-capacity run's and nothing is written past it (the
    buffer is a view into a larger sentinel-filled one); outputs unchanged."""
    import torch
    wl = synth.VARLEN_64.with_(H=2, dk=dk, dv=dv, dtype=dtype, seqlens=(700, 0, 1300, 65, 900), state_std=0.1)
    announce(f"ckpt capacity short dk={dk} dv={dv} {dtype} seg={seg} warm={warm}")
    x = synth.prefill_inputs(wl)
    cu = torch.from_numpy(wl.cu_seqlens).cuda()
    args = [dev(x[n], dtype) for n in ("q", "k", "v", "z", "beta")]
    A = dev(x["A"])
    init = dev(synth.initial_state(wl))
    n_full = kda.kda_checkpoint_count(wl.cu_seqlens, wl.T_total, 128)
    full = torch.empty((n_full, wl.H, dk, dv), dtype=torch.float32, device="cuda")
    big = torch.full((n_full + 2, wl.H, dk, dv), float("nan"), dtype=torch.float32, device="cuda")
    short = big[:n_full - 3]
    outs = []
    for ck in (full, short):
        o, S, _, _ = kda.kda_test_prefill(*args[:4], args[4], A=A, cu_seqlens=cu, cu_seqlens_host=wl.cu_seqlens,
                                          initial_state=init, interval=128, ckpt=ck, seg_chunks=seg,
                                          warm_tokens=warm)
        outs.append((o, S))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(short, full[:n_full - 3])
    assert torch.isnan(big[n_full - 3:]).all(), "a checkpoint was written past the capacity"
