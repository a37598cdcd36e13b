"""The checked build (libkda_checked.so, device-side bounds checks): every
kernel path runs under it with no check failing, and its results equal the
release build's bit for bit (the checks add no arithmetic)."""
import numpy as np
import pytest

import synth
from tests.gpu_common import announce, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    import torch
    import linear_attention_sequence_gate_amd as m
    assert torch.cuda.is_available()
    m.lib()
    return m


def both(kda, run):
    """run() under the release build and under the checked build; the checked
    build's check bits after it; the two results as lists of tensors."""
    import torch
    ref = run()
    torch.cuda.synchronize()
    with kda.using_library(kda.CHECKED_LIB_PATH):
        kda.device_check_bits(reset=True)
        got = run()
        torch.cuda.synchronize()
        bits = kda.device_check_bits(reset=True)
    return bits, [t for t in ref if t is not None], [t for t in got if t is not None]


def expect_same(kda, run):
    import torch
    bits, ref, got = both(kda, run)
    assert bits == 0, f"device-side checks failed: bits {bits:#x}"
    assert len(ref) == len(got)
    for a, b in zip(ref, got):
        assert torch.equal(a, b), "the checked build's result differs"


def prefill_run(kda, wl, seg=0, warm=-1, interval=0):
    import torch
    x = synth.prefill_inputs(wl)
    dt = wl.dtype
    cu = torch.from_numpy(wl.cu_seqlens).to("cuda") if wl.N > 1 else None
    hcu = wl.cu_seqlens if wl.N > 1 else None
    S0 = dev(synth.initial_state(wl)) if wl.state_std > 0 else None
    args = [dev(x[n], dt) for n in ("q", "k", "v", "z")]
    A, beta = dev(x["A"]), dev(x["beta"], dt)

    def run():
        o, S, ck, _ = kda.kda_test_prefill(args[0], args[1], args[2], args[3], beta, A=A, cu_seqlens=cu,
                                           cu_seqlens_host=hcu, initial_state=S0, interval=interval,
                                           seg_chunks=seg, warm_tokens=warm)
        return [o, S, ck]
    return run


@pytest.mark.parametrize("dk,dv,dtype", [(128, 128, "bf16"), (32, 128, "bf16"), (128, 32, "bf16"),
                                         (32, 64, "f32"), (128, 128, "f32"), (64, 32, "f32")])
def test_checked_prefill_varlen(kda, dk, dv, dtype):
    wl = synth.VARLEN_64.with_(H=3, dk=dk, dv=dv, dtype=dtype, seqlens=(0, 1, 63, 64, 65, 300, 17),
                               state_std=0.1)
    announce(f"checked prefill dk={dk} dv={dv} {dtype}")
    expect_same(kda, prefill_run(kda, wl, interval=64))


@pytest.mark.parametrize("warm", [-1, 0, 64])
@pytest.mark.parametrize("zshift", [0.0, -3.0])
def test_checked_prefill_segments(kda, warm, zshift):
    """segments of 2 chunks: warm-up windows, the exact passes, or both"""
    wl = synth.VARLEN_64.with_(H=2, seqlens=(700, 0, 129, 1000), state_std=0.1, z_shift=zshift)
    announce(f"checked prefill segments warm={warm} zshift={zshift}")
    expect_same(kda, prefill_run(kda, wl, seg=2, warm=warm, interval=128))


def test_checked_prefill_one_sequence(kda):
    wl = synth.PREFILL_8K.with_(H=4, seqlens=(3000,), z_shift=-2.0)
    announce("checked prefill, one 3000-token sequence")
    expect_same(kda, prefill_run(kda, wl))


def test_checked_decode_spec(kda):
    import torch
    B, K = 8, 5
    wl = synth.DECODE_B256.with_(H=4, seqlens=(1,) * B)
    announce("checked decode, verify and commit")
    x = {n: synth.token_rows(wl, n, 0, B) for n in ("q", "k", "v", "z", "beta")}
    S0 = dev(synth.initial_state(wl))
    A = dev(synth.gate_A(wl))
    t = {n: dev(x[n], wl.dtype) for n in x}
    t["g"] = kda.kda_gate(t["z"], A)
    d = {n: t[n].unsqueeze(1).repeat(1, K, *([1] * (t[n].dim() - 1))).contiguous() for n in t}
    na = torch.tensor([0, 1, 2, 3, 4, 5, 7, -1], dtype=torch.int32, device="cuda")

    def run():
        S = S0.clone()
        o = kda.kda_decode_step(t["q"], t["k"], t["v"], t["g"], t["beta"], S)
        og = kda.kda_decode_step_gated(t["q"], t["k"], t["v"], t["z"], A, t["beta"], S)
        ov = kda.kda_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], S)
        kda.kda_commit(d["k"], d["v"], d["g"], d["beta"], na, S)
        return [o, og, ov, S]
    expect_same(kda, run)


@pytest.mark.parametrize("with_ckpt", [False, True])
@pytest.mark.parametrize("dk,dv,dtype", [(128, 128, "bf16"), (64, 32, "f32")])
def test_checked_backward(kda, dk, dv, dtype, with_ckpt):
    import torch
    wl = synth.VARLEN_64.with_(H=2, dk=dk, dv=dv, dtype=dtype, seqlens=(0, 1, 63, 64, 65, 200), state_std=0.1,
                               z_shift=-2.0)
    announce(f"checked backward dk={dk} dv={dv} {dtype} ckpt={with_ckpt}")
    x = synth.prefill_inputs(wl)
    dt = wl.dtype
    cu = torch.from_numpy(wl.cu_seqlens).to("cuda")
    S0 = dev(synth.initial_state(wl))
    q, k, v, z, beta = (dev(x[n], dt) for n in ("q", "k", "v", "z", "beta"))
    g = kda.kda_gate(z, dev(x["A"]))
    rng = np.random.default_rng(7)
    dO = dev(rng.standard_normal((wl.T_total, wl.H, dv)).astype(np.float32), dt)
    dS = dev(rng.standard_normal((wl.N, wl.H, dk, dv)).astype(np.float32))
    ck = None
    if with_ckpt:
        _, _, ck = kda.kda_prefill_ckpt(q, k, v, g, beta, interval=64, cu_seqlens=cu,
                                        cu_seqlens_host=wl.cu_seqlens, initial_state=S0)
    torch.cuda.synchronize()

    def run():
        out = kda.kda_backward(q, k, v, g, beta, d_o=dO, d_final_state=dS, cu_seqlens=cu, initial_state=S0,
                               ckpt=ck, interval=64, seg_tokens=64)
        return [out[n] for n in sorted(out)]
    expect_same(kda, run)


@pytest.mark.parametrize("zshift", [0.0, -4.0])
def test_checked_serial_windows(kda, zshift):
    """the fp32 token-serial path in segments of 4 chunks: windows that hold
    (z) and windows that fall back to whole chains (z - 4), with checkpoints"""
    wl = synth.TINY_F32.with_(H=2, dk=128, dv=64, seqlens=(2000,), state_std=0.1, z_shift=zshift)
    announce(f"checked serial windows zshift={zshift}")
    expect_same(kda, prefill_run(kda, wl, seg=4, interval=192))
