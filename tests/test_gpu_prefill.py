"""GPU parity: kda_gate + kda_prefill against the fp64 oracle (token-serial
recurrence).  The GPU path applies its own gate to z and A; the oracle applies
its gate and rounds g to the storage dtype, as the gate's output contract says."""
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


def run_gpu(kda, wl, x, S0, seg=None, warm=-1):
    """kda_gate + kda_prefill; with a forced segment length (chunks) or warm-up
    (tokens; 0 = the exact summary / scan / output passes only) through the
    test entry point that takes the planner's choices as arguments."""
    import torch
    dt = wl.dtype
    cu = torch.from_numpy(wl.cu_seqlens).to("cuda") if wl.N > 1 else None
    g = kda.kda_gate(dev(x["z"], dt), dev(x["A"]))
    args = (dev(x["q"], dt), dev(x["k"], dt), dev(x["v"], dt), g, dev(x["beta"], dt))
    init = None if S0 is None else dev(S0)
    if seg is None and warm == -1:
        o, S = kda.kda_prefill(*args, cu_seqlens=cu, initial_state=init)
    else:
        o, S, _, _ = kda.kda_test_prefill(*args, cu_seqlens=cu, initial_state=init, seg_chunks=seg or 0,
                                          warm_tokens=warm)
    torch.cuda.synchronize()
    return host(o), host(S)


def run_oracle(wl, x, S0):
    g = oracle.gate(x["z"], x["A"], round_bf16=(wl.dtype == "bf16"))
    return oracle.prefill(x["q"], x["k"], x["v"], g, x["beta"], cu=wl.cu_seqlens, S0=S0)


def check(kda, wl, seg=None, tag="", warm=-1):
    announce(f"prefill {wl.name} {tag} H={wl.H} dk={wl.dk} dv={wl.dv} {wl.dtype} "
             f"lens={list(wl.seqlens)[:8]} seg={seg} warm={warm}")
    x = synth.prefill_inputs(wl)
    S0 = synth.initial_state(wl) if wl.state_std > 0 else None
    o, S = run_gpu(kda, wl, x, S0, seg, warm)
    o_ref, S_ref = run_oracle(wl, x, S0)
    e_o, e_s = relerr(o, o_ref), relerr(S, S_ref)
    print(f"  o err {e_o:.3e}  state err {e_s:.3e}")
    tol = TOL[wl.dtype]
    assert e_o < tol, f"output error {e_o:.3e}"
    assert e_s < tol, f"final state error {e_s:.3e}"
    return o, S


def test_prefill_tiny_f32(kda):
    check(kda, synth.TINY_F32)


def test_prefill_8k_bf16(kda):
    check(kda, synth.PREFILL_8K)


LENS = (0, 1, 63, 64, 65, 130, 300, 17)


@pytest.mark.parametrize("dk,dv,dtype", [(128, 128, "bf16"), (64, 64, "bf16"), (32, 32, "bf16"),
                                         (128, 32, "bf16"), (32, 128, "bf16"), (64, 128, "bf16"),
                                         (32, 32, "f32"), (32, 64, "f32"),
                                         # fp32 shapes of the token-serial kernel
                                         (128, 128, "f32"), (64, 64, "f32"), (32, 128, "f32"), (64, 32, "f32"),
                                         (64, 128, "f32"), (128, 32, "f32"), (128, 64, "f32")])
def test_prefill_varlen_dims(kda, dk, dv, dtype):
    wl = synth.VARLEN_64.with_(H=3, dk=dk, dv=dv, dtype=dtype, seqlens=LENS, state_std=0.1)
    check(kda, wl)


@pytest.mark.parametrize("warm", [-1, 0, 64])
@pytest.mark.parametrize("seg", [1, 2, 3])
@pytest.mark.parametrize("zshift", [0.0, -3.0])
def test_prefill_segmented(kda, seg, zshift, warm):
    """Segments of `seg` chunks, each given its incoming state by a warm-up
    window (default 128 tokens, or 64: windows that reach the sequence start run
    from the initial state, the others check their transition; with the weak
    decay of z - 3 the exact passes take over) or by the exact passes alone
    (warm = 0: transition/zero-state summary, scan, rerun)."""
    wl = synth.VARLEN_64.with_(H=4, seqlens=(700, 0, 64, 129, 1000, 5), state_std=0.1,
                               z_shift=zshift)
    check(kda, wl, seg=seg, tag=f"zshift={zshift}", warm=warm)


@pytest.mark.parametrize("warm", [-1, 0])
@pytest.mark.parametrize("dv", [32, 64])
def test_prefill_segmented_f32(kda, dv, warm):
    """fp32 storage through the segment passes (fp32 tolerance)."""
    wl = synth.TINY_F32.with_(H=3, dv=dv, seqlens=(700, 3, 450), state_std=0.1, z_shift=-2.0)
    check(kda, wl, seg=2, warm=warm)


def test_prefill_weak_decay_long(kda):
    """z shifted by -3 (alpha ~ 0.7): the incoming state and early tokens still
    matter thousands of tokens later."""
    wl = synth.PREFILL_8K.with_(H=4, seqlens=(4096,), z_shift=-3.0, state_std=0.1)
    check(kda, wl)
    check(kda, wl, seg=4, tag="seg4")
    check(kda, wl, seg=4, tag="seg4 exact passes", warm=0)


@pytest.mark.parametrize("warm", [-1, 0])
@pytest.mark.parametrize("case", ["beta0", "alpha1", "gmin", "alpha1_beta1_orthonormal"])
@pytest.mark.parametrize("dtype,dk", [("bf16", 32), ("f32", 32), ("f32", 64)])  # fp32 at 64: the serial path
def test_prefill_special_values(kda, case, dtype, dk, warm):
    """Exact edge values of the decay and the write strength, given to
    kda_prefill directly: beta = 0 (pure per-channel decay), g = 0 (alpha = 1,
    no forgetting), g = -5 everywhere (the strongest decay the gate allows),
    and alpha = beta = 1 with orthonormal keys (exact recall of every value).
    Segments of 2 chunks, so the warm-up windows (the transition of g = -5
    vanishes; without decay it never does and the exact passes take over) and
    the summary pass and scan (warm = 0) see them too."""
    import torch
    dv = dk
    # weak decay for beta = 0 (z shifted by -4), so the decayed state stays far
    # above the fp32 underflow over 300 tokens and the relative error means something
    wl = synth.VARLEN_64.with_(H=2, dk=dk, dv=dv, dtype=dtype, seqlens=(300, 130), state_std=0.1,
                               z_shift=-4.0 if case == "beta0" else 0.0)
    announce(f"prefill special values {case} {dtype}")
    x = synth.prefill_inputs(wl)
    T = wl.T_total
    S0 = synth.initial_state(wl)
    g = np.zeros((T, wl.H, dk), dtype=np.float32)
    if case == "beta0":
        x["beta"] = np.zeros_like(x["beta"])
        g = oracle.gate(x["z"], x["A"], round_bf16=(dtype == "bf16")).astype(np.float32)
    elif case == "gmin":
        g[:] = -5.0
    elif case == "alpha1_beta1_orthonormal":
        # per sequence and head, keys = rows of an orthogonal matrix (<= d_k of them)
        rng = np.random.default_rng(5)
        wl = wl.with_(seqlens=(dk, 17))
        T = wl.T_total
        x = {n: a[:T] for n, a in x.items() if n != "A"} | {"A": x["A"]}
        g = np.zeros((T, wl.H, dk), dtype=np.float32)
        x["beta"] = np.ones((T, wl.H), dtype=np.float32)
        for a, b in zip(wl.cu_seqlens[:-1], wl.cu_seqlens[1:]):
            for h in range(wl.H):
                qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
                x["k"][a:b, h] = qm[: b - a]
                x["q"][a:b, h] = qm[: b - a]  # query each key back
        if dtype == "bf16":  # keys must be exact in the storage dtype
            for n in ("q", "k"):
                x[n] = oracle.round_bf16(x[n]).astype(np.float32)
        S0 = np.zeros_like(synth.initial_state(wl))
    cu = torch.from_numpy(wl.cu_seqlens).to("cuda")
    o, S, _, _ = kda.kda_test_prefill(dev(x["q"], dtype), dev(x["k"], dtype), dev(x["v"], dtype), dev(g, dtype),
                                      dev(x["beta"], dtype), cu_seqlens=cu, initial_state=dev(S0), seg_chunks=2,
                                      warm_tokens=warm)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.prefill(x["q"], x["k"], x["v"], g, x["beta"], cu=wl.cu_seqlens, S0=S0)
    tol = TOL[dtype]
    assert relerr(host(o), o_ref) < tol and relerr(host(S), S_ref) < tol
    if case == "beta0":  # closed form: the state only decays, channel by channel
        for n, (a, b) in enumerate(zip(wl.cu_seqlens[:-1], wl.cu_seqlens[1:])):
            decay = np.exp(np.sum(g[a:b].astype(np.float64), axis=0))  # [H, dk]
            assert relerr(host(S[n]), decay[:, :, None] * S0[n]) < tol
    if case == "alpha1_beta1_orthonormal" and dtype == "f32":  # exact recall: o_t = v_t
        assert relerr(host(o), x["v"]) < tol


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128)])
def test_prefill_f32_serial_long(kda, dk, dv):
    """The token-serial fp32 path over one 3000-token sequence with the weak
    decay of z - 3 (the incoming state and early tokens still matter at the
    end), and the same sequence split in two calls chained through the final
    state, in place (initial_state is final_state)."""
    import torch
    wl = synth.TINY_F32.with_(H=2, dk=dk, dv=dv, seqlens=(3000,), z_shift=-3.0, state_std=0.1)
    o, S = check(kda, wl, tag="serial long")
    x = synth.prefill_inputs(wl)
    S0 = synth.initial_state(wl)
    g = kda.kda_gate(dev(x["z"]), dev(x["A"]))
    St = dev(S0)
    outs = []
    for a, b in ((0, 1700), (1700, 3000)):
        sl = lambda name: dev(x[name][a:b])
        oo, _ = kda.kda_prefill(sl("q"), sl("k"), sl("v"), g[a:b].contiguous(), sl("beta"), initial_state=St,
                                final_state=St)
        outs.append(oo)
    torch.cuda.synchronize()
    # the same arithmetic token by token: split calls equal one call exactly
    assert np.array_equal(host(torch.cat(outs)), o)
    assert np.array_equal(host(St), S)


@pytest.mark.parametrize("warm", [-1, 0])
@pytest.mark.parametrize("zshift", [0.0, -3.0])
def test_prefill_f32_serial_segments(kda, zshift, warm):
    """The token-serial path over packed sequences cut into segments of 2
    chunks: warm-up windows (flagged chains, which the weak decay of z - 3
    makes, rerun whole) or none (warm = 0: every chain reruns whole)."""
    wl = synth.TINY_F32.with_(H=3, dk=128, dv=64, seqlens=(700, 0, 129, 1000, 5), state_std=0.1,
                              z_shift=zshift)
    check(kda, wl, seg=2, tag=f"serial zshift={zshift}", warm=warm)
