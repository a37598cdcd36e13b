"""GPU parity of kda_backward against the fp64 reverse-mode oracle (itself
pinned by finite differences of the forward recurrence).

The backward's products take their operands in the input precision, as the
forward's do (bf16 operands with fp32 accumulation for bf16 inputs, fp32 for
fp32 inputs), so each case is held to its dtype's tolerance."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import TOL, announce, dev, host, relerr

pytestmark = pytest.mark.gpu

GRADS = (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dg", "dg"), ("dbeta", "dbeta"), ("d_initial_state", "dS0"))


@pytest.fixture(scope="module")
def kda():
    import torch
    import linear_attention_sequence_gate_amd as m
    assert torch.cuda.is_available()
    m.lib()
    return m


def run_case(kda, wl, with_ckpt, heads=None, seed=5, interval=64, seg_tokens=None, warm_tokens=-1):
    """GPU backward of the prefill on wl's inputs (gate applied on the host by
    the oracle, so both sides take the same g), against the oracle on `heads`."""
    import torch
    dt = wl.dtype
    x = synth.prefill_inputs(wl)
    g = oracle.gate(x["z"], x["A"])
    if dt == "bf16":
        g = oracle.round_bf16(g)
    rng = np.random.default_rng(seed)
    S0 = synth.initial_state(wl) if wl.state_std > 0 else None
    dO = rng.standard_normal((wl.T_total, wl.H, wl.dv)).astype(np.float32)
    if dt == "bf16":
        dO = oracle.round_bf16(dO).astype(np.float32)
    dS = rng.standard_normal((wl.N, wl.H, wl.dk, wl.dv)).astype(np.float32)
    cu = torch.from_numpy(wl.cu_seqlens).cuda() if wl.N > 1 else None
    d = {n: dev(x[n], dt) for n in ("q", "k", "v", "beta")}
    d["g"] = dev(g, dt)
    S0d = None if S0 is None else dev(S0)
    ck = None
    if with_ckpt:
        _, _, ck = kda.kda_prefill_ckpt(d["q"], d["k"], d["v"], d["g"], d["beta"], interval, cu_seqlens=cu,
                                        cu_seqlens_host=wl.cu_seqlens if wl.N > 1 else None,
                                        initial_state=S0d)
    out = kda.kda_backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d_o=dev(dO, dt), d_final_state=dev(dS),
                           cu_seqlens=cu, initial_state=S0d, ckpt=ck, interval=interval, seg_tokens=seg_tokens,
                           warm_tokens=warm_tokens)
    torch.cuda.synchronize()
    hs = list(range(wl.H)) if heads is None else heads
    sel = lambda a: a[:, hs]
    ref = oracle.backward(sel(x["q"]), sel(x["k"]), sel(x["v"]), sel(g), sel(x["beta"]), dO=sel(dO),
                          dS_fin=dS[:, hs], cu=wl.cu_seqlens, S0=None if S0 is None else S0[:, hs])
    tol = TOL[dt]
    for gname, rname in GRADS:
        got = host(out[gname])[:, hs]
        e = relerr(got, ref[rname])
        print(f"  {gname}: {e:.3e}")
        assert e < tol, f"{gname}: {e:.3e} >= {tol}"


@pytest.mark.parametrize("with_ckpt", [False, True])
@pytest.mark.parametrize("dk,dv,dtype", [(32, 32, "f32"), (32, 64, "f32"), (64, 64, "bf16"),
                                         (128, 128, "bf16"), (128, 32, "bf16"), (32, 128, "bf16"),
                                         (128, 128, "f32"), (64, 128, "f32"), (128, 64, "f32")])
def test_backward_varlen(kda, dk, dv, dtype, with_ckpt):
    wl = synth.VARLEN_64.with_(H=2, dk=dk, dv=dv, dtype=dtype, seqlens=(0, 1, 63, 64, 65, 200),
                               state_std=0.1, z_shift=-2.0)
    announce(f"backward dk={dk} dv={dv} {dtype} ckpt={with_ckpt} lens={wl.seqlens}")
    run_case(kda, wl, with_ckpt)


def test_backward_no_initial_state(kda):
    wl = synth.TINY_F32.with_(H=3, seqlens=(150,))
    announce("backward, zero initial state, one sequence")
    run_case(kda, wl, with_ckpt=True)


@pytest.mark.parametrize("warm", [-1, 0])
def test_backward_8k_sampled_heads(kda, warm):
    """The 8K workload's shape (H=32, d=128, bf16) with the forward's checkpoints;
    two heads against the oracle; segment end gradients from the windows (the
    default) or from the summary pass and scan."""
    wl = synth.PREFILL_8K.with_(state_std=0.1)
    announce(f"backward 8K, heads 3 and 29, window {warm}")
    run_case(kda, wl, with_ckpt=True, heads=[3, 29], warm_tokens=warm)


@pytest.mark.parametrize("warm", [-1, 0, 32])
@pytest.mark.parametrize("zshift", [0.0, -2.0])
@pytest.mark.parametrize("seg_tokens", [64, 192, 100000])
def test_backward_segment_lengths(kda, seg_tokens, zshift, warm):
    """Segments of 1 and 3 chunks and one segment per sequence, through the
    test entry point; each segment's end gradient from a window after it (128
    or 32 tokens; windows that reach a sequence's end start from the final
    state's gradient; with the slower decay of z - 2 the summary pass and scan
    take over) or from the summary pass and scan alone (warm = 0)."""
    wl = synth.VARLEN_64.with_(H=2, dk=64, dv=32, dtype="f32", seqlens=(500, 0, 64, 129),
                               state_std=0.1, z_shift=zshift)
    announce(f"backward segments of {seg_tokens} tokens, z shift {zshift}, window {warm}")
    run_case(kda, wl, with_ckpt=False, seg_tokens=seg_tokens, warm_tokens=warm)


@pytest.mark.parametrize("interval", [128, 512])
def test_backward_sparse_checkpoints(kda, interval):
    """Checkpoints every 128 or 512 tokens (the prefix cache's block): each
    64-token chunk rebuilds its state from the nearest earlier row; varlen
    lengths on both sides of the interval, segments of 3 chunks."""
    wl = synth.VARLEN_64.with_(H=2, dk=64, dv=64, dtype="bf16", seqlens=(1500, 0, 511, 512, 700),
                               state_std=0.1, z_shift=-2.0)
    announce(f"backward from interval-{interval} checkpoints")
    run_case(kda, wl, with_ckpt=True, interval=interval, seg_tokens=192)


def test_backward_truncated_checkpoints(kda):
    """A checkpoint buffer shorter than the forward wrote (rows past its end
    are missing): the chunks past it rebuild from the last row it holds, or
    from the initial state for sequences with no row in it."""
    import torch
    wl = synth.VARLEN_64.with_(H=2, dk=32, dv=32, dtype="f32", seqlens=(700, 300), state_std=0.1, z_shift=-2.0)
    announce("backward, truncated checkpoint buffer")
    x = synth.prefill_inputs(wl)
    g = oracle.gate(x["z"], x["A"])
    rng = np.random.default_rng(9)
    S0 = synth.initial_state(wl)
    dO = rng.standard_normal((wl.T_total, wl.H, wl.dv)).astype(np.float32)
    dS = rng.standard_normal((wl.N, wl.H, wl.dk, wl.dv)).astype(np.float32)
    cu = torch.from_numpy(wl.cu_seqlens).cuda()
    d = {n: dev(x[n]) for n in ("q", "k", "v", "beta")}
    d["g"] = dev(g)
    _, _, ck = kda.kda_prefill_ckpt(d["q"], d["k"], d["v"], d["g"], d["beta"], 128, cu_seqlens=cu,
                                    cu_seqlens_host=wl.cu_seqlens, initial_state=dev(S0))
    assert ck.shape[0] == 5 + 2
    out = kda.kda_backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d_o=dev(dO), d_final_state=dev(dS),
                           cu_seqlens=cu, initial_state=dev(S0), ckpt=ck[:3].contiguous(), interval=128)
    torch.cuda.synchronize()
    ref = oracle.backward(x["q"], x["k"], x["v"], g, x["beta"], dO=dO, dS_fin=dS, cu=wl.cu_seqlens, S0=S0)
    for gname, rname in GRADS:
        e = relerr(host(out[gname]), ref[rname])
        print(f"  {gname}: {e:.3e}")
        assert e < TOL["f32"]


def test_backward_many_heads(kda):
    """N * H >= 128: the planner's one-segment-per-sequence path."""
    wl = synth.VARLEN_64.with_(H=64, dk=32, dv=32, dtype="f32", seqlens=(70, 130), state_std=0.1)
    announce("backward, 2 sequences x 64 heads")
    run_case(kda, wl, with_ckpt=True, heads=[0, 33, 63])


def test_backward_varlen_64_full_size(kda):
    """The ~1M-token varlen workload (64 sequences, H=32, bf16) through the
    forward's interval-64 checkpoints and the backward: N*H = 2048 items, one
    segment per sequence, every workgroup looping over items.  dO and the final
    state's gradient are nonzero on the three shortest sequences only (the
    oracle keeps every state of a sequence, so it takes short ones): their
    gradients on three heads against the oracle, and another sequence's
    gradients exactly zero (nothing leaks across sequences)."""
    import torch
    from tests.gpu_common import dev_stream
    wl = synth.VARLEN_64
    T, H, dk, dv = wl.T_total, wl.H, wl.dk, wl.dv
    cu = wl.cu_seqlens
    lens = np.asarray(wl.seqlens)
    announce(f"backward varlen_64 full size: N={wl.N} H={H} T={T}")
    xs = {n: dev_stream(wl, n, rows=1 << 14) for n in ("q", "k", "v", "z", "beta")}
    g = kda.kda_gate(xs["z"], dev(synth.gate_A(wl)))
    del xs["z"]
    S0 = synth.initial_state(wl)
    cud = torch.from_numpy(cu).cuda()
    S0d = dev(S0)
    _, _, ck = kda.kda_prefill_ckpt(xs["q"], xs["k"], xs["v"], g, xs["beta"], 64, cu_seqlens=cud,
                                    cu_seqlens_host=cu, initial_state=S0d)
    order = np.argsort(lens)
    picked = [int(n) for n in order[:3]]
    rng = np.random.default_rng(17)
    dO = torch.zeros((T, H, dv), dtype=torch.bfloat16, device="cuda")
    dS = torch.zeros((wl.N, H, dk, dv), dtype=torch.float32, device="cuda")
    up = {}
    for n in picked:
        a, b = int(cu[n]), int(cu[n + 1])
        do_n = oracle.round_bf16(rng.standard_normal((b - a, H, dv)).astype(np.float32)).astype(np.float32)
        ds_n = rng.standard_normal((H, dk, dv)).astype(np.float32)
        dO[a:b] = dev(do_n, "bf16")
        dS[n] = dev(ds_n)
        up[n] = (do_n, ds_n)
    out = kda.kda_backward(xs["q"], xs["k"], xs["v"], g, xs["beta"], d_o=dO, d_final_state=dS, cu_seqlens=cud,
                           initial_state=S0d, ckpt=ck)
    torch.cuda.synchronize()
    del ck
    heads = [0, 13, 31]
    for n in picked:
        a, b = int(cu[n]), int(cu[n + 1])
        x = {nm: synth.token_rows(wl, nm, a, b)[:, heads] for nm in ("q", "k", "v", "z", "beta")}
        gh = oracle.gate(x["z"], synth.gate_A(wl)[heads], round_bf16=True)
        do_n, ds_n = up[n]
        ref = oracle.backward(x["q"], x["k"], x["v"], gh, x["beta"], dO=do_n[:, heads], dS_fin=ds_n[None, heads],
                              S0=S0[n:n + 1][:, heads])
        for gname, rname in GRADS:
            got = host(out[gname][n:n + 1] if gname == "d_initial_state" else out[gname][a:b])[:, heads]
            e = relerr(got, ref[rname])
            print(f"  sequence {n} (len {b - a}) {gname}: {e:.3e}")
            assert e < TOL["bf16"], f"sequence {n} {gname}: {e:.3e}"
    quiet = int(order[-1])  # the longest sequence, whose upstream gradients are zero
    a, b = int(cu[quiet]), int(cu[quiet + 1])
    for gname, _ in GRADS:
        t = out[gname][quiet] if gname == "d_initial_state" else out[gname][a:b]
        assert torch.count_nonzero(t).item() == 0, f"{gname} leaks into sequence {quiet}"
        assert torch.isfinite(out[gname]).all()


@pytest.mark.parametrize("which", ["none", "final_only", "output_only"])
def test_backward_optional_gradients(kda, which):
    """d_o and d_final_state may be omitted (zero): with neither, every gradient
    is exactly zero; with one, the result matches the oracle given zeros for
    the other."""
    import torch
    wl = synth.VARLEN_64.with_(H=2, dk=64, dv=64, dtype="bf16", seqlens=(150, 300), state_std=0.1,
                               z_shift=-2.0)
    announce(f"backward with optional upstream gradients: {which}")
    x = synth.prefill_inputs(wl)
    g = oracle.round_bf16(oracle.gate(x["z"], x["A"]))
    S0 = synth.initial_state(wl)
    rng = np.random.default_rng(23)
    dO = oracle.round_bf16(rng.standard_normal((wl.T_total, wl.H, wl.dv)).astype(np.float32)).astype(np.float32)
    dS = rng.standard_normal((wl.N, wl.H, wl.dk, wl.dv)).astype(np.float32)
    use_o, use_s = which == "output_only", which == "final_only"
    d = {n: dev(x[n], "bf16") for n in ("q", "k", "v", "beta")}
    out = kda.kda_backward(d["q"], d["k"], d["v"], dev(g, "bf16"), d["beta"],
                           d_o=dev(dO, "bf16") if use_o else None, d_final_state=dev(dS) if use_s else None,
                           cu_seqlens=torch.from_numpy(wl.cu_seqlens).cuda(), initial_state=dev(S0))
    torch.cuda.synchronize()
    if which == "none":
        for gname, _ in GRADS:
            assert torch.count_nonzero(out[gname]).item() == 0, gname
        return
    ref = oracle.backward(x["q"], x["k"], x["v"], g, x["beta"], dO=dO if use_o else np.zeros_like(dO),
                          dS_fin=dS if use_s else np.zeros_like(dS), cu=wl.cu_seqlens, S0=S0)
    for gname, rname in GRADS:
        e = relerr(host(out[gname]), ref[rname])
        print(f"  {gname}: {e:.3e}")
        assert e < TOL["bf16"], f"{gname}: {e:.3e}"
