"""Helpers shared by the GPU parity tests: device copies of the seeded inputs
and the error measure (normwise max relative error, max|x - y| / max|y|)."""
from __future__ import annotations

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def torch_dtype(name):
    import torch
    return torch.bfloat16 if name == "bf16" else torch.float32


def dev(x: np.ndarray, dtype: str = "f32"):
    """float32 numpy array (exact in `dtype`) -> device tensor of that dtype."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")
    return t.to(torch_dtype(dtype)) if dtype == "bf16" else t


def dev_unaligned(t):
    """The same values in a contiguous device tensor whose data starts one
    element past a 16-byte boundary (exercises the kernels for unaligned
    token tensors)."""
    import torch
    flat = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
    out = flat[1:1 + t.numel()].view(t.shape)
    out.copy_(t)
    assert out.data_ptr() % 16 != 0
    return out


def host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def relerr(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    if want.size == 0:
        return 0.0
    assert np.all(np.isfinite(got)), "non-finite values from the GPU"
    scale = np.max(np.abs(want))
    return float(np.max(np.abs(got - want)) / max(scale, 1e-300))


def announce(msg: str):
    print(f"[case] {msg}", flush=True)


def dev_stream(wl, name: str, set_index: int = 0, rows: int = 1 << 16):
    """A token tensor of a (possibly very long) workload, generated in windows of
    `rows` tokens straight into a device tensor of the workload's dtype, so the
    host never holds the whole fp32 copy."""
    import torch
    import synth
    T = wl.T_total
    shape = (T,) + synth._shape(wl, name, 1)[1:]
    out = torch.empty(shape, dtype=torch_dtype(wl.dtype), device="cuda")
    for t0 in range(0, T, rows):
        t1 = min(T, t0 + rows)
        x = torch.from_numpy(synth.token_rows(wl, name, t0, t1, set_index))
        out[t0:t1].copy_(x.to(torch_dtype(wl.dtype)))
    return out


def gated_prefill(kda, q, k, v, z, A, beta, seg=None, warm=-1, interval=0, **kw):
    """kda_prefill_gated; with a forced segment length (chunks) or warm-up
    window (tokens; 0 = the exact passes only) through the test entry point
    that takes the planner's choices as arguments.  Returns (o, S) or, with a
    checkpoint interval, (o, S, ckpt)."""
    if seg is None and warm == -1:
        return kda.kda_prefill_gated(q, k, v, z, A, beta, interval=interval, **kw)
    kw.pop("want_final_state", None)
    o, S, ck, _ = kda.kda_test_prefill(q, k, v, z, beta, A=A, interval=interval, seg_chunks=seg or 0,
                                       warm_tokens=warm, **kw)
    return (o, S, ck) if interval > 0 else (o, S)


_native = None


def native_oracle():
    """The oracle compiled for the host the tests run on (gcc -O3
    -march=native, into a temporary directory): the same source as the
    portable copy, faster on the full-size workloads."""
    global _native
    if _native is None:
        import os
        import tempfile
        import oracle
        out = os.path.join(tempfile.mkdtemp(prefix="kda_oracle_"), "liboracle_native.so")
        oracle.build(out=out, native=True)
        _native = oracle.load(out)
    return _native
