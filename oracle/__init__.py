"""KDA fp64 CPU oracle (ctypes binding of oracle/kda_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg import this package; the product path never does.  It shares
no code with the HIP library: both sides consume the same seeded inputs from
`synth` and nothing else.

What each function computes, and which passage it follows, is stated in
kda_oracle.c.  Arrays are converted to contiguous float64 before the call.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kda_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

_lib = None


def build(src: str = SRC, out: str = LIB, native: bool = False) -> str:
    """Compile the oracle with gcc and OpenMP: -O2 for a portable x86-64-v3
    target (the copy the tests load, which may run on another host than the
    one it was built on), or -O3 -march=native for the host it is built on
    (the benchmark's CPU baseline builds its own)."""
    arch = ["-O3", "-march=native"] if native else ["-O2", "-march=x86-64-v3"]
    cmd = ["gcc", *arch, "-fopenmp", "-fPIC", "-shared",
           "-std=c11", "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    P = ctypes.c_void_p
    I, L, D = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.oracle_gate.argtypes = [P, P, L, I, I, D, P]
    lib.oracle_prefill.argtypes = [P, P, P, P, P, P, I, I, I, I, P, P, P, I]
    lib.oracle_prefill_chunked.argtypes = [P, P, P, P, P, P, I, I, I, I, I, P, P, P, I]
    lib.oracle_decode_step.argtypes = [P, P, P, P, P, P, P, I, I, I, I]
    lib.oracle_wy_T.argtypes = [P, P, P, I, I, P]
    lib.oracle_round_bf16.argtypes = [P, L]
    lib.oracle_backward.argtypes = [P, P, P, P, P, P, I, I, I, I, P, P, P, P, P, P, P, P, P, I]
    for f in ("oracle_gate", "oracle_prefill", "oracle_prefill_chunked",
              "oracle_decode_step", "oracle_wy_T", "oracle_round_bf16", "oracle_backward"):
        getattr(lib, f).restype = None
    return lib


def load(path: str | None = None) -> ctypes.CDLL:
    """Load (building first if absent) the oracle library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _lib = _bind(ctypes.CDLL(LIB))
    return _lib


def _d(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64)


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def gate(z, A, g_min: float = -5.0, round_bf16: bool = False, lib=None) -> np.ndarray:
    """g = g_min * sigmoid(exp(A_h) z) in fp64 for z [T, H, dk], A [H].

    With round_bf16, the result is then rounded once to the nearest bf16: the
    value a bf16-output gate must return."""
    lib = lib or load()
    z = _d(z)
    A = _d(A)
    T, H, dk = z.shape
    g = np.empty_like(z)
    lib.oracle_gate(_p(z), _p(A), T, H, dk, float(g_min), _p(g))
    if round_bf16:
        lib.oracle_round_bf16(_p(g), g.size)
    return g


def round_bf16(x, lib=None) -> np.ndarray:
    lib = lib or load()
    x = _d(x).copy()
    lib.oracle_round_bf16(_p(x), x.size)
    return x


def _cu(cu, T):
    if cu is None:
        return np.array([0, T], dtype=np.int64)
    return np.ascontiguousarray(cu, dtype=np.int64)


def prefill(q, k, v, g, beta, cu=None, S0=None, chunk: int | None = None,
            want_o: bool = True, threads: int | None = None, lib=None):
    """Token-serial recurrence (chunk=None) or the chunkwise self-check form.

    q, k, g: [T, H, dk]; v: [T, H, dv]; beta: [T, H]; cu: [N+1] or None;
    S0: [N, H, dk, dv] or None.  Returns (o [T, H, dv] or None, S [N, H, dk, dv])."""
    lib = lib or load()
    q, k, v, g, beta = _d(q), _d(k), _d(v), _d(g), _d(beta)
    T, H, dk = k.shape
    dv = v.shape[2]
    cu = _cu(cu, T)
    N = cu.shape[0] - 1
    S0 = None if S0 is None else _d(S0)
    o = np.empty((T, H, dv)) if want_o else None
    S = np.empty((N, H, dk, dv))
    th = threads or default_threads()
    if chunk is None:
        lib.oracle_prefill(_p(q), _p(k), _p(v), _p(g), _p(beta), _p(cu), N, H, dk, dv,
                           _p(S0), _p(o), _p(S), th)
    else:
        lib.oracle_prefill_chunked(_p(q), _p(k), _p(v), _p(g), _p(beta), _p(cu), N, H, dk,
                                   dv, int(chunk), _p(S0), _p(o), _p(S), th)
    return o, S


def decode_step(q, k, v, g, beta, S, lib=None):
    """One token per (b, h) against states S [B, H, dk, dv]; returns (o, S_new)."""
    lib = lib or load()
    q, k, v, g, beta = _d(q), _d(k), _d(v), _d(g), _d(beta)
    S = _d(S).copy()
    B, H, dk = k.shape
    dv = v.shape[2]
    o = np.empty((B, H, dv))
    lib.oracle_decode_step(_p(q), _p(k), _p(v), _p(g), _p(beta), _p(S), _p(o), B, H, dk, dv)
    return o, S


def backward(q, k, v, g, beta, dO=None, dS_fin=None, cu=None, S0=None, threads: int | None = None,
             lib=None) -> dict:
    """Gradients of L = sum_t <dO_t, o_t> + <dS_fin, S_T> for the token-serial
    recurrence (every state of a sequence is kept: small cases).  Returns a dict
    with dq, dk, dg [T, H, dk], dv [T, H, dv], dbeta [T, H], dS0 [N, H, dk, dv]."""
    lib = lib or load()
    q, k, v, g, beta = _d(q), _d(k), _d(v), _d(g), _d(beta)
    T, H, dk = k.shape
    dv = v.shape[2]
    cu = _cu(cu, T)
    N = cu.shape[0] - 1
    S0 = None if S0 is None else _d(S0)
    dO = None if dO is None else _d(dO)
    dS_fin = None if dS_fin is None else _d(dS_fin)
    out = {"dq": np.empty((T, H, dk)), "dk": np.empty((T, H, dk)), "dv": np.empty((T, H, dv)),
           "dg": np.empty((T, H, dk)), "dbeta": np.empty((T, H)), "dS0": np.empty((N, H, dk, dv))}
    lib.oracle_backward(_p(q), _p(k), _p(v), _p(g), _p(beta), _p(cu), N, H, dk, dv, _p(S0), _p(dO), _p(dS_fin),
                        _p(out["dq"]), _p(out["dk"]), _p(out["dv"]), _p(out["dg"]), _p(out["dbeta"]),
                        _p(out["dS0"]), threads or default_threads())
    return out


def wy_T(k, g, beta, lib=None) -> np.ndarray:
    """T = (I + A)^{-1} Diag(beta) for one chunk: k, g [L, dk], beta [L]."""
    lib = lib or load()
    k, g, beta = _d(k), _d(g), _d(beta)
    L, dk = k.shape
    T = np.empty((L, L))
    lib.oracle_wy_T(_p(k), _p(g), _p(beta), L, dk, _p(T))
    return T
