"""Seeded synthetic inputs for the KDA workloads.

This module is shared by the tests, the benchmark and the oracle's callers. It
holds no step of the method itself: it draws q, k, v, beta, the gate
pre-activation z, the per-head gate parameter A, initial states and sequence
lengths, and rounds them to the storage dtype.  The log-decay g is NOT made
here: each side (HIP path, fp64 oracle) applies the gate to z and A itself.

Value recipes (one workload per named configuration):
  q, k  ~ N(0, 1), then L2-normalised over the channel axis per (token, head)
  v     ~ N(0, 1)
  beta  = 1 / (1 + exp(-N(0, 1)))          (a draw in (0, 1), per token and head)
  z     ~ N(z_shift, 1)
  A_h   ~ U(-1, 1), one per head, fp32
  S_0   ~ N(0, state_std^2) fp32, or zeros when state_std == 0
  varlen lengths: round(exp(U(ln 1024, ln 65536)))

Token-indexed tensors are drawn in blocks of BLOCK tokens, each from its own
seed (workload seed, tensor id, set index, block index), so any window of a long
input can be regenerated without drawing the rest.  For bf16 workloads every
value is rounded to the nearest bf16 (ties to even) and returned as float32
holding that exact value, so the device copy and the fp64 upcast see the same
bits.
"""
from __future__ import annotations

import concurrent.futures as _cf
import math
import os
from dataclasses import dataclass

import numpy as np

BLOCK = 4096
_TENSOR_ID = {"q": 1, "k": 2, "v": 3, "z": 4, "beta": 5}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) & np.uint32(0xFFFF0000)).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-exact."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


@dataclass(frozen=True)
class Workload:
    name: str
    H: int
    dk: int
    dv: int
    seqlens: tuple
    dtype: str  # "f32" or "bf16"
    chunk: int = 64
    z_shift: float = 0.0
    state_std: float = 0.0
    seed: int = 1000

    @property
    def N(self) -> int:
        return len(self.seqlens)

    @property
    def T_total(self) -> int:
        return int(sum(self.seqlens))

    @property
    def cu_seqlens(self) -> np.ndarray:
        cu = np.zeros(self.N + 1, dtype=np.int64)
        cu[1:] = np.cumsum(np.asarray(self.seqlens, dtype=np.int64))
        return cu.astype(np.int32)

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


def varlen_lengths(n: int, lo: int, hi: int, seed: int) -> tuple:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 99])))
    x = rng.uniform(math.log(lo), math.log(hi), size=n)
    return tuple(int(v) for v in np.rint(np.exp(x)))


# The five named workloads (the shapes of the method's target configurations).
TINY_F32 = Workload("tiny_f32", H=2, dk=32, dv=32, seqlens=(256,), dtype="f32", seed=1000)
PREFILL_8K = Workload("prefill_8k", H=32, dk=128, dv=128, seqlens=(8192,), dtype="bf16", seed=1001)
PREFILL_1M = Workload("prefill_1m", H=8, dk=128, dv=128, seqlens=(1 << 20,), dtype="bf16",
                      z_shift=3.0, seed=1002)
DECODE_B256 = Workload("decode_b256", H=32, dk=128, dv=128, seqlens=(1,) * 256, dtype="bf16",
                       state_std=0.1, seed=1003)
# lengths drawn with seed 1015: the first seed from 1004 up whose 64 lengths sum
# to within 3% of the ~1M tokens the workload describes (1,026,790 tokens)
VARLEN_64 = Workload("varlen_64", H=32, dk=128, dv=128,
                     seqlens=varlen_lengths(64, 1024, 65536, 1015), dtype="bf16",
                     state_std=0.1, seed=1004)

# speculative decode: K = 4 draft tokens for each of the 256 sequences of the
# decode workload (token tensors [B, K, H, d] are the packed [B*K, H, d] rows)
VERIFY_B256_K4 = Workload("verify_b256_k4", H=32, dk=128, dv=128, seqlens=(4,) * 256, dtype="bf16",
                          state_std=0.1, seed=1005)

WORKLOADS = {w.name: w for w in (TINY_F32, PREFILL_8K, PREFILL_1M, DECODE_B256, VARLEN_64, VERIFY_B256_K4)}


def _gen(wl: Workload, name: str, set_index: int, block: int) -> np.random.Generator:
    ss = np.random.SeedSequence([wl.seed, _TENSOR_ID[name], set_index, block])
    return np.random.Generator(np.random.PCG64(ss))


def _draw_block(wl: Workload, name: str, set_index: int, block: int, rows: int) -> np.ndarray:
    rng = _gen(wl, name, set_index, block)
    if name in ("q", "k"):
        x = rng.standard_normal((rows, wl.H, wl.dk), dtype=np.float32)
        nrm = np.sqrt(np.einsum("thc,thc->th", x, x, dtype=np.float64))
        x = (x / nrm[..., None]).astype(np.float32)
    elif name == "v":
        x = rng.standard_normal((rows, wl.H, wl.dv), dtype=np.float32)
    elif name == "z":
        x = rng.standard_normal((rows, wl.H, wl.dk), dtype=np.float32)
        if wl.z_shift:
            x += np.float32(wl.z_shift)
    elif name == "beta":
        n = rng.standard_normal((rows, wl.H), dtype=np.float64)
        x = (1.0 / (1.0 + np.exp(-n))).astype(np.float32)
    else:
        raise KeyError(name)
    return bf16_round(x) if wl.dtype == "bf16" else x


def _shape(wl: Workload, name: str, rows: int) -> tuple:
    if name == "beta":
        return (rows, wl.H)
    return (rows, wl.H, wl.dv if name == "v" else wl.dk)


def token_rows(wl: Workload, name: str, t0: int, t1: int, set_index: int = 0,
               threads: int | None = None) -> np.ndarray:
    """Rows [t0, t1) of a token-indexed tensor of the packed input (float32)."""
    t0, t1 = int(t0), int(t1)
    out = np.empty(_shape(wl, name, max(t1 - t0, 0)), dtype=np.float32)
    if t1 <= t0:
        return out
    b0, b1 = t0 // BLOCK, (t1 - 1) // BLOCK

    def work(b):
        lo, hi = max(b * BLOCK, t0), min((b + 1) * BLOCK, t1)
        blk = _draw_block(wl, name, set_index, b, BLOCK)
        out[lo - t0:hi - t0] = blk[lo - b * BLOCK:hi - b * BLOCK]

    nb = b1 - b0 + 1
    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if nb == 1 or threads <= 1:
        for b in range(b0, b1 + 1):
            work(b)
    else:
        with _cf.ThreadPoolExecutor(min(threads, nb)) as ex:
            list(ex.map(work, range(b0, b1 + 1)))
    return out


def gate_A(wl: Workload) -> np.ndarray:
    """Per-head gate parameter A_h ~ U(-1, 1), float32 [H]."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, 77])))
    return rng.uniform(-1.0, 1.0, size=wl.H).astype(np.float32)


def initial_state(wl: Workload, seq_lo: int = 0, seq_hi: int | None = None) -> np.ndarray:
    """fp32 initial states [seq_hi - seq_lo, H, dk, dv]; one seeded stream per sequence."""
    if seq_hi is None:
        seq_hi = wl.N
    out = np.zeros((seq_hi - seq_lo, wl.H, wl.dk, wl.dv), dtype=np.float32)
    if wl.state_std == 0.0:
        return out
    for i, s in enumerate(range(seq_lo, seq_hi)):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, 88, s])))
        out[i] = rng.standard_normal((wl.H, wl.dk, wl.dv), dtype=np.float32) * np.float32(wl.state_std)
    return out


def prefill_inputs(wl: Workload, t0: int = 0, t1: int | None = None, set_index: int = 0) -> dict:
    """All token tensors for rows [t0, t1) plus A (float32 arrays)."""
    if t1 is None:
        t1 = wl.T_total
    d = {n: token_rows(wl, n, t0, t1, set_index) for n in ("q", "k", "v", "z", "beta")}
    d["A"] = gate_A(wl)
    return d
