"""libkda's C ABI on the CPU: the library loads, exports every symbol the header
declares, and rejects bad arguments on the host before anything is launched.
No call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

import linear_attention_sequence_gate_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")
FAKE = 0x10000  # a non-null address; validation rejects the call before any use
BF16, F32 = kda.KDA_BF16, kda.KDA_F32


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return kda.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(kda.EXPORTED), names
    for n in names:
        assert hasattr(L, n), f"libkda does not export {n}"


def test_version_and_status_strings(L):
    assert kda.version() == 100
    for code, name in kda._STATUS.items():
        assert L.kda_status_string(code).decode() == name
    assert L.kda_status_string(99).decode() == "KDA_ERR_UNKNOWN"


def status(call):
    return call


def test_gate_validation(L):
    assert L.kda_gate(FAKE, FAKE, FAKE, -1, 2, 32, BF16, -5.0, None) == 1
    assert L.kda_gate(FAKE, FAKE, FAKE, 4, 0, 32, BF16, -5.0, None) == 1
    assert L.kda_gate(FAKE, FAKE, FAKE, 4, 2, 32, 7, -5.0, None) == 2
    assert L.kda_gate(FAKE, FAKE, FAKE, 4, 2, 32, BF16, 1.0, None) == 1
    assert L.kda_gate(FAKE, FAKE, FAKE, 4, 2, 32, BF16, float("nan"), None) == 1
    assert L.kda_gate(None, FAKE, FAKE, 4, 2, 32, BF16, -5.0, None) == 1
    assert b"null" in L.kda_last_error()
    # partial overlap of g with z (exact aliasing is allowed)
    assert L.kda_gate(FAKE, FAKE + 1 << 20, FAKE + 64, 4, 2, 32, BF16, -5.0, None) == 1
    # n_tokens == 0 is a no-op that succeeds without touching the device
    assert L.kda_gate(None, None, None, 0, 2, 32, BF16, -5.0, None) == 0


def test_decode_validation(L):
    base = dict(q=FAKE, k=FAKE + (1 << 20), v=FAKE + (2 << 20), g=FAKE + (3 << 20),
                beta=FAKE + (4 << 20), state=FAKE + (8 << 20), o=FAKE + (64 << 20))

    def call(**kw):
        a = dict(base, B=4, H=2, dk=128, dv=128, dt=BF16)
        a.update(kw)
        return L.kda_decode_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["state"], a["o"],
                                 a["B"], a["H"], a["dk"], a["dv"], a["dt"], None)

    assert call(B=-1) == 1
    assert call(H=0) == 1
    assert call(dk=48) == 2
    assert call(dv=256) == 2
    assert call(dt=5) == 2
    assert call(q=None) == 1
    assert call(state=FAKE + (8 << 20) + 4) == 1          # misaligned state
    assert call(o=FAKE + 16) == 1                          # o aliases q
    assert call(o=FAKE + (8 << 20)) == 1                   # o aliases the state
    assert call(state=FAKE + (3 << 20)) == 1               # state aliases g
    assert call(B=0, q=None, o=None) == 0                  # empty batch: no-op


def test_prefill_workspace_head_split(L, monkeypatch):
    """One long sequence whose segments leave compute units idle takes the head
    split: its workspace also holds the head's final state (fp32 [H][d_k][d_v]),
    and is never smaller than the unsplit plan's (a forced segment length turns
    the split off)."""
    ws = kda.kda_prefill_workspace_size
    split = ws(8192, 1, 32, 128, 128)
    monkeypatch.setenv("KDA_SEG_CHUNKS", "16")
    plain = ws(8192, 1, 32, 128, 128)
    monkeypatch.delenv("KDA_SEG_CHUNKS")
    assert split >= 32 * 128 * 128 * 4 and split >= plain
    assert ws(8192, 2, 32, 128, 128) > 0  # packed sequences: no split


def test_prefill_workspace_size(L):
    ws = kda.kda_prefill_workspace_size
    assert ws(8192, 1, 32, 128, 128) > 0
    assert ws(0, 1, 32, 128, 128) > 0
    assert ws(8192, 1, 32, 96, 128) == 0
    assert ws(8192, 1, 32, 128, 128, chunk=32) == 0
    assert ws(8192, 1, 32, 128, 128, dtype=F32) == 0      # fp32 needs d_k = 32
    assert ws(8192, 1, 32, 64, 64, dtype=F32) == 0
    assert ws(256, 1, 2, 32, 32, dtype=F32) > 0
    assert ws(256, 1, 16384, 32, 32) > 0
    assert ws(256, 1, 16385, 32, 32) == 0                 # H above KDA_MAX_HEADS
    assert ws((1 << 31) - 1, 1, 1, 32, 32) > 0
    assert ws(1 << 31, 1, 1, 32, 32) == 0                 # token offsets are int32
    # a sequence too short to split needs no segment buffers
    small = ws(64 * 16, 1, 32, 128, 128)
    assert small < 4096
    # a long one does (transition + incoming state per segment)
    big = ws(1 << 20, 1, 8, 128, 128)
    assert big > 8 * 128 * 256 * 4


def test_prefill_validation(L):
    T, N, H, dk, dv = 256, 1, 2, 64, 64
    need = kda.kda_prefill_workspace_size(T, N, H, dk, dv)

    def call(**kw):
        a = dict(q=FAKE, k=FAKE + (1 << 20), v=FAKE + (2 << 20), g=FAKE + (3 << 20),
                 beta=FAKE + (4 << 20), cu=None, N=N, T=T, H=H, dk=dk, dv=dv, chunk=64,
                 init=None, fin=FAKE + (8 << 20), o=FAKE + (16 << 20), dt=BF16,
                 ws=FAKE + (32 << 20), wsb=need)
        a.update(kw)
        return L.kda_prefill(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["N"], a["T"],
                             a["H"], a["dk"], a["dv"], a["chunk"], a["init"], a["fin"], a["o"],
                             a["dt"], a["ws"], a["wsb"], None)

    assert call(N=0) == 1
    assert call(T=-5) == 1
    assert call(N=3) == 1                                   # N > 1 needs cu_seqlens
    assert call(dk=96) == 2
    assert call(chunk=32) == 2
    assert call(dt=F32, dk=128, dv=128) == 2
    assert call(dt=9) == 2
    assert call(H=16385) == 2                               # H above KDA_MAX_HEADS
    assert call(T=1 << 31) == 2                             # token offsets are int32
    assert call(q=None) == 1
    assert call(o=None) == 1
    if need > 0:
        assert call(wsb=need - 1) == 3
        assert call(ws=None) == 3
    assert call(o=FAKE + 8) == 1                             # o aliases q
    assert call(fin=FAKE + (2 << 20)) == 1                   # final state aliases v
    assert call(init=FAKE + (8 << 20) + 4) == 1              # partial init/final overlap
    assert call(ws=FAKE + (16 << 20)) == 1                   # workspace aliases o
    assert call(ws=FAKE + (4 << 20)) == 1                    # workspace aliases beta


def test_verify_commit_validation(L):
    base = dict(q=FAKE, k=FAKE + (1 << 20), v=FAKE + (2 << 20), g=FAKE + (3 << 20),
                beta=FAKE + (4 << 20), state=FAKE + (8 << 20), o=FAKE + (64 << 20), n=FAKE + (96 << 20))

    def verify(**kw):
        a = dict(base, B=4, K=3, H=2, dk=64, dv=64, dt=BF16)
        a.update(kw)
        return L.kda_verify(a["q"], a["k"], a["v"], a["g"], a["beta"], a["state"], a["o"],
                            a["B"], a["K"], a["H"], a["dk"], a["dv"], a["dt"], None)

    def commit(**kw):
        a = dict(base, B=4, K=3, H=2, dk=64, dv=64, dt=BF16)
        a.update(kw)
        return L.kda_commit(a["k"], a["v"], a["g"], a["beta"], a["n"], a["state"],
                            a["B"], a["K"], a["H"], a["dk"], a["dv"], a["dt"], None)

    for call in (verify, commit):
        assert call(B=-1) == 1
        assert call(K=0) == 1
        assert call(H=0) == 1
        assert call(K=65) == 2                                # above KDA_MAX_DRAFT
        assert call(dk=48) == 2
        assert call(dt=7) == 2
        assert call(k=None) == 1
        assert call(state=FAKE + (8 << 20) + 4) == 1          # misaligned state
        assert call(state=FAKE + (3 << 20)) == 1              # state aliases g
        assert call(B=0, k=None, state=None) == 0             # empty batch: no-op
    assert verify(q=None) == 1
    assert verify(o=None) == 1
    assert verify(o=FAKE + 16) == 1                           # o aliases q
    assert verify(o=FAKE + (8 << 20)) == 1                    # o aliases the state
    assert commit(n=None) == 1


def test_checkpoint_count_host(L):
    """kda_checkpoint_count applies the planner's clamping (non-decreasing
    offsets inside [0, T_total]) and counts len // interval per sequence."""
    import numpy as np
    rng = np.random.default_rng(3)
    for _ in range(50):
        N = int(rng.integers(1, 20))
        T = int(rng.integers(0, 5000))
        cu = np.concatenate([[0], rng.integers(-100, T + 200, size=N)]).astype(np.int32)
        interval = int(rng.choice([64, 128, 512]))
        want, prev = 0, 0
        for n in range(N):
            x = min(max(int(cu[n + 1]), 0), T)
            x = max(x, prev)
            want += (x - prev) // interval
            prev = x
        assert kda.kda_checkpoint_count(cu, T, interval) == want
    assert kda.kda_checkpoint_count(None, 8192, 512) == 16
    assert L.kda_checkpoint_count(None, 0, 10, 64) == -1
    assert L.kda_checkpoint_count(None, 1, 10, 0) == -1


def test_prefill_ckpt_validation(L):
    T, N, H, dk, dv = 256, 1, 2, 64, 64
    need = kda.kda_prefill_workspace_size(T, N, H, dk, dv)

    def call(**kw):
        a = dict(q=FAKE, k=FAKE + (1 << 20), v=FAKE + (2 << 20), g=FAKE + (3 << 20),
                 beta=FAKE + (4 << 20), cu=None, N=N, T=T, H=H, dk=dk, dv=dv, chunk=64,
                 init=None, fin=FAKE + (8 << 20), o=FAKE + (16 << 20), dt=BF16,
                 ws=FAKE + (32 << 20), wsb=need, iv=64, ck=FAKE + (64 << 20), cap=4)
        a.update(kw)
        return L.kda_prefill_ckpt(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["N"], a["T"],
                                  a["H"], a["dk"], a["dv"], a["chunk"], a["init"], a["fin"], a["o"],
                                  a["dt"], a["ws"], a["wsb"], a["iv"], a["ck"], a["cap"], None)

    assert call(iv=0) == 1
    assert call(iv=100) == 1                                  # not a multiple of 64
    assert call(cap=-1) == 1
    assert call(ck=None) == 1                                 # capacity without a buffer
    assert call(ck=FAKE + (16 << 20)) == 1                    # overlaps o
    assert call(ck=FAKE + (2 << 20)) == 1                     # overlaps v
    assert call(ck=FAKE + (64 << 20) + 2) == 1                # misaligned
    assert call(dk=96) == 2                                   # prefill checks still apply


def test_prefill_gated_validation(L):
    T, N, H, dk, dv = 256, 1, 2, 64, 64
    need = kda.kda_prefill_workspace_size(T, N, H, dk, dv)

    def call(**kw):
        a = dict(q=FAKE, k=FAKE + (1 << 20), v=FAKE + (2 << 20), z=FAKE + (3 << 20), A=FAKE + (5 << 20),
                 gmin=-5.0, beta=FAKE + (4 << 20), cu=None, N=N, T=T, H=H, dk=dk, dv=dv, chunk=64,
                 init=None, fin=FAKE + (8 << 20), o=FAKE + (16 << 20), dt=BF16,
                 ws=FAKE + (32 << 20), wsb=need, iv=0, ck=None, cap=0)
        a.update(kw)
        return L.kda_prefill_gated(a["q"], a["k"], a["v"], a["z"], a["A"], a["gmin"], a["beta"], a["cu"],
                                   a["N"], a["T"], a["H"], a["dk"], a["dv"], a["chunk"], a["init"], a["fin"],
                                   a["o"], a["dt"], a["ws"], a["wsb"], a["iv"], a["ck"], a["cap"], None)

    assert call(A=None) == 1                                  # A is required when there are tokens
    assert call(gmin=-6.0) == 1                               # below the bound the kernels rely on
    assert call(gmin=0.0) == 1
    assert call(gmin=float("nan")) == 1
    assert call(A=FAKE + (16 << 20) + 64) == 1                # A inside o
    assert call(A=FAKE + (32 << 20) + 64) == 1                # A inside the workspace
    assert call(z=None) == 1
    assert call(iv=-64) == 1
    assert call(iv=100, ck=FAKE + (64 << 20), cap=4) == 1     # checkpoint rules of kda_prefill_ckpt
    assert call(dk=96) == 2                                   # prefill checks still apply
    assert call(wsb=need - 1) == 3
    assert b"kda_prefill_gated" in L.kda_last_error()
    # no tokens and no final state: nothing to do, A may be NULL
    assert call(T=0, A=None, fin=None, q=None, k=None, v=None, z=None, beta=None, o=None) == 0


def test_decode_gated_validation(L):
    B, H, dk, dv = 4, 2, 64, 64

    def call(**kw):
        a = dict(q=FAKE, k=FAKE + (1 << 20), v=FAKE + (2 << 20), z=FAKE + (3 << 20), A=FAKE + (5 << 20),
                 gmin=-5.0, beta=FAKE + (4 << 20), S=FAKE + (8 << 20), o=FAKE + (16 << 20), B=B, H=H,
                 dk=dk, dv=dv, dt=BF16)
        a.update(kw)
        return L.kda_decode_step_gated(a["q"], a["k"], a["v"], a["z"], a["A"], a["gmin"], a["beta"], a["S"],
                                       a["o"], a["B"], a["H"], a["dk"], a["dv"], a["dt"], None)

    assert call(A=None) == 1
    assert call(gmin=0.0) == 1
    assert call(gmin=float("inf")) == 1
    assert call(A=FAKE + (16 << 20)) == 1                     # A inside o
    assert call(A=FAKE + (8 << 20) + 64) == 1                 # A inside the state
    assert call(z=None) == 1
    assert call(dk=96) == 2
    assert call(S=FAKE + (8 << 20) + 4) == 1                  # state not 16-byte aligned
    assert b"kda_decode_step_gated" in L.kda_last_error()
    assert call(B=0, A=None) == 0                             # nothing to do


def test_backward_validation(L):
    T, N, H, dk, dv = 256, 1, 2, 64, 64
    need = L.kda_backward_workspace_size(T, N, H, dk, dv)
    assert need > 0
    assert L.kda_backward_workspace_size(T, N, H, 96, dv) == 0
    assert L.kda_backward_workspace_size(T, 0, H, dk, dv) == 0
    assert L.kda_backward_workspace_size(-1, N, H, dk, dv) == 0

    def call(**kw):
        a = dict(q=FAKE, k=FAKE + (1 << 20), v=FAKE + (2 << 20), g=FAKE + (3 << 20), beta=FAKE + (4 << 20),
                 cu=None, N=N, T=T, H=H, dk=dk, dv=dv, init=None, ck=None, cap=0, do=FAKE + (5 << 20),
                 dfin=None, dq=FAKE + (8 << 20), dkk=FAKE + (9 << 20), dvv=FAKE + (10 << 20),
                 dg=FAKE + (11 << 20), db=FAKE + (12 << 20), dinit=FAKE + (13 << 20), dt=BF16,
                 ws=FAKE + (64 << 20), wsb=need)
        a.update(kw)
        return L.kda_backward(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["N"], a["T"], a["H"],
                              a["dk"], a["dv"], a["init"], a["ck"], a["cap"], a["do"], a["dfin"], a["dq"],
                              a["dkk"], a["dvv"], a["dg"], a["db"], a["dinit"], a["dt"], a["ws"], a["wsb"], None)

    assert call(N=0) == 1
    assert call(N=3) == 1                                   # N > 1 needs cu_seqlens
    assert call(dk=96) == 2
    assert call(dt=7) == 2
    assert call(T=1 << 31) == 2
    assert call(q=None) == 1
    assert call(dq=None) == 1
    assert call(dinit=None) == 1
    assert call(cap=-1) == 1
    assert call(wsb=need - 1) == 3
    assert call(ws=None) == 3
    assert call(dvv=FAKE + (10 << 20) + 4) == 1             # dv not 16-byte aligned
    assert call(dq=FAKE + (1 << 20)) == 1                   # dq overlaps k
    assert call(dg=FAKE + (8 << 20) + 64) == 1              # dg overlaps dq
    assert call(ws=FAKE + (13 << 20)) == 1                  # workspace overlaps d_initial_state
    assert b"kda_backward" in L.kda_last_error()
