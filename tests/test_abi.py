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


CHECKED_ONLY = {"kda_debug_check_bits"}  # exported by the checked build alone


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(kda.EXPORTED) | CHECKED_ONLY, names
    checked = kda.LIB_PATH == kda.CHECKED_LIB_PATH  # the suite run with --kda-checked
    for n in names:
        assert hasattr(L, n) == (checked or n not in CHECKED_ONLY), f"{kda.LIB_PATH} and {n}"


def test_checked_build_exports(L):
    """The checked build (device-side bounds checks) exports every declared
    symbol, its check-bit reader included, and validates like the release
    build on the host."""
    C = kda.load(kda.CHECKED_LIB_PATH)
    for n in declared_functions():
        assert hasattr(C, n), f"libkda_checked does not export {n}"
    assert C.kda_debug_check_bits(None, 0) == 1  # null pointer, refused before any device call
    assert C.kda_gate(FAKE, FAKE + (1 << 20), FAKE + (2 << 20), 4, 2, 32, BF16, -6.0, None) == 1


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
    # g >= -5 is what the prefill and the backward need (their per-sub-tile
    # decay factors stay inside the fp32 range): a lower bound below it is refused
    assert L.kda_gate(FAKE, FAKE, FAKE, 4, 2, 32, BF16, -5.5, None) == 1
    assert b"[-5, 0)" in L.kda_last_error()
    assert L.kda_gate(None, FAKE, FAKE, 4, 2, 32, BF16, -5.0, None) == 1
    assert b"null" in L.kda_last_error()
    # partial overlap of g with z (exact aliasing is allowed); A far away
    assert L.kda_gate(FAKE, FAKE + (1 << 20), FAKE + 64, 4, 2, 32, BF16, -5.0, None) == 1
    assert b"partially overlaps" in L.kda_last_error()
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


def test_prefill_plan_is_explicit(L, monkeypatch):
    """The planner reads nothing from the environment: the workspace size
    depends only on the arguments, and forced choices go through the test entry
    point.  Its warm-up flags (int32 per segment and head) sit in the workspace
    only when the plan has a warm-up pass."""
    ws = kda.kda_prefill_workspace_size
    tws = L.kda_test_prefill_workspace_size
    base = ws(8192, 1, 32, 128, 128)
    for var in ("KDA_SEG_CHUNKS", "KDA_BWD_SEG_TOKENS", "KDA_LOG"):
        monkeypatch.setenv(var, "3")
    assert ws(8192, 1, 32, 128, 128) == base
    assert tws(8192, 1, 32, 128, 128, BF16, 0, -1) == base
    assert tws(8192, 1, 32, 128, 128, BF16, 3, -1) > base      # more segments, more summaries
    assert tws(8192, 1, 32, 128, 128, BF16, 0, 0) > 0          # exact passes only
    assert tws(8192, 1, 32, 128, 128, BF16, -1, -1) == 0       # bad segment length
    assert tws(8192, 1, 32, 128, 128, BF16, 0, 48) == 0        # warm-up not a multiple of 32
    off = ctypes.c_size_t(0)
    n = L.kda_test_prefill_flags(8192, 1, 32, 128, 128, BF16, 0, -1, ctypes.byref(off))
    assert n >= 8 * 32 and off.value % 256 == 0 and off.value + 4 * n <= base
    assert L.kda_test_prefill_flags(8192, 1, 32, 128, 128, BF16, 0, 0, ctypes.byref(off)) == 0
    # no warm-up kernel for d_k > d_v: the exact passes are the plan
    assert L.kda_test_prefill_flags(8192, 1, 32, 128, 64, BF16, 0, -1, ctypes.byref(off)) == 0
    # the test entry point validates its own arguments before the prefill's
    assert L.kda_test_prefill(FAKE, FAKE, FAKE, FAKE, None, -5.0, FAKE, None, 1, 256, 2, 64, 64, None, None,
                              FAKE, BF16, FAKE, 1 << 20, 0, None, 0, 0, 40, None) == 1
    assert L.kda_test_prefill(FAKE, FAKE, FAKE, FAKE, FAKE + (64 << 20), -6.0, FAKE, None, 1, 256, 2, 64, 64,
                              None, None, FAKE, BF16, FAKE, 1 << 20, 0, None, 0, 0, -1, None) == 1


def test_prefill_workspace_size(L):
    ws = kda.kda_prefill_workspace_size
    assert ws(8192, 1, 32, 128, 128) > 0
    assert ws(0, 1, 32, 128, 128) > 0
    assert ws(8192, 1, 32, 96, 128) == 0
    assert ws(8192, 1, 32, 128, 128, chunk=32) == 0
    # fp32 shapes without a chunk kernel run token by token: the table, a flag
    # per (segment, head) and room for a copy of the initial states
    assert 32 * 128 * 128 * 4 < ws(8192, 1, 32, 128, 128, dtype=F32) <= 32 * 128 * 128 * 4 + 256 + 256 * 4 + 512
    assert 32 * 64 * 64 * 4 < ws(8192, 1, 32, 64, 64, dtype=F32) <= 32 * 64 * 64 * 4 + 256 + 256 * 4 + 512
    assert 3 * 32 * 32 * 128 * 4 < ws(1 << 20, 3, 32, 32, 128, dtype=F32) < 3 * 32 * 32 * 128 * 4 + (1 << 20)
    assert ws(256, 1, 2, 32, 32, dtype=F32) > 0
    assert ws(256, 1, 16384, 32, 32) > 0
    assert ws(256, 1, 16385, 32, 32) == 0                 # H above KDA_MAX_HEADS
    assert ws((1 << 31) - 1, 1, 1, 32, 32) > 0
    assert ws(1 << 31, 1, 1, 32, 32) == 0                 # token offsets are int32
    # a sequence too short to split (at most the shortest segment the planner
    # makes, 4 chunks) needs no segment buffers
    small = ws(64 * 4, 1, 32, 128, 128)
    assert small < 4096
    assert ws(64 * 16, 1, 32, 128, 128) > small  # 16 chunks at H=32: four segments
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
    assert call(dt=F32, dk=96, dv=128) == 2
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
                 cu=None, N=N, T=T, H=H, dk=dk, dv=dv, init=None, ck=None, cap=0, iv=64, do=FAKE + (5 << 20),
                 dfin=None, dq=FAKE + (8 << 20), dkk=FAKE + (9 << 20), dvv=FAKE + (10 << 20),
                 dg=FAKE + (11 << 20), db=FAKE + (12 << 20), dinit=FAKE + (13 << 20), dt=BF16,
                 ws=FAKE + (64 << 20), wsb=need)
        a.update(kw)
        return L.kda_backward(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["N"], a["T"], a["H"],
                              a["dk"], a["dv"], a["init"], a["ck"], a["cap"], a["iv"], a["do"], a["dfin"], a["dq"],
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
    # checkpoints come with a positive interval that is a multiple of 64
    ck = dict(ck=FAKE + (32 << 20), cap=4)
    assert call(iv=0, **ck) == 1
    assert call(iv=96, **ck) == 1
    assert b"interval" in L.kda_last_error()
    # without checkpoints every chunk rebuilds its state from the sequence
    # start (quadratic), so long inputs are refused; the interval is then ignored
    T2 = 4097
    big = L.kda_backward_workspace_size(T2, N, H, dk, dv)
    far = dict(T=T2, wsb=big, q=FAKE, k=FAKE + (4 << 20), v=FAKE + (8 << 20), g=FAKE + (12 << 20),
               beta=FAKE + (16 << 20), do=FAKE + (20 << 20), dq=FAKE + (32 << 20), dkk=FAKE + (40 << 20),
               dvv=FAKE + (48 << 20), dg=FAKE + (56 << 20), db=FAKE + (64 << 20), dinit=FAKE + (68 << 20),
               ws=FAKE + (72 << 20))
    assert call(iv=0, **far) == 2
    assert b"without checkpoints" in L.kda_last_error()
    # the test entry point validates its segment length first
    assert L.kda_test_backward(FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 256, 2, 64, 64, None, None, 0, 64, None, None,
                               FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, BF16, FAKE, 1 << 30, -1, -1, None) == 1
    assert L.kda_test_backward(FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 256, 2, 64, 64, None, None, 0, 64, None, None,
                               FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, BF16, FAKE, 1 << 30, 0, 40, None) == 1
    # 128 heads: the planner gives the sequence one segment; forced 64-token
    # segments need a summary and an incoming gradient each
    assert L.kda_test_backward_workspace_size(4096, 1, 128, 64, 64, 64) > L.kda_test_backward_workspace_size(
        4096, 1, 128, 64, 64, 0) > 0


def test_noalloc_limits(L):
    """kda_prefill_gated_noalloc checks its workspace against the static
    scratch on the host, before touching the device: a packed batch whose
    segment buffers exceed it is refused with a message naming both sizes;
    the 8K workload fits."""
    assert kda.kda_prefill_workspace_size(8192, 1, 32, 128, 128) <= (64 << 20)
    big = kda.kda_prefill_workspace_size(1 << 20, 64, 32, 128, 128)
    assert big > (64 << 20)
    st = L.kda_prefill_gated_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, -5.0, FAKE, FAKE, 64, 1 << 20, 32, 128, 128, 64,
                                     None, None, FAKE, BF16, 0, None, 0, None)
    assert st == 2
    msg = L.kda_last_error().decode()
    assert "static scratch" in msg and str(big) in msg
    # unsupported shapes are refused as by kda_prefill_gated
    assert L.kda_prefill_gated_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, -5.0, FAKE, None, 1, 256, 2, 96, 64, 64,
                                       None, None, FAKE, BF16, 0, None, 0, None) == 2


def test_roofs_library_exports_and_validation():
    """libkda_roofs (the benchmark's measurement kernels) loads, exports what
    include/kda_roofs.h declares, and rejects bad arguments with 1 before it
    launches anything."""
    from linear_attention_sequence_gate_amd import build as kbuild
    header = os.path.join(os.path.dirname(HEADER), "kda_roofs.h")
    text = re.sub(r"/\*.*?\*/", "", open(header).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(kda_\w+)\s*\(", text)))
    assert names == ["kda_roof_mfma", "kda_roof_state_inplace", "kda_roof_stream"]
    R = ctypes.CDLL(kbuild.ROOFS_LIB)
    for n in names:
        assert hasattr(R, n)
    P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    R.kda_roof_stream.argtypes = [I, P, P, I64, P, I64, I, I, P, ctypes.POINTER(ctypes.c_float)]
    R.kda_roof_stream.restype = I
    R.kda_roof_mfma.argtypes = [I, I, P, P, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double)]
    R.kda_roof_mfma.restype = I
    ms, fl = ctypes.c_float(0.0), ctypes.c_double(0.0)
    msp = ctypes.byref(ms)
    bad = [
        (4, FAKE, FAKE, 1 << 20, FAKE, 1 << 20, 16, 1),    # unknown mode
        (-1, FAKE, FAKE, 1 << 20, FAKE, 1 << 20, 16, 1),
        (2, FAKE, FAKE, 0, None, 0, 16, 1),                # no bytes
        (2, FAKE, FAKE, 100, None, 0, 16, 1),              # not a multiple of 16
        (2, FAKE, FAKE, 1 << 20, None, 0, -1, 1),          # negative width
        (2, FAKE, FAKE, 1 << 20, None, 0, 16, 0),          # no repetitions
        (0, FAKE, None, 1 << 20, FAKE, 1 << 20, 0, 1),     # read needs a grid-stride width
        (0, FAKE, None, 1 << 20, None, 0, 16, 1),          # read needs a sink
        (0, FAKE, None, 1 << 20, FAKE, 16 * 256 - 1, 16, 1),  # sink too small
        (0, None, None, 1 << 20, FAKE, 1 << 20, 16, 1),    # read needs src
        (2, None, FAKE, 1 << 20, None, 0, 0, 1),           # copy needs src
        (1, None, None, 1 << 20, None, 0, 0, 1),           # write needs dst
        (3, FAKE, None, 1 << 20, None, 0, 0, 1),           # in place needs dst
    ]
    for mode, src, dst, nbytes, sink, words, wgs, reps in bad:
        assert R.kda_roof_stream(mode, src, dst, nbytes, sink, words, wgs, reps, None, msp) == 1, (mode, nbytes, wgs)
    assert R.kda_roof_stream(2, FAKE, FAKE, 1 << 20, None, 0, 16, 1, None, None) == 1  # no result pointer
    assert R.kda_roof_mfma(0, 16, FAKE, None, msp, ctypes.byref(fl)) == 1
    assert R.kda_roof_mfma(16, 0, FAKE, None, msp, ctypes.byref(fl)) == 1
    assert R.kda_roof_mfma(16, 16, None, None, msp, ctypes.byref(fl)) == 1
    R.kda_roof_state_inplace.argtypes = [P, I64, I, I, P, ctypes.POINTER(ctypes.c_float)]
    R.kda_roof_state_inplace.restype = I
    for buf, nbytes, delay, reps, res in ((None, 1 << 20, 0, 1, msp), (FAKE, 0, 0, 1, msp),
                                          (FAKE, (1 << 20) + 16, 0, 1, msp), (FAKE, 1 << 20, -1, 1, msp),
                                          (FAKE, 1 << 20, 4097, 1, msp), (FAKE, 1 << 20, 0, 0, msp),
                                          (FAKE, 1 << 20, 0, 1, None)):
        assert R.kda_roof_state_inplace(buf, nbytes, delay, reps, None, res) == 1, (nbytes, delay, reps)


def test_single_sequence_workspace_fits_the_noalloc_scratch():
    """One sequence at d_k = d_v = 128 needs about 50 MB of workspace at most,
    whatever its length and head count (the planner cuts it into about
    256 / H segments), so it always fits the 64 MiB static scratch of
    kda_prefill_gated_noalloc; packed sequences can need more."""
    for H in (1, 2, 4, 8, 16, 32, 64, 128, 256, 512):
        for T in (1, 255, 4096, 8192, 1 << 20, 1 << 30, (1 << 31) - 1):
            need = kda.kda_prefill_workspace_size(T, 1, H, 128, 128)
            assert 0 < need <= 50_500_000, (H, T, need)
    assert kda.kda_prefill_workspace_size(1 << 30, 64, 64, 128, 128) > (64 << 20)


def test_plan_descriptions(L):
    """The plan descriptions are host-only text: the planner's numbers and one
    line per launch, truncated like snprintf, -1 for rejected shapes."""
    txt = kda.describe_prefill_plan(8192, 32, 128, 128)
    assert "T_total=8192 N=1 H=32 d_k=128 d_v=128 dtype=bf16" in txt
    assert "warm-up window: 128 tokens" in txt
    assert f"workspace: {kda.lib().kda_prefill_workspace_size(8192, 1, 32, 128, 128, 64, BF16)} bytes" in txt
    lines = [l for l in txt.splitlines() if l.startswith("launch ")]
    assert lines[0].startswith("launch 1: prefill_warm_kernel grid ")
    assert [l.split(":")[1].split(" grid")[0].strip() for l in lines] == [
        "prefill_warm_kernel", "prefill_block_kernel (summary)", "scan_kernel", "prefill_block_kernel (output)"]
    # one sequence: the segment count is exact (8 of 1024 tokens), so the
    # segment launches carry no workgroups that only return
    assert "at most 8 segments, 7 of them non-final" in txt
    assert "prefill_warm_kernel grid 256 x " in txt and "prefill_block_kernel (summary) grid 224 x " in txt
    assert "bwd_chunk_summary_kernel (window) grid 256 x " in kda.describe_backward_plan(8192, 32, 128, 128)
    # packed sequences: the plan kernel first; no warm-up for d_k > d_v
    txt = kda.describe_prefill_plan(10000, 4, 128, 32, N=3)
    assert "launch 1: plan_kernel grid 1 x 256" in txt and "prefill_warm_kernel" not in txt
    assert "warm-up window: 0 tokens" in txt
    # the backward
    txt = kda.describe_backward_plan(8192, 32, 128, 128)
    assert f"workspace: {kda.lib().kda_backward_workspace_size(8192, 1, 32, 128, 128)} bytes" in txt
    assert "window 128 tokens" in txt and "bwd_chunk_full_kernel grid 256 x 512" in txt
    # snprintf semantics and rejections
    full = L.kda_describe_prefill_plan(8192, 1, 32, 128, 128, BF16, 0, None, 0)
    buf = ctypes.create_string_buffer(16)
    assert L.kda_describe_prefill_plan(8192, 1, 32, 128, 128, BF16, 0, buf, 16) == full
    assert len(buf.value) == 15
    assert L.kda_describe_prefill_plan(8192, 1, 32, 128, 128, BF16, 0, None, 16) == -1
    assert L.kda_describe_prefill_plan(8192, 2, 32, 128, 128, BF16, 0, None, 0) == -1  # N > 1 needs cu_seqlens
    assert L.kda_describe_prefill_plan(8192, 1, 32, 96, 128, BF16, 0, None, 0) == -1
    # the token-serial fp32 path: its one launch (two when packed)
    n32 = L.kda_describe_prefill_plan(8192, 1, 32, 128, 128, F32, 0, None, 0)
    buf = ctypes.create_string_buffer(n32 + 1)
    assert L.kda_describe_prefill_plan(8192, 1, 32, 128, 128, F32, 0, buf, n32 + 1) == n32
    txt = buf.value.decode()
    assert "token-serial" in txt and "plan_kernel" not in txt
    # eight segments of 1024 tokens per head: 256 windowed workgroups of 8 waves, then the flagged chains
    assert "segments: 16 chunks" in txt and "prefill_serial_kernel (windowed) grid 256 x 512" in txt
    assert "prefill_serial_kernel (chains) grid 32 x 256" in txt
    n32p = L.kda_describe_prefill_plan(8192, 4, 8, 64, 32, F32, 1, None, 0)
    buf = ctypes.create_string_buffer(n32p + 1)
    L.kda_describe_prefill_plan(8192, 4, 8, 64, 32, F32, 1, buf, n32p + 1)
    txt = buf.value.decode()
    assert "plan_kernel" in txt and "x 192 threads" in txt and "(chains) grid 32 x 64" in txt
    assert L.kda_describe_backward_plan(-1, 1, 32, 128, 128, BF16, None, 0) == -1
    assert L.kda_describe_backward_plan(64, 1, 32, 128, 128, 7, None, 0) == -1
