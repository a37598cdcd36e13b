"""Python binding of libkda (the KDA forward pass for MI355X / gfx950).

Argument marshalling only: every entry point takes torch tensors that live on
the current HIP device, passes their device pointers and sizes to the C ABI in
include/kda.h, and raises on a non-OK status.  torch is used for device memory
and streams; all arithmetic happens in libkda's kernels.  If libkda.so has not
been built, importing the binding functions raises: there is no fallback.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda.so")
# the same library with device-side bounds checks (kda_debug_check_bits)
CHECKED_LIB_PATH = os.path.join(HERE, "libkda_checked.so")

KDA_F32, KDA_BF16 = 0, 1
_STATUS = {0: "KDA_OK", 1: "KDA_ERR_INVALID_ARGUMENT", 2: "KDA_ERR_UNSUPPORTED",
           3: "KDA_ERR_WORKSPACE_TOO_SMALL", 4: "KDA_ERR_HIP"}
EXPORTED = ("kda_status_string", "kda_last_error", "kda_version", "kda_gate",
            "kda_prefill_workspace_size", "kda_prefill", "kda_decode_step", "kda_verify", "kda_commit",
            "kda_prefill_ckpt", "kda_checkpoint_count", "kda_prefill_gated", "kda_decode_step_gated",
            "kda_backward_workspace_size", "kda_backward", "kda_test_prefill", "kda_test_prefill_workspace_size",
            "kda_test_prefill_flags", "kda_prefill_gated_noalloc", "kda_test_backward",
            "kda_test_backward_workspace_size", "kda_describe_prefill_plan", "kda_describe_backward_plan")

_lib = None


class KDAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libkda (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = load(LIB_PATH)
    return _lib


@contextlib.contextmanager
def using_library(path: str):
    """Route every binding call to the library at `path` (say the checked
    build, CHECKED_LIB_PATH) inside the block."""
    global _lib
    prev = _lib
    _lib = load(path)
    try:
        yield _lib
    finally:
        _lib = prev


def device_check_bits(reset: bool = False) -> int:
    """The checked build's device-side check bits (0: every check held);
    synchronises with the device."""
    L = lib()
    if not hasattr(L, "kda_debug_check_bits"):
        raise RuntimeError("the loaded library is not the checked build")
    bits = ctypes.c_uint(0)
    _check(L.kda_debug_check_bits(ctypes.byref(bits), int(reset)))
    return bits.value


def load(path: str) -> ctypes.CDLL:
    """Load a build of libkda and declare its signatures."""
    if not os.path.exists(path):
        raise ImportError(f"{os.path.basename(path)} not found at {path}; build it with "
                          "`python -m linear_attention_sequence_gate_amd.build`")
    L = ctypes.CDLL(path)
    P, I, I64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    L.kda_status_string.argtypes = [I]
    L.kda_status_string.restype = ctypes.c_char_p
    L.kda_last_error.argtypes = []
    L.kda_last_error.restype = ctypes.c_char_p
    L.kda_version.argtypes = []
    L.kda_version.restype = I
    L.kda_gate.argtypes = [P, P, P, I64, I, I, I, F, P]
    L.kda_gate.restype = I
    L.kda_prefill_workspace_size.argtypes = [I64, I, I, I, I, I, I]
    L.kda_prefill_workspace_size.restype = SZ
    L.kda_prefill.argtypes = [P, P, P, P, P, P, I, I64, I, I, I, I, P, P, P, I, P, SZ, P]
    L.kda_prefill.restype = I
    L.kda_decode_step.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, P]
    L.kda_decode_step.restype = I
    L.kda_verify.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, P]
    L.kda_verify.restype = I
    L.kda_commit.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, P]
    L.kda_commit.restype = I
    L.kda_prefill_ckpt.argtypes = [P, P, P, P, P, P, I, I64, I, I, I, I, P, P, P, I, P, SZ, I, P, I64, P]
    L.kda_prefill_ckpt.restype = I
    L.kda_prefill_gated.argtypes = [P, P, P, P, P, F, P, P, I, I64, I, I, I, I, P, P, P, I, P, SZ, I, P, I64,
                                    P]
    L.kda_prefill_gated.restype = I
    L.kda_decode_step_gated.argtypes = [P, P, P, P, P, F, P, P, P, I, I, I, I, I, P]
    L.kda_decode_step_gated.restype = I
    L.kda_backward_workspace_size.argtypes = [I64, I, I, I, I]
    L.kda_backward_workspace_size.restype = SZ
    L.kda_backward.argtypes = [P, P, P, P, P, P, I, I64, I, I, I, P, P, I64, I, P, P, P, P, P, P, P, P, I, P,
                               SZ, P]
    L.kda_backward.restype = I
    L.kda_test_prefill.argtypes = [P, P, P, P, P, F, P, P, I, I64, I, I, I, P, P, P, I, P, SZ, I, P, I64, I, I,
                                   P]
    L.kda_test_prefill.restype = I
    L.kda_test_prefill_workspace_size.argtypes = [I64, I, I, I, I, I, I, I]
    L.kda_test_prefill_workspace_size.restype = SZ
    L.kda_test_prefill_flags.argtypes = [I64, I, I, I, I, I, I, I, ctypes.POINTER(SZ)]
    L.kda_test_prefill_flags.restype = I64
    L.kda_prefill_gated_noalloc.argtypes = [P, P, P, P, P, F, P, P, I, I64, I, I, I, I, P, P, P, I, I, P, I64,
                                            P]
    L.kda_prefill_gated_noalloc.restype = I
    L.kda_test_backward.argtypes = [P, P, P, P, P, P, I, I64, I, I, I, P, P, I64, I, P, P, P, P, P, P, P, P, I,
                                    P, SZ, I64, I64, P]
    L.kda_test_backward.restype = I
    L.kda_test_backward_workspace_size.argtypes = [I64, I, I, I, I, I64]
    L.kda_test_backward_workspace_size.restype = SZ
    L.kda_checkpoint_count.argtypes = [P, I, I64, I]
    L.kda_checkpoint_count.restype = I64
    L.kda_describe_prefill_plan.argtypes = [I64, I, I, I, I, I, I, ctypes.c_char_p, SZ]
    L.kda_describe_prefill_plan.restype = I64
    L.kda_describe_backward_plan.argtypes = [I64, I, I, I, I, I, ctypes.c_char_p, SZ]
    L.kda_describe_backward_plan.restype = I64
    if hasattr(L, "kda_debug_check_bits"):
        L.kda_debug_check_bits.argtypes = [ctypes.POINTER(ctypes.c_uint), I]
        L.kda_debug_check_bits.restype = I
    return L


def _check(status: int):
    if status != 0:
        raise KDAError(status, lib().kda_last_error().decode())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dense(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("libkda takes dense row-major tensors")


def version() -> int:
    return lib().kda_version()


def kda_gate(z, A, g=None, g_min: float = -5.0, stream=None):
    """g = g_min * sigmoid(exp(A[h]) * z) for z [T, H, d_k]; A fp32 [H]."""
    import torch
    _dense(z, A, g)
    if g is None:
        g = torch.empty_like(z)
    T, H, dk = z.shape
    _check(lib().kda_gate(_ptr(z), _ptr(A), _ptr(g), T, H, dk, _dtype_code(z), float(g_min),
                          _stream(stream)))
    return g


def kda_prefill_workspace_size(T_total: int, N: int, H: int, d_k: int, d_v: int, chunk: int = 64,
                               dtype: int = KDA_BF16) -> int:
    return int(lib().kda_prefill_workspace_size(T_total, N, H, d_k, d_v, chunk, dtype))


def kda_prefill(q, k, v, g, beta, cu_seqlens=None, initial_state=None, final_state=None, o=None,
                workspace=None, chunk: int = 64, want_final_state: bool = True, stream=None):
    """Chunkwise KDA prefill over packed sequences.

    q, k, g: [T, H, d_k]; v: [T, H, d_v]; beta: [T, H]; cu_seqlens: int32 [N+1]
    device tensor or None (one sequence); initial_state: fp32 [N, H, d_k, d_v]
    or None.  Returns (o, final_state)."""
    import torch
    _dense(q, k, v, g, beta, cu_seqlens, initial_state, final_state, o)
    T, H, dk = k.shape
    dv = v.shape[2]
    N = 1 if cu_seqlens is None else cu_seqlens.shape[0] - 1
    code = _dtype_code(k)
    if o is None:
        o = torch.empty((T, H, dv), dtype=v.dtype, device=v.device)
    if final_state is None and want_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=k.device)
    need = kda_prefill_workspace_size(T, N, H, dk, dv, chunk, code)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=k.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().kda_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N, T,
                             H, dk, dv, chunk, _ptr(initial_state), _ptr(final_state), _ptr(o), code,
                             _ptr(workspace), wbytes, _stream(stream)))
    return o, final_state


def kda_decode_step(q, k, v, g, beta, state, o=None, stream=None):
    """One token per sequence; state fp32 [B, H, d_k, d_v] is updated in place. Returns o."""
    import torch
    _dense(q, k, v, g, beta, state, o)
    B, H, dk = k.shape
    dv = v.shape[2]
    if o is None:
        o = torch.empty((B, H, dv), dtype=v.dtype, device=v.device)
    _check(lib().kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(o),
                                 B, H, dk, dv, _dtype_code(k), _stream(stream)))
    return o


def kda_verify(q, k, v, g, beta, state, o=None, stream=None):
    """K draft tokens per sequence from the resident state (not modified).

    q, k, g: [B, K, H, d_k]; v: [B, K, H, d_v]; beta: [B, K, H]; state fp32
    [B, H, d_k, d_v].  Returns o [B, K, H, d_v]."""
    import torch
    _dense(q, k, v, g, beta, state, o)
    B, K, H, dk = k.shape
    dv = v.shape[3]
    if o is None:
        o = torch.empty((B, K, H, dv), dtype=v.dtype, device=v.device)
    _check(lib().kda_verify(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(o),
                            B, K, H, dk, dv, _dtype_code(k), _stream(stream)))
    return o


def kda_commit(k, v, g, beta, n_accept, state, stream=None):
    """Replay the first n_accept[b] (int32 device [B]) cached draft tokens onto
    the state in place."""
    _dense(k, v, g, beta, n_accept, state)
    B, K, H, dk = k.shape
    dv = v.shape[3]
    _check(lib().kda_commit(_ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(n_accept), _ptr(state),
                            B, K, H, dk, dv, _dtype_code(k), _stream(stream)))
    return state


def _describe(fn, *args) -> str:
    n = int(fn(*args, None, 0))
    if n < 0:
        raise KDAError(1, "shape outside the supported set")
    buf = ctypes.create_string_buffer(n + 1)
    fn(*args, buf, n + 1)
    return buf.value.decode()


def describe_prefill_plan(T_total: int, H: int, d_k: int, d_v: int, N: int = 1, packed: bool | None = None,
                          dtype: int = None) -> str:
    """The launch plan kda_prefill would use for these sizes (host only)."""
    dtype = KDA_BF16 if dtype is None else dtype
    packed = N > 1 if packed is None else packed
    return _describe(lib().kda_describe_prefill_plan, T_total, N, H, d_k, d_v, dtype, int(packed))


def describe_backward_plan(T_total: int, H: int, d_k: int, d_v: int, N: int = 1, dtype: int = None) -> str:
    """The launch plan kda_backward would use for these sizes (host only)."""
    dtype = KDA_BF16 if dtype is None else dtype
    return _describe(lib().kda_describe_backward_plan, T_total, N, H, d_k, d_v, dtype)


def kda_checkpoint_count(cu_seqlens_host, T_total: int, interval: int) -> int:
    """Checkpoints kda_prefill_ckpt writes; cu_seqlens_host: int32 numpy [N+1] or None."""
    import numpy as np
    if cu_seqlens_host is None:
        return int(lib().kda_checkpoint_count(None, 1, T_total, interval))
    cu = np.ascontiguousarray(cu_seqlens_host, dtype=np.int32)
    return int(lib().kda_checkpoint_count(cu.ctypes.data, cu.shape[0] - 1, T_total, interval))


def kda_prefill_ckpt(q, k, v, g, beta, interval: int, ckpt=None, cu_seqlens=None, cu_seqlens_host=None,
                     initial_state=None, final_state=None, o=None, workspace=None, chunk: int = 64,
                     stream=None):
    """kda_prefill plus state checkpoints every `interval` tokens of each sequence.
    Returns (o, final_state, ckpt) with ckpt fp32 [n_ckpt, H, d_k, d_v]."""
    import torch
    _dense(q, k, v, g, beta, cu_seqlens, initial_state, final_state, o, ckpt)
    T, H, dk = k.shape
    dv = v.shape[2]
    N = 1 if cu_seqlens is None else cu_seqlens.shape[0] - 1
    code = _dtype_code(k)
    if o is None:
        o = torch.empty((T, H, dv), dtype=v.dtype, device=v.device)
    if final_state is None:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=k.device)
    if ckpt is None:
        if cu_seqlens is not None and cu_seqlens_host is None:
            cu_seqlens_host = cu_seqlens.cpu().numpy()
        n = kda_checkpoint_count(cu_seqlens_host, T, interval)
        ckpt = torch.empty((max(n, 0), H, dk, dv), dtype=torch.float32, device=k.device)
    need = kda_prefill_workspace_size(T, N, H, dk, dv, chunk, code)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=k.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().kda_prefill_ckpt(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N, T,
                                  H, dk, dv, chunk, _ptr(initial_state), _ptr(final_state), _ptr(o), code,
                                  _ptr(workspace), wbytes, int(interval), _ptr(ckpt) if ckpt.numel() else None,
                                  ckpt.shape[0], _stream(stream)))
    return o, final_state, ckpt


def kda_prefill_gated(q, k, v, z, A, beta, g_min: float = -5.0, cu_seqlens=None, initial_state=None,
                      final_state=None, o=None, workspace=None, interval: int = 0, ckpt=None,
                      cu_seqlens_host=None, chunk: int = 64, want_final_state: bool = True, stream=None):
    """kda_prefill with the gate fused: the decay is g = g_min * sigmoid(exp(A[h]) * z),
    computed inside the prefill from z [T, H, d_k] and A fp32 [H].  With interval > 0
    it also writes state checkpoints as kda_prefill_ckpt does.
    Returns (o, final_state) or, with interval > 0, (o, final_state, ckpt)."""
    import torch
    _dense(q, k, v, z, A, beta, cu_seqlens, initial_state, final_state, o, ckpt)
    T, H, dk = k.shape
    dv = v.shape[2]
    N = 1 if cu_seqlens is None else cu_seqlens.shape[0] - 1
    code = _dtype_code(k)
    if o is None:
        o = torch.empty((T, H, dv), dtype=v.dtype, device=v.device)
    if final_state is None and (want_final_state or interval > 0):
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=k.device)
    if interval > 0 and ckpt is None:
        if cu_seqlens is not None and cu_seqlens_host is None:
            cu_seqlens_host = cu_seqlens.cpu().numpy()
        n = kda_checkpoint_count(cu_seqlens_host, T, interval)
        ckpt = torch.empty((max(n, 0), H, dk, dv), dtype=torch.float32, device=k.device)
    need = kda_prefill_workspace_size(T, N, H, dk, dv, chunk, code)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=k.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    cap = 0 if ckpt is None else ckpt.shape[0]
    _check(lib().kda_prefill_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A), float(g_min), _ptr(beta),
                                   _ptr(cu_seqlens), N, T, H, dk, dv, chunk, _ptr(initial_state),
                                   _ptr(final_state), _ptr(o), code, _ptr(workspace), wbytes, int(interval),
                                   _ptr(ckpt) if cap else None, cap, _stream(stream)))
    if interval > 0:
        return o, final_state, ckpt
    return o, final_state


def kda_prefill_gated_noalloc(q, k, v, z, A, beta, o, final_state=None, g_min: float = -5.0, cu_seqlens=None,
                              initial_state=None, interval: int = 0, ckpt=None, chunk: int = 64, stream=None):
    """kda_prefill_gated without a workspace: the library's static scratch is
    used instead (calls on one GPU must not overlap).  The caller passes the
    outputs (o [T, H, d_v], final_state or None, ckpt when interval > 0).
    Returns (o, final_state)."""
    _dense(q, k, v, z, A, beta, o, final_state, cu_seqlens, initial_state, ckpt)
    T, H, dk = k.shape
    dv = v.shape[2]
    N = 1 if cu_seqlens is None else cu_seqlens.shape[0] - 1
    cap = 0 if ckpt is None else ckpt.shape[0]
    _check(lib().kda_prefill_gated_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A), float(g_min), _ptr(beta),
                                           _ptr(cu_seqlens), N, T, H, dk, dv, chunk, _ptr(initial_state),
                                           _ptr(final_state), _ptr(o), _dtype_code(k), int(interval),
                                           _ptr(ckpt) if cap else None, cap, _stream(stream)))
    return o, final_state


def kda_decode_step_gated(q, k, v, z, A, beta, state, o=None, g_min: float = -5.0, stream=None):
    """kda_decode_step with the gate fused: the decay is g = g_min * sigmoid(exp(A[h]) * z),
    computed inside the step from z [B, H, d_k] and A fp32 [H].  Returns o; state is
    updated in place."""
    import torch
    _dense(q, k, v, z, A, beta, state, o)
    B, H, dk = k.shape
    dv = v.shape[2]
    if o is None:
        o = torch.empty((B, H, dv), dtype=v.dtype, device=v.device)
    _check(lib().kda_decode_step_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A), float(g_min), _ptr(beta),
                                       _ptr(state), _ptr(o), B, H, dk, dv, _dtype_code(k), _stream(stream)))
    return o


def kda_backward(q, k, v, g, beta, d_o=None, d_final_state=None, cu_seqlens=None, initial_state=None,
                 ckpt=None, interval: int = 64, workspace=None, stream=None, seg_tokens: int | None = None,
                 warm_tokens: int = -1):
    """Gradients of L = sum_t <d_o[t], o[t]> + <d_final_state, S_T> for kda_prefill on the
    same inputs.  ckpt: the forward's checkpoints every `interval` tokens (64 is
    the fast path; None: every chunk's state is rebuilt from the initial state,
    for short inputs only).  seg_tokens and warm_tokens (tests only) force the
    segment length and the end-of-segment window through kda_test_backward.  Returns a dict of fp32 tensors dq, dk, dg
    [T, H, d_k], dv [T, H, d_v], dbeta [T, H], d_initial_state [N, H, d_k, d_v]."""
    import torch
    _dense(q, k, v, g, beta, d_o, d_final_state, cu_seqlens, initial_state, ckpt, workspace)
    T, H, dk = k.shape
    dv = v.shape[2]
    N = 1 if cu_seqlens is None else cu_seqlens.shape[0] - 1
    dev = k.device
    f = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)
    out = {"dq": f(T, H, dk), "dk": f(T, H, dk), "dv": f(T, H, dv), "dg": f(T, H, dk), "dbeta": f(T, H),
           "d_initial_state": f(N, H, dk, dv)}
    test = seg_tokens is not None or warm_tokens != -1
    if not test:
        need = int(lib().kda_backward_workspace_size(T, N, H, dk, dv))
    else:
        need = int(lib().kda_test_backward_workspace_size(T, N, H, dk, dv, int(seg_tokens or 0)))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = workspace.numel() * workspace.element_size()
    cap = 0 if ckpt is None else ckpt.shape[0]
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N, T, H, dk, dv,
            _ptr(initial_state), _ptr(ckpt) if cap else None, cap, int(interval), _ptr(d_o), _ptr(d_final_state),
            _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]),
            _ptr(out["d_initial_state"]), _dtype_code(k), _ptr(workspace), wbytes]
    if not test:
        _check(lib().kda_backward(*args, _stream(stream)))
    else:
        _check(lib().kda_test_backward(*args, int(seg_tokens or 0), int(warm_tokens), _stream(stream)))
    return out


def kda_test_prefill(q, k, v, g_or_z, beta, A=None, g_min: float = -5.0, cu_seqlens=None, initial_state=None,
                     final_state=None, o=None, workspace=None, interval: int = 0, ckpt=None, cu_seqlens_host=None,
                     seg_chunks: int = 0, warm_tokens: int = -1, stream=None):
    """TEST ONLY: the prefill with the planner's choices made explicit (segment
    length in chunks, 0 = the planner's; warm-up tokens, -1 = the planner's, 0 =
    the exact summary / scan / output passes only).  With A, g_or_z holds the
    gate's input z (as kda_prefill_gated); without, the log-decay g.  Returns
    (o, final_state, ckpt or None, workspace)."""
    import torch
    _dense(q, k, v, g_or_z, A, beta, cu_seqlens, initial_state, final_state, o, ckpt, workspace)
    T, H, dk = k.shape
    dv = v.shape[2]
    N = 1 if cu_seqlens is None else cu_seqlens.shape[0] - 1
    code = _dtype_code(k)
    if o is None:
        o = torch.empty((T, H, dv), dtype=v.dtype, device=v.device)
    if final_state is None:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=k.device)
    if interval > 0 and ckpt is None:
        if cu_seqlens is not None and cu_seqlens_host is None:
            cu_seqlens_host = cu_seqlens.cpu().numpy()
        n = kda_checkpoint_count(cu_seqlens_host, T, interval)
        ckpt = torch.empty((max(n, 0), H, dk, dv), dtype=torch.float32, device=k.device)
    need = int(lib().kda_test_prefill_workspace_size(T, N, H, dk, dv, code, seg_chunks, warm_tokens))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=k.device)
    wbytes = workspace.numel() * workspace.element_size()
    cap = 0 if ckpt is None else ckpt.shape[0]
    _check(lib().kda_test_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(g_or_z), _ptr(A), float(g_min), _ptr(beta),
                                  _ptr(cu_seqlens), N, T, H, dk, dv, _ptr(initial_state), _ptr(final_state),
                                  _ptr(o), code, _ptr(workspace), wbytes, int(interval),
                                  _ptr(ckpt) if cap else None, cap, int(seg_chunks), int(warm_tokens),
                                  _stream(stream)))
    return o, final_state, ckpt, workspace


def test_prefill_flags(workspace, T_total: int, N: int, H: int, d_k: int, d_v: int, dtype: int = KDA_BF16,
                       seg_chunks: int = 0, warm_tokens: int = -1):
    """TEST ONLY: the warm-up flags [nseg_max, H] (int32, 1 = the segment's
    warm-up left M non-zero) that a kda_test_prefill call with these choices left
    in its workspace; rows past the real segment count are unspecified.  None
    when the plan has no warm-up pass."""
    import torch
    off = ctypes.c_size_t(0)
    n = int(lib().kda_test_prefill_flags(T_total, N, H, d_k, d_v, dtype, seg_chunks, warm_tokens,
                                         ctypes.byref(off)))
    if n < 0:
        raise ValueError("bad arguments")
    if n == 0:
        return None
    raw = workspace[off.value:off.value + 4 * n]
    return raw.view(torch.int32).view(n // H, H)
