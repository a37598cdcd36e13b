"""Pins for the fp64 oracle: checks against what the pages and the mathematics
fix, none of which re-types the oracle's own loops.

Each pin takes a loaded oracle library handle so the same battery can run on
deliberately broken copies of the oracle (tests/test_oracle_mutants.py).

  gate_closed_forms      g(0) = g_min/2; g(z) + g(-z) = g_min; saturation at g_min
                         and 0; agreement with scipy's expit; the printed
                         "at most 99.33% forgotten per step" (tests/golden).
  gate_metamorphic       the per-head scale enters only as e^{A_h} z: g(z, A) =
                         g(e^{A} z, 0) with e^{A} from numpy; g(z, ln 2) =
                         g(2z, 0); g(z, -1) = g(z/e, 0); g(+-ln 3, 0) =
                         -5 * (3/4, 1/4) exactly.
  bf16_rounding          nearest-bf16 rounding against a brute-force search.
  brute_force_T_le_4     the recurrence as a Kronecker-vectorised affine map
                         (dense (dk*dv+1)^2 matrices), T <= 4.
  beta_zero_pure_decay   beta = 0: S_T = Diag(exp(sum g)) S_0, a closed form.
  exact_recall           alpha = 1, beta = 1, orthonormal keys: S_T = sum k v^T
                         and querying k_j returns v_j.
  delta_overwrite        alpha = 1, beta = 1, one key written twice: the read-out
                         is the second value whatever S_0 held.
  linearity_kcp          S_T(S_0) = S_T(0) + M S_0 with M the product of the
                         per-token transitions; segment composition.
  chunked_equals_serial  the chunkwise form reproduces the serial one.
  wy_solve_vs_scipy      the per-chunk (I + A)^{-1} Diag(beta) against LAPACK.
  decode_equals_prefill  T decode steps = a T-token prefill.
  varlen_independent     packed sequences = separate runs; empty sequences pass
                         their state through.
  backward_vs_finite_differences
                         every gradient of the reverse-mode oracle (dq, dk, dv,
                         dg, dbeta, dS0) against central differences of the
                         forward recurrence, on two packed sequences.
"""
from __future__ import annotations

import json
import os

import numpy as np
import scipy.linalg
import scipy.special

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _inputs(rng, T, H, dk, dv, gmax=5.0):
    q = _unit(rng.standard_normal((T, H, dk)))
    k = _unit(rng.standard_normal((T, H, dk)))
    v = rng.standard_normal((T, H, dv))
    g = -rng.uniform(0.0, gmax, (T, H, dk))
    beta = rng.uniform(0.05, 0.95, (T, H))
    return q, k, v, g, beta


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(np.max(np.abs(b)), 1e-300)
    err = np.max(np.abs(a - b)) / scale if a.size else 0.0
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    assert err <= tol, f"{what}: normwise-max relative error {err:.3e} > {tol:.1e}"


def gate_closed_forms(lib):
    A = np.array([-1.0, 0.0, 0.7])
    z0 = np.zeros((1, 3, 4))
    g0 = oracle.gate(z0, A, lib=lib)
    assert np.all(g0 == -2.5), f"g(z=0) must be g_min/2 = -2.5 exactly, got {g0.ravel()}"
    rng = np.random.default_rng(5)
    z = rng.uniform(-10, 10, (64, 3, 8))
    g = oracle.gate(z, A, lib=lib)
    gm = oracle.gate(-z, A, lib=lib)
    _close(g + gm, np.full_like(g, -5.0), 1e-15, "g(z) + g(-z) = g_min")
    ref = -5.0 * scipy.special.expit(np.exp(A)[None, :, None] * z)
    _close(g, ref, 1e-14, "gate vs -5*expit(e^A z)")
    assert np.all((g <= 0.0) & (g >= -5.0)), "g must lie in [g_min, 0]"
    zs = np.linspace(-20, 20, 401)[:, None, None] * np.ones((1, 3, 1))
    gs = oracle.gate(zs, A, lib=lib)[:, :, 0]
    assert np.all(np.diff(gs, axis=0) <= 0.0), "g must not increase with z"
    hi = oracle.gate(np.full((1, 3, 1), 1000.0), A, lib=lib)
    lo = oracle.gate(np.full((1, 3, 1), -1000.0), A, lib=lib)
    assert np.all(hi == -5.0), "g saturates at g_min for large z"
    assert np.all((lo <= 0.0) & (lo > -1e-9)), "g tends to 0 for very negative z"
    with open(os.path.join(GOLDEN, "gate_bound.json")) as f:
        gold = json.load(f)
    alpha_min = float(np.min(np.exp(oracle.gate(np.full((1, 3, 1), 1000.0), A, lib=lib))))
    forget = round(100.0 * (1.0 - alpha_min), gold["printed_decimals"])
    assert forget == gold["max_forget_percent_printed"], f"max forgetting {forget}%"


def gate_metamorphic(lib):
    """The head's parameter only rescales the pre-activation: with e^{A_h}
    computed independently (numpy), g(z, A) = g(e^{A} z, 0), so a gate that
    drops the exponential, flips its sign or applies A elsewhere fails."""
    rng = np.random.default_rng(17)
    A = np.array([-1.0, -0.3, 0.0, 0.5, 1.0])
    z = rng.uniform(-4, 4, (50, 5, 6))
    g = oracle.gate(z, A, lib=lib)
    scaled = np.exp(A)[None, :, None] * z
    g0 = oracle.gate(scaled, np.zeros(5), lib=lib)
    _close(g, g0, 1e-14, "g(z, A) = g(e^A z, 0)")
    # exact special scales: A = ln 2 doubles z, A = -1 divides it by e
    g2 = oracle.gate(z[:, :1], np.array([np.log(2.0)]), lib=lib)
    _close(g2, oracle.gate(2.0 * z[:, :1], np.zeros(1), lib=lib), 1e-14, "g(z, ln 2) = g(2z, 0)")
    gm = oracle.gate(z[:, :1], np.array([-1.0]), lib=lib)
    _close(gm, oracle.gate(z[:, :1] / np.e, np.zeros(1), lib=lib), 1e-14, "g(z, -1) = g(z/e, 0)")
    # and A = 0 is the plain sigmoid scaled by g_min, at a few exact points:
    # sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4
    pts = np.array([np.log(3.0), -np.log(3.0)]).reshape(2, 1, 1)
    _close(oracle.gate(pts, np.zeros(1), lib=lib).ravel(), np.array([-3.75, -1.25]), 1e-15,
           "g(+-ln 3, 0) = -5 * (3/4, 1/4)")


def _bf16_brute(x: float) -> float:
    f = np.float32(x)
    bits = int(np.array([f], dtype=np.float32).view(np.uint32)[0]) >> 16
    best, best_err, best_bits = None, None, None
    for b in (bits - 1, bits, bits + 1, bits + 2):
        b &= 0xFFFF
        val = float(np.array([b << 16], dtype=np.uint32).view(np.float32)[0])
        if not np.isfinite(val):
            continue
        e = abs(val - x)
        if best is None or e < best_err or (e == best_err and (b & 1) == 0 and (best_bits & 1) == 1):
            best, best_err, best_bits = val, e, b
    return best


def bf16_rounding(lib):
    rng = np.random.default_rng(11)
    xs = list(rng.uniform(-5, 0, 300)) + list(rng.standard_normal(300) * 1e3)
    # exact midpoints between neighbouring bf16 values (ties) and their neighbours
    for b in (0x3F80, 0x3F81, 0xC0A0, 0xC09F, 0x4000, 0xBF00):
        lo = float(np.array([b << 16], dtype=np.uint32).view(np.float32)[0])
        hi = float(np.array([(b + 1) << 16], dtype=np.uint32).view(np.float32)[0])
        mid = 0.5 * (lo + hi)
        xs += [mid, np.nextafter(mid, lo), np.nextafter(mid, hi)]
    xs = np.array(xs)
    got = oracle.round_bf16(xs, lib=lib)
    want = np.array([_bf16_brute(x) for x in xs])
    assert np.array_equal(got, want), f"bf16 rounding differs at {np.nonzero(got != want)[0][:5]}"


def _kron_run(q, k, v, g, beta, S0):
    """Recurrence as an affine map on vec(S) (column-major) plus a constant 1."""
    T, dk = k.shape
    dv = v.shape[1]
    n = dk * dv
    x = np.concatenate([S0.reshape(-1, order="F"), [1.0]])
    outs = []
    for t in range(T):
        M = (np.eye(dk) - beta[t] * np.outer(k[t], k[t])) @ np.diag(np.exp(g[t]))
        F = np.zeros((n + 1, n + 1))
        F[:n, :n] = np.kron(np.eye(dv), M)
        F[:n, n] = beta[t] * np.outer(k[t], v[t]).reshape(-1, order="F")
        F[n, n] = 1.0
        x = F @ x
        outs.append(np.kron(np.eye(dv), q[t][None, :]) @ x[:n])
    return np.array(outs), x[:n].reshape(dk, dv, order="F")


def brute_force_T_le_4(lib):
    rng = np.random.default_rng(21)
    for T in (1, 2, 3, 4):
        for dk, dv in ((3, 2), (4, 5)):
            q, k, v, g, beta = _inputs(rng, T, 2, dk, dv)
            S0 = rng.standard_normal((1, 2, dk, dv))
            o, S = oracle.prefill(q, k, v, g, beta, S0=S0, lib=lib)
            for h in range(2):
                ro, rS = _kron_run(q[:, h], k[:, h], v[:, h], g[:, h], beta[:, h], S0[0, h])
                _close(o[:, h], ro, 1e-13, f"o, T={T} h={h}")
                _close(S[0, h], rS, 1e-13, f"S, T={T} h={h}")


def beta_zero_pure_decay(lib):
    rng = np.random.default_rng(31)
    T, H, dk, dv = 40, 2, 6, 5
    q, k, v, g, _ = _inputs(rng, T, H, dk, dv, gmax=0.3)
    beta = np.zeros((T, H))
    S0 = rng.standard_normal((1, H, dk, dv))
    o, S = oracle.prefill(q, k, v, g, beta, S0=S0, lib=lib)
    G = np.cumsum(g, axis=0)  # [T, H, dk]
    for h in range(H):
        _close(S[0, h], np.exp(G[-1, h])[:, None] * S0[0, h], 1e-13, "S_T = Diag(e^{sum g}) S_0")
        ro = (np.exp(G[:, h]) * q[:, h]) @ S0[0, h]
        _close(o[:, h], ro, 1e-13, "o_t = S_0^T (e^{G_t} . q_t)")


def exact_recall(lib):
    rng = np.random.default_rng(41)
    dk, dv, T = 8, 5, 6
    Q, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Q[:, :T].T[:, None, :]
    v = rng.standard_normal((T, 1, dv))
    g = np.zeros((T, 1, dk))
    beta = np.ones((T, 1))
    q = np.repeat(k[:1], T, axis=0)  # always query the first key
    o, S = oracle.prefill(q, k, v, g, beta, lib=lib)
    _close(S[0, 0], sum(np.outer(k[i, 0], v[i, 0]) for i in range(T)), 1e-13, "S_T = sum k v^T")
    _close(o[:, 0], np.repeat(v[:1, 0], T, axis=0), 1e-13, "query k_1 returns v_1")
    for j in range(T):
        _close(S[0, 0].T @ k[j, 0], v[j, 0], 1e-13, f"query k_{j} returns v_{j}")


def delta_overwrite(lib):
    rng = np.random.default_rng(51)
    dk, dv = 7, 4
    kk = _unit(rng.standard_normal(dk))
    v1, v2 = rng.standard_normal(dv), rng.standard_normal(dv)
    k = np.stack([kk, kk])[:, None, :]
    q = k.copy()
    v = np.stack([v1, v2])[:, None, :]
    g = np.zeros((2, 1, dk))
    beta = np.ones((2, 1))
    S0 = rng.standard_normal((1, 1, dk, dv))
    o, _ = oracle.prefill(q, k, v, g, beta, S0=S0, lib=lib)
    _close(o[0, 0], v1, 1e-13, "first write is read back")
    _close(o[1, 0], v2, 1e-13, "second write replaces the first")


def linearity_kcp(lib):
    rng = np.random.default_rng(61)
    T, H, dk, dv = 37, 2, 6, 4
    q, k, v, g, beta = _inputs(rng, T, H, dk, dv, gmax=0.5)
    S0 = rng.standard_normal((1, H, dk, dv))
    _, S_full = oracle.prefill(q, k, v, g, beta, S0=S0, lib=lib)
    _, S_zero = oracle.prefill(q, k, v, g, beta, lib=lib)
    I = np.broadcast_to(np.eye(dk), (1, H, dk, dk)).copy()
    _, Mo = oracle.prefill(q, k, np.zeros((T, H, dk)), g, beta, S0=I, lib=lib)
    for h in range(H):
        M = np.eye(dk)
        for t in range(T):
            M = (np.eye(dk) - beta[t, h] * np.outer(k[t, h], k[t, h])) @ np.diag(np.exp(g[t, h])) @ M
        _close(Mo[0, h], M, 1e-13, "transition from a v=0, S_0=I run")
        _close(S_full[0, h], S_zero[0, h] + M @ S0[0, h], 1e-13, "S_T(S_0) = S_T(0) + M S_0")
    # two segments composed: S = S~_2 + M_2 S_{t1}
    t1 = 15
    _, S_a = oracle.prefill(q[:t1], k[:t1], v[:t1], g[:t1], beta[:t1], S0=S0, lib=lib)
    _, St_b = oracle.prefill(q[t1:], k[t1:], v[t1:], g[t1:], beta[t1:], lib=lib)
    _, M_b = oracle.prefill(q[t1:], k[t1:], np.zeros((T - t1, H, dk)), g[t1:], beta[t1:], S0=I, lib=lib)
    for h in range(H):
        _close(S_full[0, h], St_b[0, h] + M_b[0, h] @ S_a[0, h], 1e-13, "segment composition")


def chunked_equals_serial(lib):
    rng = np.random.default_rng(71)
    lens = [0, 1, 63, 64, 65, 130, 7]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H, dk, dv = int(cu[-1]), 2, 8, 6
    for gmax in (5.0, 0.05):
        q, k, v, g, beta = _inputs(rng, T, H, dk, dv, gmax=gmax)
        S0 = rng.standard_normal((len(lens), H, dk, dv))
        o_s, S_s = oracle.prefill(q, k, v, g, beta, cu=cu, S0=S0, lib=lib)
        for C in (1, 3, 16, 64):
            o_c, S_c = oracle.prefill(q, k, v, g, beta, cu=cu, S0=S0, chunk=C, lib=lib)
            _close(o_c, o_s, 1e-12, f"chunked o, C={C}")
            _close(S_c, S_s, 1e-12, f"chunked S, C={C}")


def wy_solve_vs_scipy(lib):
    rng = np.random.default_rng(81)
    for L in (1, 5, 16, 64):
        dk = 12
        k = _unit(rng.standard_normal((L, dk)))
        g = -rng.uniform(0.0, 1.0, (L, dk))
        beta = rng.uniform(0.05, 0.95, L)
        G = np.cumsum(g, axis=0)
        A = np.zeros((L, L))
        for r in range(L):
            for i in range(r):
                A[r, i] = beta[r] * np.sum(k[r] * k[i] * np.exp(G[r] - G[i]))
        want = scipy.linalg.solve_triangular(np.eye(L) + A, np.diag(beta), lower=True)
        _close(oracle.wy_T(k, g, beta, lib=lib), want, 1e-13, f"(I+A)^-1 Diag(beta), L={L}")


def decode_equals_prefill(lib):
    rng = np.random.default_rng(91)
    T, B, H, dk, dv = 9, 3, 2, 5, 6
    q, k, v, g, beta = _inputs(rng, T * B, H, dk, dv)
    sh = lambda x: x.reshape((B, T) + x.shape[1:])
    q, k, v, g, beta = map(sh, (q, k, v, g, beta))
    S0 = rng.standard_normal((B, H, dk, dv))
    cu = np.arange(B + 1) * T
    flat = lambda x: x.reshape((B * T,) + x.shape[2:])
    o_p, S_p = oracle.prefill(flat(q), flat(k), flat(v), flat(g), flat(beta), cu=cu, S0=S0, lib=lib)
    S = S0.copy()
    outs = []
    for t in range(T):
        o, S = oracle.decode_step(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], S, lib=lib)
        outs.append(o)
    o_d = np.stack(outs, axis=1).reshape(B * T, H, dv)
    _close(o_d, o_p, 1e-13, "decode outputs = prefill outputs")
    _close(S, S_p, 1e-13, "decode state = prefill final state")


def varlen_independent(lib):
    rng = np.random.default_rng(101)
    lens = [5, 0, 17, 1, 30]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H, dk, dv = int(cu[-1]), 3, 4, 3
    q, k, v, g, beta = _inputs(rng, T, H, dk, dv, gmax=0.3)
    S0 = rng.standard_normal((len(lens), H, dk, dv))
    o, S = oracle.prefill(q, k, v, g, beta, cu=cu, S0=S0, lib=lib)
    for n, L in enumerate(lens):
        a, b = cu[n], cu[n + 1]
        if L == 0:
            assert np.array_equal(S[n], S0[n]), "an empty sequence passes its state through"
            continue
        o1, S1 = oracle.prefill(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], S0=S0[n:n + 1], lib=lib)
        _close(o[a:b], o1, 1e-14, f"varlen o, seq {n}")
        _close(S[n], S1[0], 1e-14, f"varlen S, seq {n}")


def backward_vs_finite_differences(lib):
    """L = sum_t <dO_t, o_t> + <dS_fin, S_T>: each input perturbed by +-h in
    the forward oracle, (L(x + h) - L(x - h)) / 2h, against the backward."""
    rng = np.random.default_rng(111)
    lens = [3, 0, 4]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H, dk, dv = int(cu[-1]), 2, 3, 4
    q, k, v, g, beta = _inputs(rng, T, H, dk, dv, gmax=1.5)
    S0 = rng.standard_normal((len(lens), H, dk, dv))
    dO = rng.standard_normal((T, H, dv))
    dS = rng.standard_normal((len(lens), H, dk, dv))
    x = {"q": q, "k": k, "v": v, "g": g, "beta": beta, "S0": S0}

    def loss(x):
        o, S = oracle.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], cu=cu, S0=x["S0"], lib=lib)
        return float(np.sum(o * dO) + np.sum(S * dS))

    grads = oracle.backward(q, k, v, g, beta, dO=dO, dS_fin=dS, cu=cu, S0=S0, lib=lib)
    names = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "S0": "dS0"}
    h = 1e-6
    for name, gname in names.items():
        num = np.zeros_like(x[name])
        for idx in np.ndindex(x[name].shape):
            xp = {n: a.copy() for n, a in x.items()}
            xm = {n: a.copy() for n, a in x.items()}
            xp[name][idx] += h
            xm[name][idx] -= h
            num[idx] = (loss(xp) - loss(xm)) / (2 * h)
        _close(grads[gname], num, 1e-7, f"backward {gname} vs finite differences")


ALL_PINS = [gate_closed_forms, gate_metamorphic, bf16_rounding, brute_force_T_le_4, beta_zero_pure_decay,
            exact_recall, delta_overwrite, linearity_kcp, chunked_equals_serial,
            wy_solve_vs_scipy, decode_equals_prefill, varlen_independent, backward_vs_finite_differences]
