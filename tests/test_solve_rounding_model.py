"""A CPU model of the prefill block's bf16 rounding points, checked against
the fp64 oracle: which roundings of the UT/WY solve matter.

Per 32-token block of one head (two 16-token sub-tiles), as the bf16 kernel
computes it ("NLP——技术报告解读-Kimi-K3", Model Architecture / Kimi Delta
Attention (KDA): the chunkwise form with the WY solve): decayed q/k operand
tiles in bf16; A = Diag(beta) strict(K.K^T) and P = incl(Q.K^T) from them,
stored in bf16; each 16x16 diagonal inverse (I + A_aa)^{-1} by the Neumann
product (I + Q)(I + Q^2)(I + Q^4)(I + Q^8), Q = -A_aa, with every power an
operand in bf16, the inverse stored in bf16; the block substitution
U_0 = D_0 beta_0 X_0, U_1 = D_1 (beta_1 X_1 - A_10 U_0) with its right-hand
sides as operands; X = V - K.e^G S and O = Q.e^G S + P U with S an operand in
bf16; U an operand in bf16; the state kept in fp32.  Each rounding group can
be switched off.  The model is test infrastructure (it is neither the kernel
nor the oracle); it reproduces the kernel's measured errors on prefill_8k to
three digits.

Readings it pins: the inverse's powers and its storage contribute nothing
measurable; the substitution's right-hand sides do, and carrying them as two
bf16 parts (hi + lo) is as good as an exact substitution."""
import numpy as np
import pytest

import oracle
import synth


def rb(x):
    return synth.bf16_round(np.asarray(x, dtype=np.float32)).astype(np.float64)


def f32(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def split2(x):
    hi = rb(x)
    return hi + rb(f32(x) - hi)


def model(q, k, v, g, beta, S0, flags, sub="bf16", BC=32):
    """q, k, g [T, H, dk]; v [T, H, dv]; beta [T, H]; S0 [H, dk, dv].
    flags: the rounding groups on; sub: the substitution's right-hand sides,
    "bf16", "split" (two bf16 parts) or "exact"."""
    r = {n: (rb if n in flags else f32) for n in ("tiles", "AP", "pow", "D", "U", "S_op", "out")}
    rs = {"bf16": rb, "split": split2, "exact": f32}[sub]
    T, H, dk = k.shape
    S = S0.astype(np.float64).copy()
    o = np.zeros((T, H, v.shape[2]))
    for b0 in range(0, T, BC):
        b1 = min(T, b0 + BC)
        n = b1 - b0
        qb, kb, vb = (np.transpose(x[b0:b1], (1, 0, 2)).astype(np.float64) for x in (q, k, v))
        bb = beta[b0:b1].T.astype(np.float64)
        G = np.cumsum(np.transpose(g[b0:b1], (1, 0, 2)).astype(np.float32), axis=1, dtype=np.float32)
        G = G.astype(np.float64)
        Gl = G[:, n - 1]
        # each row's decay reference: the start of its 16-token sub-tile
        ref = np.where((np.arange(n) >= 16)[None, :, None], G[:, min(15, n - 1)][:, None, :], 0.0)
        KG = r["tiles"](kb * np.exp(G))
        QG = r["tiles"](qb * np.exp(G))
        KH = r["tiles"](kb * np.exp(Gl[:, None] - G))
        Lk = r["tiles"](kb * np.exp(G - ref))
        Lq = r["tiles"](qb * np.exp(G - ref))
        A = np.zeros((H, n, n))
        P = np.zeros((H, n, n))
        for i in range(n):
            Ri = r["tiles"](kb[:, :i + 1] * np.exp(ref[:, i:i + 1] - G[:, :i + 1]))
            A[:, i, :i] = f32(np.einsum("hc,hjc->hj", Lk[:, i], Ri[:, :i]) * bb[:, i:i + 1])
            P[:, i, :i + 1] = f32(np.einsum("hc,hjc->hj", Lq[:, i], Ri))
        A, P = r["AP"](A), r["AP"](P)
        D = []
        for a in range((n + 15) // 16):
            s0, s1 = 16 * a, min(n, 16 * a + 16)
            Q = -A[:, s0:s1, s0:s1]
            I = np.eye(s1 - s0)[None]
            if "pow" in flags:
                f2 = rb(Q @ Q)
                p4 = f2 @ f2
                f4 = rb(p4)
                q8 = f4 @ f4
                e = I + p4 + q8 + f4 @ rb(q8)
                e2 = e + f2 @ rb(e)
                d = e2 + Q @ rb(e2)
            else:
                d = np.linalg.inv(I + A[:, s0:s1, s0:s1])
            D.append(r["D"](d))
        X = vb - KG @ r["S_op"](S)
        bX = bb[:, :, None] * X
        U = np.zeros_like(X)
        U[:, :16] = D[0] @ rs(bX[:, :16])
        if n > 16:
            U[:, 16:] = D[1] @ rs(bX[:, 16:] - A[:, 16:, :16] @ rs(U[:, :16]))
        Ub = r["U"](U)
        o[b0:b1] = np.transpose(r["out"](QG @ r["S_op"](S) + P @ Ub), (1, 0, 2))
        S = f32(np.exp(Gl)[:, :, None] * S + np.transpose(KH, (0, 2, 1)) @ Ub)
    return o, S


ALL = {"tiles", "AP", "pow", "D", "U", "S_op", "out"}


@pytest.fixture(scope="module")
def case():
    """prefill_8k's inputs, heads 0-1, the first 2048 tokens; g in fp32 as the
    fused gate keeps it."""
    wl = synth.PREFILL_8K
    heads, T = [0, 1], 2048
    x = {n: synth.token_rows(wl, n, 0, T)[:, heads] for n in ("q", "k", "v", "z", "beta")}
    g = oracle.gate(x["z"], synth.gate_A(wl)[heads]).astype(np.float32)
    S0 = np.zeros((len(heads), wl.dk, wl.dv))
    o_ref, S_ref = oracle.prefill(x["q"], x["k"], x["v"], g, x["beta"], S0=S0[None])
    return x, g, S0, o_ref, S_ref[0]


def errors(case, flags, sub="bf16"):
    x, g, S0, o_ref, S_ref = case
    o, S = model(x["q"], x["k"], x["v"], g, x["beta"], S0, flags, sub)
    eo = (np.abs(o - o_ref).max(axis=(0, 2)) / np.abs(o_ref).max(axis=(0, 2))).max()
    es = (np.abs(S - S_ref).max(axis=(1, 2)) / np.abs(S_ref).max(axis=(1, 2))).max()
    return eo, es


def test_model_without_rounding_is_the_recurrence(case):
    eo, es = errors(case, set(), "exact")
    assert eo < 1e-5 and es < 1e-5, (eo, es)


def test_inverse_powers_and_storage_do_not_matter(case):
    base = errors(case, ALL)
    for off in ({"pow"}, {"D"}, {"pow", "D"}):
        e = errors(case, ALL - off)
        assert abs(e[0] - base[0]) <= 0.02 * base[0] and abs(e[1] - base[1]) <= 0.02 * base[1], (off, e, base)


def test_split_right_hand_sides_match_an_exact_substitution(case):
    bf = errors(case, ALL, "bf16")
    sp = errors(case, ALL, "split")
    ex = errors(case, ALL, "exact")
    assert abs(sp[0] - ex[0]) <= 0.01 * ex[0] and abs(sp[1] - ex[1]) <= 0.01 * ex[1], (sp, ex)
    assert sp[1] < 0.85 * bf[1], (sp, bf)
    assert bf[0] < 2e-2 and sp[0] < 2e-2
