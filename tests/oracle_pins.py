"""Pins that tie the CPU oracle to facts fixed by the pages and by mathematics.

Each pin takes the oracle library handle (so the mutation tests can run the
same pins against deliberately broken builds of the oracle) and raises
AssertionError when the oracle disagrees.  None of them re-types the oracle's
own formula: they use printed values, closed forms, invariants, special cases
and a brute-force form with explicit transition matrices.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden():
    """The tutorial's worked two-cell example and its printed results (tests/golden/)."""
    with open(os.path.join(GOLDEN, "worked_example.json")) as fh:
        return json.load(fh)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand_inputs(rng, B, T, H, dk, dv, la_range=(-0.1, -0.001)):
    q = _unit(rng.standard_normal((B, T, H, dk)))
    k = _unit(rng.standard_normal((B, T, H, dk)))
    v = rng.standard_normal((B, T, H, dv))
    la = rng.uniform(*la_range, size=(B, T, H))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    return q, k, v, la, b


def _one_step(lib, S0, k, v, alpha, beta, q=None):
    dv, dk = np.asarray(S0).shape
    q = np.zeros(dk) if q is None else np.asarray(q, dtype=np.float64)
    la = -np.inf if alpha == 0.0 else math.log(alpha)
    o, fin = oracle.recurrent(q.reshape(1, 1, 1, dk), np.reshape(k, (1, 1, 1, dk)),
                              np.reshape(v, (1, 1, 1, dv)), np.full((1, 1, 1), la),
                              np.full((1, 1, 1), beta),
                              init_state=np.reshape(S0, (1, 1, dv, dk)), lib=lib)
    return fin[0, 0], o[0, 0, 0]


# -- printed values -----------------------------------------------------------

def pin_worked_example(lib):
    """Tutorial, two-cell hand computation: [[2,10]] -> [[2.25, 5.0]] for
    alpha=0.5, beta=0.25 and [[6, 10]] for alpha=beta=1; the result of measuring
    the error on the undecayed state ([[2, 5]]) must not come out."""
    gold = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    for case in gold["cases"]:
        S, _ = _one_step(lib, np.array(case["state"]), np.array(case["key"]),
                         np.array(case["value"]), case["alpha"], case["beta"])
        assert np.allclose(S, case["expected"], rtol=0, atol=1e-14), (S, case)
        if "wrong_if_undecayed_error" in case:
            assert not np.allclose(S, case["wrong_if_undecayed_error"], atol=1e-3)


def pin_delta_vs_additive(lib):
    """Tutorial, associative-memory section: 1-D memory, write 2 then 6 with
    alpha = beta = 1: the delta rule reads back 6 (the additive rule would read 8)."""
    gold = json.load(open(os.path.join(GOLDEN, "worked_example.json")))["additive_vs_delta"]
    w = gold["writes"]
    T = len(w)
    k = np.ones((1, T, 1, 1))
    v = np.array(w, dtype=np.float64).reshape(1, T, 1, 1)
    o, fin = oracle.recurrent(k, k, v, np.zeros((1, T, 1)), np.ones((1, T, 1)), lib=lib)
    assert abs(o[0, -1, 0, 0] - gold["delta_read_beta_one"]) < 1e-14, o
    assert abs(fin[0, 0, 0, 0] - gold["delta_read_beta_one"]) < 1e-14
    assert abs(o[0, -1, 0, 0] - gold["additive_read"]) > 1.0


# -- closed forms and invariants ------------------------------------------------

def pin_interpolation(lib):
    """With a unit key, S_t k_t = (1 - beta) alpha S_{t-1} k_t + beta v_t
    (tutorial, delta-rule read-back; the gated form reads the decayed state)."""
    rng = np.random.default_rng(11)
    for dv, dk in [(5, 7), (16, 16), (3, 32)]:
        S0 = rng.standard_normal((dv, dk))
        k = _unit(rng.standard_normal(dk))
        v = rng.standard_normal(dv)
        a, b = 0.83, 0.37
        S, _ = _one_step(lib, S0, k, v, a, b)
        want = (1 - b) * a * (S0 @ k) + b * v
        assert np.abs(S @ k - want).max() < 1e-13


def pin_orthogonal_untouched(lib):
    """Directions orthogonal to k_t are only decayed: S_t x = alpha S_{t-1} x
    for x perpendicular to k_t (blog, Householder-transition remark)."""
    rng = np.random.default_rng(12)
    dv, dk = 6, 9
    S0 = rng.standard_normal((dv, dk))
    k = _unit(rng.standard_normal(dk))
    v = rng.standard_normal(dv)
    a, b = 0.61, 0.9
    S, _ = _one_step(lib, S0, k, v, a, b)
    for _ in range(4):
        x = rng.standard_normal(dk)
        x -= (x @ k) * k
        assert np.abs(S @ x - a * (S0 @ x)).max() < 1e-13


def pin_beta_zero_pure_decay(lib):
    """beta = 0: S_t = gamma_t S_0 and o_t = gamma_t S_0 q_t, gamma_t = prod alpha."""
    rng = np.random.default_rng(13)
    q, k, v, la, _ = _rand_inputs(rng, 1, 40, 2, 8, 5)
    S0 = rng.standard_normal((1, 2, 5, 8))
    o, fin = oracle.recurrent(q, k, v, la, np.zeros_like(la), init_state=S0, lib=lib)
    gam = np.exp(np.cumsum(la, axis=1))  # [1, T, H]
    for h in range(2):
        want_o = gam[0, :, h, None] * (q[0, :, h] @ S0[0, h].T)
        assert np.abs(o[0, :, h] - want_o).max() < 1e-13
        assert np.abs(fin[0, h] - gam[0, -1, h] * S0[0, h]).max() < 1e-13


def pin_alpha_to_zero(lib):
    """alpha -> 0 clears memory (paper, introduction): with log alpha = -60,
    S_t = beta_t v_t k_t^T and o_t = beta_t (k_t . q_t) v_t, with no NaN."""
    rng = np.random.default_rng(14)
    q, k, v, _, b = _rand_inputs(rng, 1, 30, 3, 8, 6)
    S0 = rng.standard_normal((1, 3, 6, 8))
    la = np.full(b.shape, -60.0)
    o, fin = oracle.recurrent(q, k, v, la, b, init_state=S0, lib=lib)
    assert np.isfinite(o).all() and np.isfinite(fin).all()
    kq = (k * q).sum(-1)
    want = b[..., None] * kq[..., None] * v
    assert np.abs(o - want).max() < 1e-12
    want_S = b[0, -1, :, None, None] * v[0, -1, :, :, None] * k[0, -1, :, None, :]
    assert np.abs(fin[0] - want_S).max() < 1e-12


def pin_ssd_closed_form(lib):
    """Orthonormal keys and S_0 = 0 (L <= dk): the delta correction vanishes
    and the layer equals the decayed linear attention in its parallel form
    O = ((Q K^T) o Gamma)(diag(beta) V), Gamma_ij = gamma_i / gamma_j for
    i >= j (paper 2.1, the SSD matrix form; blog section on Mamba2)."""
    rng = np.random.default_rng(15)
    L, dk, dv = 12, 16, 7
    Qo, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    K = Qo[:L]                             # orthonormal rows
    Q = _unit(rng.standard_normal((L, dk)))
    V = rng.standard_normal((L, dv))
    la = rng.uniform(-0.3, -0.01, size=L)
    b = rng.uniform(0.1, 0.9, size=L)
    o, _ = oracle.recurrent(Q.reshape(1, L, 1, dk), K.reshape(1, L, 1, dk),
                            V.reshape(1, L, 1, dv), la.reshape(1, L, 1), b.reshape(1, L, 1),
                            lib=lib)
    gam = np.exp(np.cumsum(la))
    Gam = np.tril(gam[:, None] / gam[None, :])
    want = ((Q @ K.T) * Gam) @ (b[:, None] * V)
    assert np.abs(o[0, :, 0] - want).max() < 1e-13


def pin_naive_product(lib):
    """Brute force: the ordered-step recurrence equals multiplying explicit
    transition matrices, S_t = S_{t-1} A_t + B_t with A_t = alpha_t (I - beta_t
    k_t k_t^T), B_t = beta_t v_t k_t^T (tutorial, decode recursion; paper eq. 10)."""
    rng = np.random.default_rng(16)
    for (T, H, dk, dv) in [(8, 2, 4, 3), (5, 1, 3, 4), (7, 3, 2, 2)]:
        q, k, v, la, b = _rand_inputs(rng, 2, T, H, dk, dv, la_range=(-0.7, -0.01))
        S0 = rng.standard_normal((2, H, dv, dk))
        o1, f1 = oracle.recurrent(q, k, v, la, b, init_state=S0, lib=lib)
        o2, f2 = oracle.naive_product(q, k, v, la, b, init_state=S0, lib=lib)
        assert np.abs(o1 - o2).max() < 1e-13 and np.abs(f1 - f2).max() < 1e-13


def pin_composition_order(lib):
    """Two steps compose in order: S_{t+1} = S_{t-1} A_t A_{t+1} + B_t A_{t+1}
    + B_{t+1}; the swapped product differs (tutorial, decode recursion)."""
    rng = np.random.default_rng(17)
    dk, dv = 4, 3
    S0 = rng.standard_normal((dv, dk))
    ks = _unit(rng.standard_normal((2, dk)))
    vs = rng.standard_normal((2, dv))
    al, be = [0.7, 0.9], [0.6, 0.3]
    A = [al[i] * (np.eye(dk) - be[i] * np.outer(ks[i], ks[i])) for i in range(2)]
    Bm = [be[i] * np.outer(vs[i], ks[i]) for i in range(2)]
    want = S0 @ A[0] @ A[1] + Bm[0] @ A[1] + Bm[1]
    swapped = S0 @ A[1] @ A[0] + Bm[1] @ A[0] + Bm[0]
    _, fin = oracle.recurrent(np.zeros((1, 2, 1, dk)), ks.reshape(1, 2, 1, dk),
                              vs.reshape(1, 2, 1, dv), np.log(al).reshape(1, 2, 1),
                              np.array(be).reshape(1, 2, 1), init_state=S0.reshape(1, 1, dv, dk),
                              lib=lib)
    assert np.abs(fin[0, 0] - want).max() < 1e-13
    assert np.abs(fin[0, 0] - swapped).max() > 1e-3


def pin_chunked_matches_recurrent(lib, chunked_fn=None):
    """The chunkwise WY/UT form reproduces eq. (10) at any chunk size, with
    partial last chunks, alpha = 1 (DeltaNet) and alpha -> 0."""
    chunked_fn = chunked_fn or oracle.chunked
    rng = np.random.default_rng(18)
    q, k, v, la, b = _rand_inputs(rng, 2, 150, 2, 12, 10)
    S0 = 0.3 * rng.standard_normal((2, 2, 10, 12))
    o_r, f_r = oracle.recurrent(q, k, v, la, b, init_state=S0, lib=lib)
    scale = np.sqrt((o_r ** 2).mean())
    for C in (16, 37, 64):
        o_c, f_c = chunked_fn(q, k, v, la, b, init_state=S0, chunk=C)
        assert np.abs(o_c - o_r).max() < 1e-12 * max(1.0, scale), C
        assert np.abs(f_c - f_r).max() < 1e-12
    for la_case in (np.zeros_like(la), np.full_like(la, -60.0)):
        o_r, f_r = oracle.recurrent(q, k, v, la_case, b, init_state=S0, lib=lib)
        o_c, f_c = chunked_fn(q, k, v, la_case, b, init_state=S0, chunk=32)
        assert np.isfinite(o_c).all()
        assert np.abs(o_c - o_r).max() < 1e-11 and np.abs(f_c - f_r).max() < 1e-11


def pin_resume(lib):
    """Save-then-resume equals one uninterrupted run (tutorial: the single-step,
    chunked-prefill and resume paths must agree; no reset inside a request)."""
    rng = np.random.default_rng(19)
    q, k, v, la, b = _rand_inputs(rng, 1, 100, 2, 8, 6)
    S0 = rng.standard_normal((1, 2, 6, 8))
    o, f = oracle.recurrent(q, k, v, la, b, init_state=S0, lib=lib)
    for split in (1, 37, 64, 99):
        sl1, sl2 = slice(0, split), slice(split, 100)
        o1, f1 = oracle.recurrent(q[:, sl1], k[:, sl1], v[:, sl1], la[:, sl1], b[:, sl1],
                                  init_state=S0, lib=lib)
        o2, f2 = oracle.recurrent(q[:, sl2], k[:, sl2], v[:, sl2], la[:, sl2], b[:, sl2],
                                  init_state=f1, lib=lib)
        assert np.abs(np.concatenate([o1, o2], axis=1) - o).max() < 1e-13
        assert np.abs(f2 - f).max() < 1e-13


def pin_packed_vs_separate(lib):
    """A packed batch resets the state at every boundary: equal to separate
    runs, including an empty sequence, and a NaN in one sequence stays there."""
    rng = np.random.default_rng(20)
    lens = [5, 0, 17, 1, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q, k, v, la, b = _rand_inputs(rng, 1, T, 2, 6, 4)
    S0 = rng.standard_normal((len(lens), 2, 4, 6))
    o, f = oracle.recurrent(q, k, v, la, b, init_state=S0, cu_seqlens=cu, lib=lib)
    for n in range(len(lens)):
        s, e = cu[n], cu[n + 1]
        on, fn = oracle.recurrent(q[:, s:e], k[:, s:e], v[:, s:e], la[:, s:e], b[:, s:e],
                                  init_state=S0[n:n + 1], lib=lib)
        assert np.array_equal(on, o[:, s:e]) and np.array_equal(fn[0], f[n])
    assert np.array_equal(f[1], S0[1])            # empty sequence: final = initial
    v_bad = v.copy()
    v_bad[0, cu[2] + 3, 1, 0] = np.nan
    o2, f2 = oracle.recurrent(q, k, v_bad, la, b, init_state=S0, cu_seqlens=cu, lib=lib)
    for n in (0, 1, 3, 4):
        s, e = cu[n], cu[n + 1]
        assert np.array_equal(o2[:, s:e], o[:, s:e]) and np.array_equal(f2[n], f[n])


def pin_linearity(lib):
    """For fixed q, k, alpha, beta the map (S_0, V) -> (O, S_T) is linear
    (eq. 10 is affine in S with the write term linear in v)."""
    rng = np.random.default_rng(21)
    q, k, v1, la, b = _rand_inputs(rng, 1, 33, 2, 7, 5)
    v2 = rng.standard_normal(v1.shape)
    S1, S2 = rng.standard_normal((2, 1, 2, 5, 7))
    a1, a2 = 0.7, -1.3
    o1, f1 = oracle.recurrent(q, k, v1, la, b, init_state=S1, lib=lib)
    o2, f2 = oracle.recurrent(q, k, v2, la, b, init_state=S2, lib=lib)
    o3, f3 = oracle.recurrent(q, k, a1 * v1 + a2 * v2, la, b, init_state=a1 * S1 + a2 * S2,
                              lib=lib)
    assert np.abs(o3 - (a1 * o1 + a2 * o2)).max() < 1e-12
    assert np.abs(f3 - (a1 * f1 + a2 * f2)).max() < 1e-12


def pin_contraction(lib):
    """For unit keys and beta in [0, 2], ||alpha (I - beta k k^T)||_2 <= alpha,
    so ||S_t||_F <= alpha_t ||S_{t-1}||_F + beta_t ||v_t|| (paper 2.2: the
    transition is a generalized Householder matrix)."""
    rng = np.random.default_rng(22)
    T, dk, dv = 50, 8, 5
    q, k, v, la, _ = _rand_inputs(rng, 1, T, 1, dk, dv)
    b = rng.uniform(0.0, 2.0, size=(1, T, 1))
    S = rng.standard_normal((1, 1, dv, dk))
    for t in range(T):
        _, f = oracle.recurrent(q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1], la[:, t:t + 1],
                                b[:, t:t + 1], init_state=S, lib=lib)
        bound = np.exp(la[0, t, 0]) * np.linalg.norm(S) + b[0, t, 0] * np.linalg.norm(v[0, t, 0])
        assert np.linalg.norm(f) <= bound * (1 + 1e-12)
        S = f


def pin_l2_normalise(lib):
    """q/k normalisation (paper 3.4, token mixer block): unit norms, the same
    direction (x = ||x|| x_hat), and an all-zero vector stays zero."""
    rng = np.random.default_rng(23)
    x = rng.standard_normal((3, 7, 16)) * rng.uniform(0.1, 10.0, size=(3, 7, 1))
    x[1, 2] = 0.0
    y = oracle.l2_normalise(x)
    n = np.linalg.norm(y, axis=-1)
    n[1, 2] = 1.0
    assert np.abs(n - 1.0).max() < 1e-14
    assert np.abs(y[1, 2]).max() == 0.0
    assert np.abs(np.linalg.norm(x, axis=-1, keepdims=True) * y - x).max() < 1e-12


def pin_qk_l2norm_scale_invariance(lib):
    """With q/k normalisation the result does not depend on the length of any
    q_t or k_t: positive per-(token, head) scalings of q and k leave o and the
    final state unchanged, and on unit q, k the option is the identity.  A
    normalisation applied to only one of q, k, or not at all, fails this."""
    rng = np.random.default_rng(24)
    B, T, H, dk, dv = 2, 70, 2, 16, 8
    q, k, v, la, b = _rand_inputs(rng, B, T, H, dk, dv)
    S0 = 0.1 * rng.standard_normal((B, H, dv, dk))
    o1, f1 = oracle.recurrent(q, k, v, la, b, init_state=S0, lib=lib)
    o2, f2 = oracle.recurrent(q, k, v, la, b, init_state=S0, lib=lib, qk_l2norm=True)
    assert max(np.abs(o1 - o2).max(), np.abs(f1 - f2).max()) < 1e-12
    cq = rng.uniform(0.2, 5.0, size=(B, T, H, 1))
    ck = rng.uniform(0.2, 5.0, size=(B, T, H, 1))
    o3, f3 = oracle.recurrent(cq * q, ck * k, v, la, b, init_state=S0, lib=lib, qk_l2norm=True)
    assert max(np.abs(o1 - o3).max(), np.abs(f1 - f3).max()) < 1e-12
    o4, _ = oracle.recurrent(cq * q, ck * k, v, la, b, init_state=S0, lib=lib)
    assert np.abs(o4 - o1).max() > 1e-3      # without the option the scalings matter


def pin_l2_normalise_bwd(lib):
    """The normalisation's gradient equals the central finite difference of
    sum(g * l2_normalise(x)) on every element; it is orthogonal to x (the
    normalisation ignores the length), scales as 1/c under x -> c x, and is
    zero for an all-zero x."""
    rng = np.random.default_rng(25)
    x = rng.standard_normal((4, 3, 6)) * rng.uniform(0.2, 5.0, size=(4, 3, 1))
    x[2, 1] = 0.0
    g = rng.standard_normal(x.shape)
    d = oracle.l2_normalise_bwd(x, g)
    h = 1e-6
    for pos in np.ndindex(*x.shape):
        if pos[:2] == (2, 1):
            continue
        xp, xm = x.copy(), x.copy()
        xp[pos] += h
        xm[pos] -= h
        fd = float((g * (oracle.l2_normalise(xp) - oracle.l2_normalise(xm))).sum()) / (2 * h)
        assert abs(fd - d[pos]) <= 1e-7 * (1.0 + abs(fd)), (pos, fd, d[pos])
    assert np.abs((x * d).sum(axis=-1)).max() < 1e-12
    assert np.abs(d[2, 1]).max() == 0.0
    assert np.abs(oracle.l2_normalise_bwd(3.5 * x, g) - d / 3.5).max() < 1e-12


def pin_bwd_l2norm_finite_difference(lib):
    """recurrent_bwd(..., qk_l2norm=True) equals the central finite difference
    of the loss of recurrent(..., qk_l2norm=True) on every element of q and k
    (raw vectors of different lengths), and its other gradients equal those
    of the rule on the normalised q, k."""
    rng = np.random.default_rng(26)
    T, H, dk, dv = 5, 2, 4, 3
    q, k, v, la, b = _rand_inputs(rng, 1, T, H, dk, dv, la_range=(-0.7, -0.05))
    q = q * rng.uniform(0.3, 3.0, size=(1, T, H, 1))
    k = k * rng.uniform(0.3, 3.0, size=(1, T, H, 1))
    S0 = rng.standard_normal((1, H, dv, dk))
    Wo = rng.standard_normal((1, T, H, dv))
    WS = rng.standard_normal((1, H, dv, dk))

    def loss(qq, kk):
        o, fin = oracle.recurrent(qq, kk, v, la, b, init_state=S0, lib=lib, qk_l2norm=True)
        return float((Wo * o).sum() + (WS * fin).sum())

    grads = oracle.recurrent_bwd(q, k, v, la, b, Wo, init_state=S0, d_final=WS, lib=lib, qk_l2norm=True)
    h = 1e-6
    for idx, x in enumerate((q, k)):
        for pos in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[pos] += h
            xm[pos] -= h
            fd = (loss(xp, k) - loss(xm, k)) / (2 * h) if idx == 0 else (loss(q, xp) - loss(q, xm)) / (2 * h)
            assert abs(fd - grads[idx][pos]) <= 1e-6 * (1.0 + abs(fd)), (idx, pos, fd, grads[idx][pos])
    plain = oracle.recurrent_bwd(oracle.l2_normalise(q), oracle.l2_normalise(k), v, la, b, Wo, init_state=S0,
                                 d_final=WS, lib=lib)
    for x, y in zip(grads[2:], plain[2:]):
        assert np.abs(x - y).max() < 1e-12


# -- gradients ------------------------------------------------------------------

def _loss(lib, q, k, v, la, b, S0, cu, Wo, WS):
    o, fin = oracle.recurrent(q, k, v, la, b, init_state=S0, cu_seqlens=cu, lib=lib)
    return float((Wo * o).sum() + (WS * fin).sum())


def pin_bwd_finite_difference(lib):
    """Every gradient recurrent_bwd returns equals the central finite
    difference of the loss sum(Wo * o) + sum(WS * S_final) computed with the
    forward oracle, element by element, on a packed batch with an empty
    sequence and initial states (q, k, v, log alpha, beta and S_0)."""
    rng = np.random.default_rng(30)
    lens = [3, 0, 5]
    cu = np.cumsum([0] + lens)
    T, H, dk, dv = int(cu[-1]), 2, 4, 3
    q, k, v, la, b = _rand_inputs(rng, 1, T, H, dk, dv, la_range=(-0.7, -0.05))
    b = rng.uniform(0.1, 1.9, size=b.shape)
    S0 = rng.standard_normal((len(lens), H, dv, dk))
    Wo = rng.standard_normal((1, T, H, dv))
    WS = rng.standard_normal((len(lens), H, dv, dk))
    grads = oracle.recurrent_bwd(q, k, v, la, b, Wo, init_state=S0, d_final=WS, cu_seqlens=cu, lib=lib)
    args = [q, k, v, la, b, S0]
    h = 1e-6
    for idx, (x, g) in enumerate(zip(args, grads)):
        assert g.shape == x.shape, (idx, g.shape, x.shape)
        for pos in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[pos] += h
            xm[pos] -= h
            ap, am = list(args), list(args)
            ap[idx], am[idx] = xp, xm
            fd = (_loss(lib, *ap, cu, Wo, WS) - _loss(lib, *am, cu, Wo, WS)) / (2 * h)
            assert abs(fd - g[pos]) <= 1e-6 * (1.0 + abs(fd)), (idx, pos, fd, g[pos])


def pin_bwd_frozen_state(lib):
    """alpha = 1, beta = 0 freeze the state (S_t = S_0, o_t = S_0 q_t), so
    with G_t = d_final + sum_{s >= t} do_s q_s^T the gradients are
    dq_t = S_0^T do_t, dv = dk = 0, dbeta_t = (G_t k_t) . (v_t - S_0 k_t),
    dlog_alpha_t = <G_t, S_0> and d_S0 = G_1."""
    rng = np.random.default_rng(31)
    T, dk, dv = 9, 5, 4
    q, k, v, _, _ = _rand_inputs(rng, 1, T, 1, dk, dv)
    la, b = np.zeros((1, T, 1)), np.zeros((1, T, 1))
    S0 = rng.standard_normal((1, 1, dv, dk))
    do = rng.standard_normal((1, T, 1, dv))
    dfin = rng.standard_normal((1, 1, dv, dk))
    dq, dkk, dvv, dla, db, dinit = oracle.recurrent_bwd(q, k, v, la, b, do, init_state=S0, d_final=dfin,
                                                        lib=lib)
    S = S0[0, 0]
    G = dfin[0, 0].copy()
    for t in range(T - 1, -1, -1):
        G += np.outer(do[0, t, 0], q[0, t, 0])
        assert np.abs(dq[0, t, 0] - S.T @ do[0, t, 0]).max() < 1e-12
        assert abs(db[0, t, 0] - (G @ k[0, t, 0]) @ (v[0, t, 0] - S @ k[0, t, 0])) < 1e-12
        assert abs(dla[0, t, 0] - (G * S).sum()) < 1e-12
    assert np.abs(dvv).max() == 0.0 and np.abs(dkk).max() < 1e-12
    assert np.abs(dinit[0, 0] - G).max() < 1e-12


def pin_bwd_linearity(lib):
    """The gradients are linear in the incoming gradients (d_o, d_final)."""
    rng = np.random.default_rng(32)
    B, T, H, dk, dv = 2, 11, 2, 6, 5
    q, k, v, la, b = _rand_inputs(rng, B, T, H, dk, dv)
    S0 = rng.standard_normal((B, H, dv, dk))
    do1, do2 = rng.standard_normal((2, B, T, H, dv))
    df1, df2 = rng.standard_normal((2, B, H, dv, dk))
    a1, a2 = 0.6, -1.7
    g1 = oracle.recurrent_bwd(q, k, v, la, b, do1, init_state=S0, d_final=df1, lib=lib)
    g2 = oracle.recurrent_bwd(q, k, v, la, b, do2, init_state=S0, d_final=df2, lib=lib)
    g3 = oracle.recurrent_bwd(q, k, v, la, b, a1 * do1 + a2 * do2, init_state=S0,
                              d_final=a1 * df1 + a2 * df2, lib=lib)
    for x1, x2, x3 in zip(g1, g2, g3):
        assert np.abs(x3 - (a1 * x1 + a2 * x2)).max() < 1e-11


ALL_PINS = [pin_worked_example, pin_delta_vs_additive, pin_interpolation,
            pin_orthogonal_untouched, pin_beta_zero_pure_decay, pin_alpha_to_zero,
            pin_ssd_closed_form, pin_naive_product, pin_composition_order,
            pin_chunked_matches_recurrent, pin_resume, pin_packed_vs_separate, pin_linearity,
            pin_contraction, pin_l2_normalise, pin_qk_l2norm_scale_invariance,
            pin_bwd_finite_difference, pin_bwd_frozen_state, pin_bwd_linearity,
            pin_l2_normalise_bwd, pin_bwd_l2norm_finite_difference]
