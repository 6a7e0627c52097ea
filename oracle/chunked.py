"""Chunkwise (WY/UT) form of the gated delta rule in numpy fp64.

TEST INFRASTRUCTURE (part of the oracle package).  It restates the chunked
algorithm so that the per-chunk intermediates (Gamma, A, T, W, U, P, the
chunk-start states) can be inspected; it is pinned to the token recurrence in
tests/test_oracle_pins.py (agreement to ~1e-13 at several chunk sizes,
partial last chunks, alpha = 1 and alpha -> 0).

Notation (row-stacked chunk blocks, tokens as rows; paper-notes blog,
"Chunkwise Training", which fixes the row convention the paper mixes):
  g_r      = sum_{i<=r} log alpha_i inside the chunk, so gamma^r = exp(g_r)
             (inclusive of token r, gamma^0 = 1)            [paper 2.1, eq. (2)]
  Gamma_ri = exp(g_r - g_i) for i <= r, else 0  (masked before exp, so the
             unmasked upper triangle never overflows)        [paper 3.3; blog (3)]
  A        = strictLower(diag(beta) (Gamma o K K^T))
  T        = (I + A)^{-1}                                   [paper 3.3, UT transform]
  W_dec    = T diag(beta) diag(gamma) K   (W with the left arrow)
  U        = T diag(beta) V               (U tilde)
  V'       = U - W_dec S^T                (effective values)
  O        = diag(gamma) Q S^T + (Q K^T o Gamma) V'         [blog (4) summary]
  S_next   = gamma^C S + V'^T diag(gamma^C / gamma^r) K     [paper 3.3]

Reading notes (each also listed with its evidence in the repository's design
notes): the output mask is the decay mask Gamma, not the causal 0/1 mask the
translated paper prints in section 3.3 (the blog derives Gamma and flags the
printed M; with M the result departs from eq. (10) whenever alpha != 1).
W_dec computed as T diag(beta gamma) K with T from the Gamma-weighted A equals
the blog's diag(gamma) [(I + strictLower(diag(beta) K K^T))^{-1} diag(beta) K],
because I + A_Gamma = diag(gamma) (I + L) diag(gamma)^{-1}.
"""
from __future__ import annotations

import numpy as np


def _chunk(Q, K, V, la, b, S):
    """One chunk; returns (O, S_next, intermediates)."""
    c = Q.shape[0]
    g = np.cumsum(la)
    incl = np.tril(np.ones((c, c), dtype=bool))
    diff = np.where(incl, g[:, None] - g[None, :], 0.0)
    Gamma = np.where(incl, np.exp(diff), 0.0)
    A = np.tril(b[:, None] * (Gamma * (K @ K.T)), -1)
    T = np.linalg.inv(np.eye(c) + A)
    gam = np.exp(g)
    W_dec = T @ (b[:, None] * gam[:, None] * K)
    U = T @ (b[:, None] * V)
    Vp = U - W_dec @ S.T
    P = (Q @ K.T) * Gamma
    O = gam[:, None] * (Q @ S.T) + P @ Vp
    K_end = np.exp(g[-1] - g)[:, None] * K
    S_next = np.exp(g[-1]) * S + Vp.T @ K_end
    inter = dict(g=g, Gamma=Gamma, A=A, T=T, W_dec=W_dec, U=U, Vp=Vp, P=P, S_start=S)
    return O, S_next, inter


def chunked_single(q, k, v, log_alpha, beta, S0=None, chunk=64, keep=False):
    """One (sequence, head): q,k [L,dk], v [L,dv], log_alpha, beta [L],
    S0 [dv,dk] or None.  Chunks start at token 0; the last may be partial.
    Returns (o [L,dv], S_final [dv,dk], list of per-chunk intermediates)."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    la, b = np.asarray(log_alpha, np.float64), np.asarray(beta, np.float64)
    L, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((L, dv))
    inters = []
    for s in range(0, L, chunk):
        e = min(L, s + chunk)
        O, S, inter = _chunk(q[s:e], k[s:e], v[s:e], la[s:e], b[s:e], S)
        o[s:e] = O
        if keep:
            inters.append(inter)
    return o, S, inters


def chunked(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None, chunk=64):
    """Batched/packed wrapper with the same conventions as oracle.recurrent."""
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    la, b = np.asarray(log_alpha), np.asarray(beta)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is None:
        bounds = [(bb, 0, T) for bb in range(B)]
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        bounds = [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
    o = np.zeros((B, T, H, dv))
    fin = np.zeros((len(bounds), H, dv, dk))
    for n, (bb, s, e) in enumerate(bounds):
        for h in range(H):
            S0 = None if init_state is None else init_state[n, h]
            if e > s:
                oo, S, _ = chunked_single(q[bb, s:e, h], k[bb, s:e, h], v[bb, s:e, h],
                                          la[bb, s:e, h], b[bb, s:e, h], S0, chunk)
                o[bb, s:e, h] = oo
            else:
                S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
            fin[n, h] = S
    return o, fin
