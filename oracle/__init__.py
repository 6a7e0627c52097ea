"""CPU fp64 oracle of the gated delta rule -- TEST INFRASTRUCTURE.

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of
`bench.py` may import this package.  It shares no code with the HIP path
(`gated_delta_rule_24_amd`), and neither imports the other.

Functions:
  recurrent(...)      the definition, token by token (C, fp64, OpenMP over
                      independent (sequence, head) chains)   -- THE oracle
  naive_product(...)  explicit dk x dk transition matrices (C, fp64), for
                      brute force on tiny inputs
  chunked(...)        the chunkwise WY/UT form in numpy fp64, exposing the
                      per-chunk intermediates (see oracle/chunked.py)
  checked_step(...)   one token on a single head with the method's
                      preconditions enforced (shapes, finite entries, gates
                      in [0, 1], unit key)
  l2_normalise(x)     x / ||x||_2 per vector (fp64), the q/k normalisation of
                      the paper's token-mixer block; recurrent(...,
                      qk_l2norm=True) applies it to q and k first
  recurrent_bwd(...)  gradients of recurrent() with respect to q, k, v,
                      log alpha, beta and the initial state, given the
                      gradients of o and of the final state (C, fp64, the
                      chain rule through each token, newest first);
                      qk_l2norm=True differentiates recurrent(...,
                      qk_l2norm=True)
  l2_normalise_bwd(x, g)  the gradient through l2_normalise (fp64)

Parity pins (all in tests/test_oracle_pins.py): the tutorial's worked
two-cell example (tests/golden/), the delta-vs-additive 1-D example, the
unit-key interpolation identity, untouched orthogonal directions, beta = 0
pure decay, alpha -> 0 memory clearing, the SSD decay-mask closed form with
orthonormal keys, brute force against naive_product, chunk-size invariance of
chunked(), save-then-resume, packed-vs-separate, linearity in (S0, v), the
contraction bound, and for the q/k normalisation unit norms, kept directions,
invariance of the result under positive per-token scaling of q and k, and
zero vectors staying zero; for the gradients, central finite differences of
recurrent() on every input element (packed sequences, initial and final
state terms included), the closed form at alpha = 1, beta = 0 (a frozen
state), and linearity in (d_o, d_final); for the normalisation's gradient,
central finite differences of l2_normalise and of recurrent(...,
qk_l2norm=True), orthogonality to x, the 1/c scaling and zero vectors.  No function here is "parity
unpinned".
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import numpy as np

from . import chunked as _chunked_mod

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "liboracle.so")
_lib = None


def load(path: Optional[str] = None):
    """Load (building first if absent) the oracle library."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        from . import build as _b
        _b.build(p)
    lib = ctypes.CDLL(p)
    dp = ctypes.POINTER(ctypes.c_double)
    lp = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    lib.oracle_gdn_recurrent.argtypes = [i64, lp, i64, i64, i64, dp, dp, dp, dp, dp, dp, dp, dp,
                                         ctypes.c_int]
    lib.oracle_gdn_recurrent.restype = ctypes.c_int
    lib.oracle_gdn_naive_product.argtypes = [i64, lp, i64, i64, i64, dp, dp, dp, dp, dp, dp, dp,
                                             dp]
    lib.oracle_gdn_naive_product.restype = ctypes.c_int
    lib.oracle_gdn_recurrent_bwd.argtypes = [i64, lp, i64, i64, i64, dp, dp, dp, dp, dp, dp, dp, dp,
                                             dp, dp, dp, dp, dp, dp, ctypes.c_int]
    lib.oracle_gdn_recurrent_bwd.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _flatten(q, k, v, log_alpha, beta, cu_seqlens):
    """[B,T,H,d] (or [T,H,d]) inputs -> packed [B*T,H,d] plus cu offsets."""
    q = np.asarray(q)
    if q.ndim == 3:
        q, k, v = q[None], np.asarray(k)[None], np.asarray(v)[None]
        log_alpha, beta = np.asarray(log_alpha)[None], np.asarray(beta)[None]
    B, T, H, dk = q.shape
    dv = np.asarray(v).shape[-1]
    if cu_seqlens is None:
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        if B != 1:
            raise ValueError("cu_seqlens requires a packed batch (B == 1)")
        cu = np.asarray(cu_seqlens, dtype=np.int64)
    return (B, T, H, dk, dv, cu, _f64(q).reshape(B * T, H, dk), _f64(k).reshape(B * T, H, dk),
            _f64(v).reshape(B * T, H, dv), _f64(log_alpha).reshape(B * T, H),
            _f64(beta).reshape(B * T, H))


def l2_normalise(x):
    """x / ||x||_2 over the last axis, in fp64.  The Gated DeltaNet paper
    L2-normalises q and k before the gated delta rule (section 3.4, token
    mixer block; the paper notes list it for training stability).  The pages
    give no epsilon; an all-zero vector is left as zero."""
    x = _f64(x)
    n = np.sqrt((x * x).sum(axis=-1, keepdims=True))
    return np.divide(x, n, out=np.zeros_like(x), where=n > 0)


def l2_normalise_bwd(x, d_xhat):
    """Gradient through l2_normalise, in fp64: given g = dL/dx^ for
    x^ = x / ||x|| (last axis), returns dL/dx.  The Jacobian of x / ||x|| is
    (I - x^ x^T) / ||x|| (symmetric), so dL/dx = (g - x^ (x^ . g)) / ||x||.
    The pages give no gradients; this is the derivative of the definition
    above.  An all-zero x, which l2_normalise leaves at zero, gets a zero
    gradient."""
    x, g = _f64(x), _f64(d_xhat)
    n = np.sqrt((x * x).sum(axis=-1, keepdims=True))
    xh = np.divide(x, n, out=np.zeros_like(x), where=n > 0)
    along = (xh * g).sum(axis=-1, keepdims=True)
    return np.divide(g - xh * along, n, out=np.zeros_like(x), where=n > 0)


def recurrent(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None, threads=0,
              lib=None, qk_l2norm=False):
    """Token-by-token recurrence in fp64.

    q, k: [B,T,H,dk]; v: [B,T,H,dv]; log_alpha, beta: [B,T,H] (any float
    dtype; widened to fp64).  With cu_seqlens (int [N+1]) the batch is packed
    (B == 1) and sequence n covers tokens cu[n]..cu[n+1]-1.  qk_l2norm:
    l2_normalise q and k first.
    Returns (o [B,T,H,dv] fp64, final_state [N,H,dv,dk] fp64).
    """
    if qk_l2norm:
        q, k = l2_normalise(q), l2_normalise(k)
    B, T, H, dk, dv, cu, qf, kf, vf, laf, bf = _flatten(q, k, v, log_alpha, beta, cu_seqlens)
    N = len(cu) - 1
    o = np.zeros((B * T, H, dv), dtype=np.float64)
    fin = np.zeros((N, H, dv, dk), dtype=np.float64)
    init = None if init_state is None else _f64(init_state).reshape(N, H, dv, dk)
    lib = lib or load()
    rc = lib.oracle_gdn_recurrent(N, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, dk,
                                  dv, _ptr(qf), _ptr(kf), _ptr(vf), _ptr(laf), _ptr(bf),
                                  _ptr(init), _ptr(o), _ptr(fin), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_gdn_recurrent failed with code {rc}")
    return o.reshape(B, T, H, dv), fin


def recurrent_bwd(q, k, v, log_alpha, beta, d_o, init_state=None, d_final=None, cu_seqlens=None,
                  threads=0, lib=None, qk_l2norm=False):
    """Gradients of recurrent(...) in fp64: the chain rule through each token
    of the recurrence, newest first (see oracle_gdn_recurrent_bwd in
    gdn_oracle.c for the step).  The pages give no gradient formulas.

    d_o: [B,T,H,dv], the gradient of a loss with respect to o; d_final:
    [N,H,dv,dk] or None (zeros), its gradient with respect to the final state.
    Returns (dq, dk [B,T,H,dk], dv [B,T,H,dv], dlog_alpha, dbeta [B,T,H],
    d_init [N,H,dv,dk]), all fp64.  Memory per (sequence, head) chain is
    (L + 1) dv dk doubles for a sequence of L tokens.  qk_l2norm: the
    gradients of recurrent(..., qk_l2norm=True), i.e. those of the rule on
    the normalised q, k carried back through l2_normalise_bwd.
    """
    if qk_l2norm:
        qn, kn = l2_normalise(q), l2_normalise(k)
        dq, dkk, *rest = recurrent_bwd(qn, kn, v, log_alpha, beta, d_o, init_state, d_final, cu_seqlens,
                                       threads, lib)
        return (l2_normalise_bwd(q, dq), l2_normalise_bwd(k, dkk), *rest)
    B, T, H, dk, dv, cu, qf, kf, vf, laf, bf = _flatten(q, k, v, log_alpha, beta, cu_seqlens)
    N = len(cu) - 1
    dof = _f64(d_o).reshape(B * T, H, dv)
    init = None if init_state is None else _f64(init_state).reshape(N, H, dv, dk)
    dfin = None if d_final is None else _f64(d_final).reshape(N, H, dv, dk)
    dq = np.zeros((B * T, H, dk))
    dkk = np.zeros((B * T, H, dk))
    dvv = np.zeros((B * T, H, dv))
    dla = np.zeros((B * T, H))
    db = np.zeros((B * T, H))
    dinit = np.zeros((N, H, dv, dk))
    lib = lib or load()
    rc = lib.oracle_gdn_recurrent_bwd(N, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, dk, dv,
                                      _ptr(qf), _ptr(kf), _ptr(vf), _ptr(laf), _ptr(bf), _ptr(init),
                                      _ptr(dof), _ptr(dfin), _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dla),
                                      _ptr(db), _ptr(dinit), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_gdn_recurrent_bwd failed with code {rc}")
    return (dq.reshape(B, T, H, dk), dkk.reshape(B, T, H, dk), dvv.reshape(B, T, H, dv),
            dla.reshape(B, T, H), db.reshape(B, T, H), dinit)


def naive_product(q, k, v, log_alpha, beta, init_state=None, cu_seqlens=None, lib=None):
    """Brute-force form with explicit transition matrices (tiny inputs only)."""
    B, T, H, dk, dv, cu, qf, kf, vf, laf, bf = _flatten(q, k, v, log_alpha, beta, cu_seqlens)
    N = len(cu) - 1
    o = np.zeros((B * T, H, dv), dtype=np.float64)
    fin = np.zeros((N, H, dv, dk), dtype=np.float64)
    init = None if init_state is None else _f64(init_state).reshape(N, H, dv, dk)
    lib = lib or load()
    rc = lib.oracle_gdn_naive_product(N, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H,
                                      dk, dv, _ptr(qf), _ptr(kf), _ptr(vf), _ptr(laf), _ptr(bf),
                                      _ptr(init), _ptr(o), _ptr(fin))
    if rc != 0:
        raise ValueError(f"oracle_gdn_naive_product failed with code {rc}")
    return o.reshape(B, T, H, dv), fin


def num_threads(lib=None):
    return (lib or load()).oracle_num_threads()


chunked = _chunked_mod.chunked
chunked_single = _chunked_mod.chunked_single


def _step_violations(S, k, v, alpha, beta, unit_tol):
    """The preconditions of one gated-delta step on a single head, as
    (violated?, reason) pairs in the order they are checked.  Later entries
    assume the earlier ones hold (shapes before values)."""
    yield (S.ndim != 2 or S.size == 0 or k.ndim != 1 or v.ndim != 1,
           "the state must be a non-empty dv x dk matrix, key and value vectors")
    yield (S.shape != (v.shape[0], k.shape[0]),
           f"state shape {S.shape} does not match (len(value), len(key)) = {(v.shape[0], k.shape[0])}")
    yield (not (np.isfinite(S).all() and np.isfinite(k).all() and np.isfinite(v).all()
                and np.isfinite([alpha, beta]).all()),
           "every entry must be finite")
    yield (not (0.0 <= alpha <= 1.0) or not (0.0 <= beta <= 1.0),
           f"gate alpha = {alpha} and write strength beta = {beta} must lie in [0, 1]")
    yield (abs(float(np.linalg.norm(k)) - 1.0) > unit_tol,
           f"the key must have unit L2 norm (got {float(np.linalg.norm(k)):.12g})")


def checked_step(S, k, v, alpha, beta, unit_tol=1e-9):
    """One token of the gated delta rule, S_t = alpha S (I - beta k k^T) +
    beta v k^T (the Gated DeltaNet paper's eq. (10), section 3.1), on a
    single head with its preconditions enforced: ValueError if the state is
    not a non-empty dv x dk matrix matching len(v) x len(k), if anything is
    not finite, if alpha or beta leaves [0, 1] (the gate and write strength,
    section 2.2 and 3.1), or if k is not a unit vector within `unit_tol` (the
    token-mixer block L2-normalises keys before the rule, section 3.4).

    S: (dv, dk) array-like, k: (dk,), v: (dv,).  Returns the new state as a
    float64 (dv, dk) array.  The arithmetic is the C recurrence (one token,
    fp64); only the checks live here.
    """
    S = np.asarray(S, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    alpha, beta = float(alpha), float(beta)
    for bad, reason in _step_violations(S, k, v, alpha, beta, unit_tol):
        if bad:
            raise ValueError(reason)
    dv, dk = S.shape
    la = np.full((1, 1, 1), -np.inf if alpha == 0.0 else math.log(alpha))
    _, fin = recurrent(np.zeros((1, 1, 1, dk)), k.reshape(1, 1, 1, dk), v.reshape(1, 1, 1, dv), la,
                       np.full((1, 1, 1), beta), init_state=S.reshape(1, 1, dv, dk))
    return fin[0, 0]
