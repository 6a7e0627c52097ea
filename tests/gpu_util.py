"""Helpers for the GPU parity tests: move seeded workloads to the device, call
the HIP path through the binding, and compare with the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import gated_delta_rule_24_amd as gdn
import oracle
import workloads as W

TORCH_DT = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}

# Parity bounds (max |err| relative to RMS of the oracle's o, applied to o and
# to the final state): 1e-4 for fp32 inputs, 2e-2 for 16-bit inputs with fp32
# accumulation and fp32 state.
TOL = {"fp32": 1e-4, "bf16": 2e-2, "fp16": 2e-2}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(x, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dtype)


def rescale_qk(inp, seed, lo=0.3, hi=3.0, zero_tokens=()):
    """Give every (token, head) of q and k its own length in [lo, hi]
    (re-rounded to the input dtype); `zero_tokens` make q and k all zero."""
    rng = np.random.default_rng(seed)
    for name in ("q", "k"):
        x = getattr(inp, name) * rng.uniform(lo, hi, size=inp.q.shape[:3] + (1,)).astype(np.float32)
        for t in zero_tokens:
            x[:, t] = 0.0
        setattr(inp, name, W.cast(x.astype(np.float32), inp.in_dtype))
    return inp


def run_chunk(inp, out_dtype=torch.float32, init_override="default", final=True, **kw):
    dt = TORCH_DT[inp.in_dtype]
    init = inp.init_state if isinstance(init_override, str) else init_override
    q, k, v = dev(inp.q, dt), dev(inp.k, dt), dev(inp.v, dt)
    la, b = dev(inp.log_alpha), dev(inp.beta)
    S0 = None if init is None else dev(init)
    cu = None if inp.cu_seqlens is None else dev(inp.cu_seqlens, torch.int32)
    o, S = gdn.chunk_fwd(q, k, v, la, b, init_state=S0, cu_seqlens=cu, out_dtype=out_dtype, final_state=final, **kw)
    torch.cuda.synchronize()
    return o, S


def oracle_chunk(inp, heads=None, seqs=None, threads=0, qk_l2norm=False):
    """fp64 oracle on a subset of heads / sequences (all by default).
    Returns (o [B,T,Hs,dv], final [Ns,Hs,dv,dk], heads, seqs)."""
    H = inp.H
    heads = list(range(H)) if heads is None else list(heads)
    bounds = inp.seq_bounds()
    seqs = list(range(len(bounds))) if seqs is None else list(seqs)
    o = np.zeros(inp.q.shape[:2] + (len(heads), inp.dv))
    fin = np.zeros((len(seqs), len(heads), inp.dv, inp.dk))
    for si, n in enumerate(seqs):
        b, s, e = bounds[n]
        sl = (slice(b, b + 1), slice(s, e), heads)
        init = None if inp.init_state is None else inp.init_state[n:n + 1][:, heads]
        oo, ff = oracle.recurrent(inp.q[sl], inp.k[sl], inp.v[sl], inp.log_alpha[sl], inp.beta[sl],
                                  init_state=init, threads=threads, qk_l2norm=qk_l2norm)
        o[b, s:e] = oo[0]
        fin[si] = ff[0]
    return o, fin, heads, seqs


def rel_err(got, want, scale):
    got = np.asarray(got, dtype=np.float64)
    return float(np.abs(got - want).max() / scale) if got.size else 0.0


def check_parity(inp, o_gpu, S_gpu, heads=None, seqs=None, tol=None, label="", qk_l2norm=False):
    """Compare the GPU outputs with the oracle on the chosen heads/sequences.
    Returns (err_o, err_S) as max|err| / RMS(o)."""
    tol = TOL[inp.in_dtype] if tol is None else tol
    o_ref, S_ref, heads, seqs = oracle_chunk(inp, heads, seqs, qk_l2norm=qk_l2norm)
    bounds = inp.seq_bounds()
    mask = np.zeros(inp.q.shape[:2], dtype=bool)
    for n in seqs:
        b, s, e = bounds[n]
        mask[b, s:e] = True
    og = o_gpu.float().cpu().numpy()[:, :, heads]
    o_sel, ref_sel = og[mask], o_ref[mask]
    rms = float(np.sqrt((ref_sel ** 2).mean())) if ref_sel.size else 1.0
    rms = rms if rms > 0 else 1.0
    e_o = rel_err(o_sel, ref_sel, rms)
    e_S = 0.0
    if S_gpu is not None:
        Sg = S_gpu.cpu().numpy()[seqs][:, heads]
        e_S = rel_err(Sg, S_ref, rms)
    log(f"[parity] {label or inp.name}: max|do|/rms={e_o:.3e} max|dS|/rms={e_S:.3e} (tol {tol:.0e}, "
        f"rms {rms:.4f}, heads {heads if len(heads) < 6 else len(heads)}, seqs {len(seqs)})")
    assert np.isfinite(o_sel).all()
    assert e_o <= tol, f"o error {e_o:.3e} > {tol:.0e}"
    assert e_S <= tol, f"state error {e_S:.3e} > {tol:.0e}"
    return e_o, e_S
