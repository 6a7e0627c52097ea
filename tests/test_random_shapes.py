"""GPU parity on seeded random shapes: each case draws the path's shape
parameters (packed or equal-length batch, sequence lengths from empty to a
few chunks, heads, dk, dv, input and output dtypes, initial state or none,
q/k L2 normalisation, gate ranges) from its seed, runs gdn_chunk_fwd through
the C ABI and compares o and the final state with the fp64 oracle.  Half the
cases average at most 16 tokens per sequence, so the short-call kernels are
drawn as often as the chunked passes."""
import numpy as np
import pytest
import torch

import workloads as W

from .gpu_util import TOL, check_parity, log, run_chunk

pytestmark = pytest.mark.gpu

_OUT = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}


def _draw(seed):
    rng = np.random.default_rng(1000 + seed)
    dt = ["fp32", "bf16", "fp16"][rng.integers(3)]
    dk = int(rng.choice([32, 64, 128] + ([256] if dt != "fp32" else [])))
    dv = int(16 * rng.integers(1, 13))
    H = int(rng.integers(1, 4))
    short = seed % 2 == 0
    N = int(rng.integers(1, 7))
    if short:
        lens = [int(x) for x in rng.integers(0, 33, size=N)]
        while sum(lens) > 16 * N:   # keep the call's average at 16 tokens or fewer
            lens[int(np.argmax(lens))] //= 2
    else:
        lens = [int(x) for x in rng.integers(0, 260, size=N)]
        lens[0] = max(lens[0], 17 * N)   # average above 16 tokens
    packed = bool(rng.integers(2)) or len(set(lens)) > 1
    odt = ["fp32", "bf16", "fp16"][rng.integers(3)] if dt != "fp32" else "fp32"
    init = bool(rng.integers(2))
    qk_norm = bool(rng.integers(2))
    gate = ["mild", "strong", "none"][rng.integers(3)]
    return dict(dt=dt, dk=dk, dv=dv, H=H, lens=lens, packed=packed, odt=odt, init=init, qk_norm=qk_norm,
                gate=gate, seed=seed)


@pytest.mark.parametrize("seed", range(24))
def test_random_shape(seed):
    c = _draw(seed)
    name = (f"random {seed}: lens {c['lens']} H{c['H']} dk{c['dk']} dv{c['dv']} {c['dt']}->{c['odt']} "
            f"init {c['init']} l2 {c['qk_norm']} gates {c['gate']}")
    init_std = 0.1 if c["init"] else None
    if c["packed"]:
        inp = W.packed_inputs(c["lens"], H=c["H"], dk=c["dk"], dv=c["dv"], in_dtype=c["dt"], seed=2000 + seed,
                              init_std=init_std, name=name)
    else:
        inp = W.chunk_inputs(len(c["lens"]), c["lens"][0], c["H"], c["dk"], c["dv"], c["dt"], seed=2000 + seed,
                             init_std=init_std, name=name)
    if c["gate"] == "strong":
        inp.log_alpha[:] = inp.log_alpha * 50.0
    elif c["gate"] == "none":
        inp.log_alpha[:] = 0.0
    if c["qk_norm"]:
        inp.k[:] = inp.k * 2.0   # not unit rows (scaled exactly)
    o, S = run_chunk(inp, out_dtype=_OUT[c["odt"]], init_override="default" if c["init"] else None,
                     qk_l2norm=c["qk_norm"])
    log(f"[random] {name}")
    tol = TOL[c["dt"]]
    if c["odt"] != "fp32":
        # o rounded to a 16-bit type: up to half a unit in the last place of
        # the largest |o| on top (strong decay makes max|o| / RMS(o) large)
        of = o.float()
        half_ulp = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}[c["odt"]]
        tol += half_ulp * float(of.abs().max()) / max(float(of.pow(2).mean().sqrt()), 1e-12)
    check_parity(inp, o, S, tol=tol, qk_l2norm=c["qk_norm"])
