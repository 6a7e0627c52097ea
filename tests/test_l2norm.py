"""GPU parity of the fused q/k L2 normalisation (GDN_QK_L2NORM): the HIP path
on q and k of arbitrary per-token lengths against the fp64 oracle that
normalises them first (paper section 3.4, token mixer block)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_24_amd as gdn
import oracle
import workloads as W

from .gpu_util import TOL, check_parity, dev, log, rescale_qk, run_chunk

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,T,H,dk,dv,dt,seed", [
    (2, 200, 3, 128, 128, "bf16", 51),
    (1, 130, 2, 64, 48, "fp32", 52),
    (1, 77, 2, 32, 32, "fp16", 53),
])
def test_chunk_l2norm(B, T, H, dk, dv, dt, seed):
    inp = rescale_qk(W.chunk_inputs(B, T, H, dk, dv, dt, seed=seed, init_std=0.1, name=f"l2norm {dt}"), seed)
    o, S = run_chunk(inp, qk_l2norm=True)
    check_parity(inp, o, S, qk_l2norm=True)


def test_chunk_l2norm_packed_with_zero_vectors():
    lens = [5, 0, 70, 129, 64]
    inp = W.packed_inputs(lens, H=2, dk=128, dv=128, in_dtype="bf16", seed=54, name="l2norm packed")
    inp = rescale_qk(inp, 54, zero_tokens=(3, 80, 150))
    o, S = run_chunk(inp, qk_l2norm=True)
    assert torch.isfinite(o).all() and torch.isfinite(S).all()
    check_parity(inp, o, S, qk_l2norm=True)


def test_chunk_l2norm_is_identity_on_unit_keys():
    # On already normalised q, k the option changes nothing beyond rounding.
    inp = W.chunk_inputs(1, 150, 2, 128, 128, "fp32", seed=55, init_std=0.1)
    o1, S1 = run_chunk(inp)
    o2, S2 = run_chunk(inp, qk_l2norm=True)
    rms = float(o1.pow(2).mean().sqrt())
    e = max(float((o1 - o2).abs().max()), float((S1 - S2).abs().max())) / rms
    log(f"[l2norm identity] {e:.2e}")
    assert e <= TOL["fp32"]


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_decode_l2norm(dt):
    N, H, dk, dv = 3, 4, 128, 64
    d = W.decode_inputs(N, H, dk, dv, pool=3, in_dtype=dt, seed=56)
    rng = np.random.default_rng(56)
    tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[dt]
    state = dev(d.state)
    S_ref = d.state.astype(np.float64)
    worst = 0.0
    for s in range(3):
        q = W.cast((d.q[s] * rng.uniform(0.3, 3.0, size=(N, H, 1))).astype(np.float32), dt)
        k = W.cast((d.k[s] * rng.uniform(0.3, 3.0, size=(N, H, 1))).astype(np.float32), dt)
        if s == 1:
            q[0, 0] = 0.0
            k[1, 2] = 0.0
        o = gdn.decode_step(state, dev(q, tdt), dev(k, tdt), dev(d.v[s], tdt), dev(d.log_alpha[s]), dev(d.beta[s]),
                            qk_l2norm=True)
        torch.cuda.synchronize()
        # each of the N states is a one-token sequence: [B=N, T=1, H, .]
        o_ref, f_ref = oracle.recurrent(q[:, None], k[:, None], d.v[s][:, None], d.log_alpha[s][:, None],
                                        d.beta[s][:, None], init_state=S_ref, qk_l2norm=True)
        S_ref = f_ref
        rms = float(np.sqrt((o_ref ** 2).mean()))
        e = max(float(np.abs(o.cpu().numpy() - o_ref[:, 0]).max()),
                float(np.abs(state.cpu().numpy() - S_ref).max())) / rms
        worst = max(worst, e)
    log(f"[decode l2norm {dt}] worst {worst:.2e}")
    assert worst <= TOL[dt]
