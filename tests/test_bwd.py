"""GPU parity of the backward pass (gdn_chunk_bwd through the C ABI) against
the fp64 oracle's gradients (oracle.recurrent_bwd), element by element.

Every gradient is computed in fp32 on the GPU for any input dtype, and the
oracle gets the same input values, so the bound is the fp32 one for all
cases: max |err| <= 1e-4 * RMS of the oracle's gradient, per gradient
tensor."""
import numpy as np
import pytest
import torch

import gated_delta_rule_24_amd as gdn
import oracle
import workloads as W

from .gpu_util import TORCH_DT, dev, log, rescale_qk

pytestmark = pytest.mark.gpu
GRAD_TOL = 1e-4
NAMES = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "d_init")


def _run(inp, d_o, d_final, qk_l2norm=False):
    dt = TORCH_DT[inp.in_dtype]
    q, k, v = dev(inp.q, dt), dev(inp.k, dt), dev(inp.v, dt)
    la, b = dev(inp.log_alpha), dev(inp.beta)
    S0 = None if inp.init_state is None else dev(inp.init_state)
    cu = None if inp.cu_seqlens is None else dev(inp.cu_seqlens, torch.int32)
    out = gdn.chunk_bwd(q, k, v, la, b, dev(d_o), init_state=S0, d_final=None if d_final is None else dev(d_final),
                        cu_seqlens=cu, qk_l2norm=qk_l2norm)
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in out]


def _check(inp, d_o, d_final, label, heads=None, tol=GRAD_TOL, qk_l2norm=False):
    got = _run(inp, d_o, d_final, qk_l2norm)
    H = inp.H
    heads = list(range(H)) if heads is None else list(heads)
    sl = (slice(None), slice(None), heads)
    init = None if inp.init_state is None else inp.init_state[:, heads]
    ref = oracle.recurrent_bwd(inp.q[sl], inp.k[sl], inp.v[sl], inp.log_alpha[sl], inp.beta[sl], d_o[sl],
                               init_state=init, d_final=None if d_final is None else d_final[:, heads],
                               cu_seqlens=inp.cu_seqlens, qk_l2norm=qk_l2norm)
    errs = []
    for name, g, r in zip(NAMES, got, ref):
        g = g[:, heads] if name == "d_init" else g[:, :, heads]
        rms = float(np.sqrt((r ** 2).mean())) if r.size else 1.0
        rms = rms if rms > 0 else 1.0
        assert np.isfinite(g).all(), f"{label}: {name} not finite"
        e = float(np.abs(g - r).max()) / rms if r.size else 0.0
        errs.append(e)
    log(f"[bwd] {label}: " + " ".join(f"{n} {e:.2e}" for n, e in zip(NAMES, errs)) + f" (tol {tol:.0e})")
    for n, e in zip(NAMES, errs):
        assert e <= tol, f"{label}: {n} error {e:.3e} > {tol:.0e}"


CASES = [
    # B, T, H, dk, dv, dtype, init_std, d_final
    (1, 130, 2, 64, 32, "fp32", 0.1, True),
    (2, 64, 1, 32, 16, "bf16", None, False),
    (1, 10, 2, 128, 128, "fp32", 0.1, True),
    (2, 200, 2, 128, 128, "bf16", 0.1, True),
    (1, 100, 1, 128, 256, "fp16", 0.1, True),
    (1, 257, 3, 32, 48, "fp32", None, True),
    (1, 190, 2, 64, 48, "bf16", 0.1, True),   # an odd count of 16-column value blocks above one
]


@pytest.mark.parametrize("B,T,H,dk,dv,dt,init_std,dfin", CASES, ids=lambda x: str(x))
def test_bwd_small(B, T, H, dk, dv, dt, init_std, dfin):
    inp = W.chunk_inputs(B, T, H, dk, dv, dt, seed=60 + T + dk, init_std=init_std)
    d_o, d_final = W.incoming_grads(inp, seed=61 + T, final=dfin)
    _check(inp, d_o, d_final, f"B{B} T{T} H{H} dk{dk} dv{dv} {dt}")


@pytest.mark.parametrize("B,T,H,dk,dv,dt,seed", [
    (2, 150, 2, 128, 128, "bf16", 64),
    (1, 130, 2, 64, 48, "fp32", 65),
    (1, 77, 3, 32, 32, "fp16", 66),
])
def test_bwd_l2norm(B, T, H, dk, dv, dt, seed):
    """GDN_QK_L2NORM differentiated: q and k of per-token lengths in [0.3, 3]
    against the oracle's gradients through the normalisation."""
    inp = rescale_qk(W.chunk_inputs(B, T, H, dk, dv, dt, seed=seed, init_std=0.1), seed)
    d_o, d_final = W.incoming_grads(inp, seed=seed + 1)
    _check(inp, d_o, d_final, f"l2norm B{B} T{T} H{H} dk{dk} dv{dv} {dt}", qk_l2norm=True)


def test_bwd_l2norm_packed_with_zero_vectors():
    """Packed batch with all-zero q and k at some tokens: their gradients are
    zero, the rest match the oracle."""
    inp = W.packed_inputs([5, 0, 70, 129, 64], H=2, dk=128, dv=128, in_dtype="bf16", seed=67)
    inp = rescale_qk(inp, 67, zero_tokens=(3, 80, 150))
    d_o, d_final = W.incoming_grads(inp, seed=68)
    _check(inp, d_o, d_final, "l2norm packed, zero vectors", qk_l2norm=True)
    dq, dk = _run(inp, d_o, d_final, qk_l2norm=True)[:2]
    for t in (3, 80, 150):
        assert np.abs(dq[:, t]).max() == 0.0 and np.abs(dk[:, t]).max() == 0.0


def test_bwd_packed():
    inp = W.packed_inputs([5, 0, 64, 1, 130, 63, 65], H=2, dk=128, dv=128, in_dtype="bf16", seed=62)
    d_o, d_final = W.incoming_grads(inp, seed=63)
    _check(inp, d_o, d_final, "packed [5,0,64,1,130,63,65]")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("gate", ["-60", "0", "beta2"])
def test_bwd_gates(gate, dtype):
    """Gate extremes; bf16 inputs take the kernels' split-bf16 products."""
    inp = W.chunk_inputs(1, 150, 2, 64, 64, dtype, seed=64, init_std=0.1)
    if gate == "beta2":
        inp.beta[:] = np.random.default_rng(64).uniform(0.0, 2.0, size=inp.beta.shape).astype(np.float32)
    else:
        inp.log_alpha[:] = float(gate)
    d_o, d_final = W.incoming_grads(inp, seed=65)
    _check(inp, d_o, d_final, f"gates {gate} {dtype}")


@pytest.mark.parametrize("gate", ["-60", "-5"])
def test_bwd_gates_d128_bf16(gate):
    """Strong decay at the benchmark head size: every split bf16 product (dk = dv = 128)
    with gamma down to e^-60 per token."""
    inp = W.chunk_inputs(1, 200, 2, 128, 128, "bf16", seed=70, init_std=0.1)
    inp.log_alpha[:] = float(gate)
    d_o, d_final = W.incoming_grads(inp, seed=71)
    _check(inp, d_o, d_final, f"gates {gate} d128 bf16")


def test_bwd_prefill_shape_sampled():
    """H=16, dk=dv=128, bf16, 1024 tokens per sequence (16 chunks), two
    heads checked against the oracle."""
    inp = W.chunk_inputs(2, 1024, 16, 128, 128, "bf16", seed=66)
    d_o, d_final = W.incoming_grads(inp, seed=67)
    _check(inp, d_o, d_final, "B2 T1024 H16 d128 bf16", heads=[0, 11])


def test_bwd_malformed_cu_reported():
    inp = W.packed_inputs([10, 20], H=1, dk=64, dv=32, in_dtype="fp32", seed=68)
    d_o, _ = W.incoming_grads(inp, seed=69, final=False)
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    la, b = dev(inp.log_alpha), dev(inp.beta)
    cu = torch.tensor([0, 25, 30], dtype=torch.int32, device="cuda")
    bad = torch.tensor([0, 31, 30], dtype=torch.int32, device="cuda")
    ws = torch.empty(1 << 24, dtype=torch.uint8, device="cuda")
    gdn.chunk_bwd(q, k, v, la, b, dev(d_o), cu_seqlens=cu, workspace=ws)
    assert gdn.chunk_fwd_check(ws) == 0
    dq, *_ = gdn.chunk_bwd(q, k, v, la, b, dev(d_o), cu_seqlens=bad, workspace=ws)
    assert gdn.chunk_fwd_check(ws) == 2


def test_bwd_empty_inputs():
    """No tokens: the initial state's gradient is the final state's gradient
    (the state passes through unchanged), and nothing else is written."""
    for lens in ([0, 0, 0], None):
        if lens is None:
            inp = W.chunk_inputs(2, 0, 2, 64, 32, "fp32", seed=70, init_std=0.1, name="bwd empty batch")
        else:
            inp = W.packed_inputs(lens, H=2, dk=64, dv=32, in_dtype="fp32", seed=71, name="bwd empty packed")
        d_o, d_final = W.incoming_grads(inp, seed=72)
        got = _run(inp, d_o, d_final)
        assert got[0].size == 0 and got[3].size == 0
        assert np.array_equal(got[5], d_final)


@pytest.mark.parametrize("dt,dk", [("bf16", 128), ("fp32", 64), ("fp16", 32)])
def test_bwd_deterministic(dt, dk):
    """Two calls on the same inputs give bit-identical gradients: every sum in
    the backward kernels has a fixed order (no atomics; the dbeta, dgamma and
    dkappa parts go to one slot per writer and are added in a fixed order)."""
    lens = [300, 0, 129, 64, 1]
    inp = W.packed_inputs(lens, H=4, dk=dk, dv=64, in_dtype=dt, seed=91, name=f"bwd twice {dt}")
    d_o, d_final = W.incoming_grads(inp, seed=92)
    first = _run(inp, d_o, d_final)
    second = _run(inp, d_o, d_final)
    for name, a, b in zip(NAMES, first, second):
        assert np.array_equal(a, b), f"{name} differs between two identical calls"
    log(f"[bwd] {inp.name}: six gradients bit-identical over two calls")
