"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle,
element by element, on seeded inputs.  Small cases span several 16-row tiles,
several chunks and a ragged last chunk; the five benchmark workloads are
checked at full size on every head and sequence (the oracle runs the chains on
all host cores in seconds); decode follows every state at step 0 and a sample
of states over 1000 steps."""
import numpy as np
import pytest
import torch

import workloads as W

from .gpu_util import TOL, check_parity, dev, log, run_chunk

pytestmark = pytest.mark.gpu


# ---- decode ----------------------------------------------------------------------

def _decode_case(N, H, dk, dv, in_dtype, seed, steps=3, out_dtype=torch.float32, tol=None):
    import gated_delta_rule_24_amd as gdn
    import oracle
    d = W.decode_inputs(N, H, dk, dv, pool=steps, in_dtype=in_dtype, seed=seed)
    dt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[in_dtype]
    state = dev(d.state)
    S_ref = d.state.astype(np.float64)
    worst = 0.0
    for s in range(steps):
        o = gdn.decode_step(state, dev(d.q[s], dt), dev(d.k[s], dt), dev(d.v[s], dt), dev(d.log_alpha[s]),
                            dev(d.beta[s]), out_dtype=out_dtype)
        torch.cuda.synchronize()
        # each resident state is its own length-1 sequence: [N, 1, H, d]
        o_ref, S_ref = oracle.recurrent(d.q[s][:, None], d.k[s][:, None], d.v[s][:, None],
                                        d.log_alpha[s][:, None], d.beta[s][:, None], init_state=S_ref)
        o_ref = o_ref[:, 0]
        rms = float(np.sqrt((o_ref ** 2).mean()))
        e_o = float(np.abs(o.float().cpu().numpy() - o_ref).max() / rms)
        e_S = float(np.abs(state.cpu().numpy() - S_ref).max() / rms)
        worst = max(worst, e_o, e_S)
        S_ref = state.cpu().numpy().astype(np.float64)   # continue each step from the GPU state
    tol = TOL[in_dtype] if tol is None else tol
    log(f"[decode] N={N} H={H} dk={dk} dv={dv} {in_dtype}: worst {worst:.3e} (tol {tol:.0e})")
    assert worst <= tol


@pytest.mark.parametrize("N,H,dk,dv,dt", [
    (3, 2, 128, 128, "fp32"), (5, 3, 128, 128, "bf16"), (2, 2, 64, 48, "fp16"), (4, 1, 32, 100, "bf16"),
    (2, 2, 256, 64, "fp32"), (1, 1, 32, 1, "fp32"),
])
def test_decode_small(N, H, dk, dv, dt):
    _decode_case(N, H, dk, dv, dt, seed=100 + N + dk)


# ---- chunked, small ------------------------------------------------------------------

SMALL = [
    # B, T, H, dk, dv, dtype, init_std
    (1, 256, 1, 32, 32, "fp32", None),
    (2, 200, 3, 128, 128, "bf16", None),
    (1, 130, 2, 64, 32, "fp16", 0.1),
    (1, 77, 1, 32, 64, "fp32", 0.1),
    (2, 95, 2, 256, 64, "bf16", 0.1),
    (1, 64, 2, 128, 256, "bf16", 0.1),
    (3, 1, 2, 128, 128, "bf16", 0.1),
    (1, 300, 1, 128, 128, "fp32", 0.1),
    (2, 200, 2, 128, 16, "bf16", 0.1),     # one 16-column value tile per head
    (1, 130, 3, 64, 16, "fp32", None),
    (1, 150, 2, 128, 512, "bf16", 0.1),    # dv above 256
    (1, 100, 1, 64, 1024, "fp16", None),   # the largest dv
    (1, 190, 2, 32, 320, "fp32", 0.1),
]


@pytest.mark.parametrize("B,T,H,dk,dv,dt,init_std", SMALL, ids=lambda x: str(x))
def test_chunk_small(B, T, H, dk, dv, dt, init_std):
    inp = W.chunk_inputs(B, T, H, dk, dv, dt, seed=T + dk + dv, init_std=init_std,
                         name=f"small B{B} T{T} H{H} dk{dk} dv{dv} {dt}")
    o, S = run_chunk(inp)
    check_parity(inp, o, S)


def test_chunk_packed_small():
    lens = [5, 0, 64, 1, 130, 63, 65, 200]
    inp = W.packed_inputs(lens, H=2, dk=128, dv=128, in_dtype="bf16", seed=7, name="packed-small")
    o, S = run_chunk(inp)
    check_parity(inp, o, S)


def test_chunk_packed_small_fp32():
    lens = [33, 1, 129, 0, 64]
    inp = W.packed_inputs(lens, H=3, dk=64, dv=80, in_dtype="fp32", seed=8, name="packed-small-fp32")
    o, S = run_chunk(inp)
    check_parity(inp, o, S)


def test_chunk_extreme_gates():
    # log alpha = -60 (memory cleared every token) and log alpha = 0 (pure delta rule)
    for la_val in (-60.0, 0.0):
        inp = W.chunk_inputs(1, 150, 2, 128, 128, "bf16", seed=9, init_std=0.1, name=f"gates la={la_val}")
        inp.log_alpha[:] = la_val
        o, S = run_chunk(inp)
        check_parity(inp, o, S)


# ---- the five workloads at full size (sampled) -------------------------------------------

def test_workload_tiny():
    inp = W.tiny()
    o, S = run_chunk(inp)
    check_parity(inp, o, S)


def test_workload_prefill():
    inp = W.prefill()
    log("[prefill] inputs ready")
    o, S = run_chunk(inp)
    check_parity(inp, o, S)


def test_workload_long():
    inp = W.long_context()
    log("[long] inputs ready")
    o, S = run_chunk(inp)
    check_parity(inp, o, S)


def test_workload_packed():
    inp = W.packed()
    log(f"[packed] lengths {np.diff(inp.cu_seqlens).tolist()}")
    o, S = run_chunk(inp)
    check_parity(inp, o, S)


def test_workload_continuation():
    """Continuation at serving shape: 256 resident state sets x 16 heads take
    2..16 tokens each in one packed call, final states written over the
    initial ones; every fifth sequence (all heads) against the oracle."""
    import gated_delta_rule_24_amd as gdn
    inp = W.continuation()
    lens = np.diff(inp.cu_seqlens)
    log(f"[continuation] {len(lens)} sequences, {int(lens.sum())} tokens, lengths {lens.min()}..{lens.max()}")
    q, k, v = (dev(x, torch.bfloat16) for x in (inp.q, inp.k, inp.v))
    la, b = dev(inp.log_alpha), dev(inp.beta)
    S = dev(inp.init_state)
    o, S_out = gdn.chunk_fwd(q, k, v, la, b, init_state=S, cu_seqlens=dev(inp.cu_seqlens, torch.int32), final_state=S)
    torch.cuda.synchronize()
    assert S_out.data_ptr() == S.data_ptr()
    check_parity(inp, o, S, seqs=range(0, len(lens), 5))


def test_workload_decode():
    """The 256 x 16 decode workload: 1000 in-place steps on the GPU.  Step 0 is
    compared on every (sequence, head) state; the oracle then follows a sample
    of states and is compared at steps 1, 63, 64 and 999."""
    import gated_delta_rule_24_amd as gdn
    import oracle
    d = W.decode()
    state = dev(d.state)
    pool = [(dev(d.q[p], torch.bfloat16), dev(d.k[p], torch.bfloat16), dev(d.v[p], torch.bfloat16),
             dev(d.log_alpha[p]), dev(d.beta[p])) for p in range(d.pool)]
    sample_n, sample_h = [0, 77, 255], [0, 15]
    # step 0 on every (sequence, head) state
    o = gdn.decode_step(state, *pool[0])
    torch.cuda.synchronize()
    o_ref, S_all = oracle.recurrent(d.q[0][:, None], d.k[0][:, None], d.v[0][:, None],
                                    d.log_alpha[0][:, None], d.beta[0][:, None], init_state=d.state)
    rms = float(np.sqrt((o_ref ** 2).mean()))
    worst = max(float(np.abs(o.cpu().numpy() - o_ref[:, 0]).max()),
                float(np.abs(state.cpu().numpy() - S_all).max())) / rms
    log(f"[decode-1000] step 0, all {d.state.shape[0] * d.state.shape[1]} states: {worst:.3e}")
    S_ref = S_all[np.ix_(sample_n, sample_h)]
    del S_all
    checks = {1, 63, 64, 999}
    for s in range(1, 1000):
        p = s % d.pool
        o = gdn.decode_step(state, *pool[p])
        sl = np.ix_(sample_n, sample_h)
        o_ref, S_ref = oracle.recurrent(d.q[p][sl][:, None], d.k[p][sl][:, None], d.v[p][sl][:, None],
                                        d.log_alpha[p][sl][:, None], d.beta[p][sl][:, None],
                                        init_state=S_ref)
        if s in checks:
            torch.cuda.synchronize()
            og = o.cpu().numpy()[sl]
            Sg = state.cpu().numpy()[sl]
            rms = float(np.sqrt((o_ref[:, 0] ** 2).mean()))
            e = max(float(np.abs(og - o_ref[:, 0]).max()), float(np.abs(Sg - S_ref).max())) / rms
            worst = max(worst, e)
            log(f"[decode-1000] step {s}: {e:.3e}")
    assert worst <= TOL["bf16"]


def test_chunk_large_values():
    """v scaled by 3000 (|v| up to about 1.5e4, state entries up to about 1e4): inside the
    fp16-operand range the bf16 path keeps the same relative bound."""
    inp = W.chunk_inputs(2, 300, 2, 128, 128, "bf16", seed=31, init_std=None, name="large v")
    inp.v[:] = W.bf16_round(inp.v * 3000.0)
    o, S = run_chunk(inp)
    log(f"[large v] max |v| {np.abs(inp.v).max():.3e}, max |S| {float(S.abs().max()):.3e}")
    assert float(S.abs().max()) > 1e3
    check_parity(inp, o, S)
