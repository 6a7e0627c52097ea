"""GPU path tests through the C ABI: the single-step, chunked and
save-then-resume paths agree; packed batches equal separate runs (reset at
every boundary, no leak of NaN across sequences); results are deterministic;
in-place state continuation; device-side rejection of malformed cu_seqlens;
empty inputs; output dtypes; the extended write-strength range."""
import numpy as np
import pytest
import torch

import gated_delta_rule_24_amd as gdn
import oracle
import workloads as W

from .gpu_util import TOL, check_parity, dev, log, run_chunk

pytestmark = pytest.mark.gpu
BF = torch.bfloat16
SHORT_AVG = 16   # gdn.h: a call averaging at most this many tokens per sequence runs token-serially


def _dev_inputs(inp):
    dt = {"fp32": torch.float32, "bf16": BF, "fp16": torch.float16}[inp.in_dtype]
    return (dev(inp.q, dt), dev(inp.k, dt), dev(inp.v, dt), dev(inp.log_alpha), dev(inp.beta))


def _rms(x):
    return float(np.sqrt((np.asarray(x, np.float64) ** 2).mean()))


def test_resume_equals_uninterrupted():
    """Save-then-resume at split points that are and are not chunk multiples."""
    inp = W.chunk_inputs(1, 300, 3, 128, 128, "bf16", seed=31, init_std=0.1)
    q, k, v, la, b = _dev_inputs(inp)
    S0 = dev(inp.init_state)
    o_full, S_full = gdn.chunk_fwd(q, k, v, la, b, init_state=S0)
    o_ref, S_ref = oracle.recurrent(inp.q, inp.k, inp.v, inp.log_alpha, inp.beta, init_state=inp.init_state)
    rms = _rms(o_ref)
    for split in (1, 37, 64, 100, 128, 299):
        o1, S1 = gdn.chunk_fwd(q[:, :split].contiguous(), k[:, :split].contiguous(), v[:, :split].contiguous(),
                               la[:, :split].contiguous(), b[:, :split].contiguous(), init_state=S0)
        o2, S2 = gdn.chunk_fwd(q[:, split:].contiguous(), k[:, split:].contiguous(), v[:, split:].contiguous(),
                               la[:, split:].contiguous(), b[:, split:].contiguous(), init_state=S1)
        o = torch.cat([o1, o2], dim=1)
        torch.cuda.synchronize()
        e_o = float((o - o_full).abs().max()) / rms
        e_S = float((S2 - S_full).abs().max()) / rms
        e_ref = float(np.abs(o.cpu().numpy() - o_ref).max()) / rms
        log(f"[resume] split {split}: vs uninterrupted o {e_o:.2e} S {e_S:.2e}; vs oracle {e_ref:.2e}")
        assert e_o <= TOL["bf16"] and e_S <= TOL["bf16"] and e_ref <= TOL["bf16"]


def test_decode_continues_chunked_state():
    """Each decode step agrees with the chunked path continued from the same
    state: K single-token decode steps vs one K-token chunked call."""
    Ktok = 20
    inp = W.chunk_inputs(4, Ktok, 2, 128, 128, "bf16", seed=32, init_std=0.1)
    q, k, v, la, b = _dev_inputs(inp)
    S0 = dev(inp.init_state)
    o_chunk, S_chunk = gdn.chunk_fwd(q, k, v, la, b, init_state=S0)
    state = S0.clone()
    outs = []
    for t in range(Ktok):
        outs.append(gdn.decode_step(state, q[:, t].contiguous(), k[:, t].contiguous(), v[:, t].contiguous(),
                                    la[:, t].contiguous(), b[:, t].contiguous()))
    o_dec = torch.stack(outs, dim=1)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.recurrent(inp.q, inp.k, inp.v, inp.log_alpha, inp.beta, init_state=inp.init_state)
    rms = _rms(o_ref)
    e1 = float((o_dec - o_chunk).abs().max()) / rms
    e2 = float((state - S_chunk).abs().max()) / rms
    e3 = float(np.abs(o_dec.cpu().numpy() - o_ref).max()) / rms
    log(f"[decode vs chunk] o {e1:.2e} S {e2:.2e}; decode vs oracle {e3:.2e}")
    assert max(e1, e2, e3) <= TOL["bf16"]


@pytest.mark.parametrize("Ktok", [2, 16])
def test_continuation_equals_decode_steps(Ktok):
    """Serving shape (256 resident states x 16 heads): appending Ktok tokens to
    every state with one packed chunked call, states updated in place, agrees
    with Ktok single-token decode steps on a copy of the same states."""
    N, H = 256, 16
    inp = W.packed_inputs([Ktok] * N, H=H, dk=128, dv=128, in_dtype="bf16", seed=40 + Ktok)
    q, k, v, la, b = _dev_inputs(inp)
    cu = dev(inp.cu_seqlens, torch.int32)
    S_chunk = dev(inp.init_state)
    o_chunk, _ = gdn.chunk_fwd(q, k, v, la, b, init_state=S_chunk, cu_seqlens=cu, final_state=S_chunk)
    state = dev(inp.init_state)
    tok = lambda x, t: x[0].reshape(N, Ktok, *x.shape[2:])[:, t].contiguous()
    outs = [gdn.decode_step(state, tok(q, t), tok(k, t), tok(v, t), tok(la, t), tok(b, t)) for t in range(Ktok)]
    o_dec = torch.stack(outs, dim=1).reshape(1, N * Ktok, H, 128)
    torch.cuda.synchronize()
    rms = float(o_chunk.float().pow(2).mean().sqrt())
    e_o = float((o_dec - o_chunk).abs().max()) / rms
    e_s = float((state - S_chunk).abs().max()) / rms
    log(f"[continuation K={Ktok}] chunk vs {Ktok} decode steps: o {e_o:.2e} S {e_s:.2e} (rms {rms:.3f})")
    assert max(e_o, e_s) <= TOL["bf16"]


def test_packed_equals_separate_bitwise():
    lens = [70, 1, 0, 129, 64, 33]
    inp = W.packed_inputs(lens, H=2, dk=128, dv=128, in_dtype="bf16", seed=33)
    o_p, S_p = run_chunk(inp)
    q, k, v, la, b = _dev_inputs(inp)
    cu = inp.cu_seqlens
    for n in range(len(lens)):
        s, e = int(cu[n]), int(cu[n + 1])
        o_n, S_n = gdn.chunk_fwd(q[:, s:e].contiguous(), k[:, s:e].contiguous(), v[:, s:e].contiguous(),
                                 la[:, s:e].contiguous(), b[:, s:e].contiguous(),
                                 init_state=dev(inp.init_state[n:n + 1]))
        torch.cuda.synchronize()
        if e - s > SHORT_AVG:
            # both calls run the chunked kernels: the same arithmetic, bit for bit
            assert torch.equal(o_n, o_p[:, s:e]), f"sequence {n} output differs"
            assert torch.equal(S_n[0], S_p[n]), f"sequence {n} final state differs"
        else:
            # a lone short sequence runs token-serially: equal to the bound
            rms = max(float(o_p.float().pow(2).mean().sqrt()), 1e-6)
            err = max(float((o_n - o_p[:, s:e]).abs().max()) if e > s else 0.0,
                      float((S_n[0] - S_p[n]).abs().max())) / rms
            assert err <= TOL["bf16"], f"sequence {n}: {err:.3e}"


def test_deterministic():
    inp = W.chunk_inputs(2, 333, 3, 128, 128, "bf16", seed=34, init_std=0.1)
    o1, S1 = run_chunk(inp)
    o2, S2 = run_chunk(inp)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    d = W.decode_inputs(8, 4, 128, 128, pool=1, seed=35)
    st1, st2 = dev(d.state), dev(d.state)
    args = (dev(d.q[0], BF), dev(d.k[0], BF), dev(d.v[0], BF), dev(d.log_alpha[0]), dev(d.beta[0]))
    a1 = gdn.decode_step(st1, *args)
    a2 = gdn.decode_step(st2, *args)
    torch.cuda.synchronize()
    assert torch.equal(a1, a2) and torch.equal(st1, st2)


def test_nan_stays_in_its_sequence():
    lens = [90, 130, 40]
    inp = W.packed_inputs(lens, H=2, dk=128, dv=128, in_dtype="bf16", seed=36)
    o_clean, S_clean = run_chunk(inp)
    bad = W.packed_inputs(lens, H=2, dk=128, dv=128, in_dtype="bf16", seed=36)
    bad.v[0, int(bad.cu_seqlens[1]) + 5, 1, 3] = np.nan
    o_bad, S_bad = run_chunk(bad)
    cu = inp.cu_seqlens
    for n in (0, 2):
        s, e = int(cu[n]), int(cu[n + 1])
        assert torch.equal(o_bad[:, s:e], o_clean[:, s:e])
        assert torch.equal(S_bad[n], S_clean[n])
    assert torch.isnan(S_bad[1]).any()


def test_in_place_state_continuation():
    inp = W.packed_inputs([100, 17, 64], H=2, dk=128, dv=128, in_dtype="bf16", seed=37)
    q, k, v, la, b = _dev_inputs(inp)
    cu = dev(inp.cu_seqlens, torch.int32)
    S0 = dev(inp.init_state)
    o_a, S_a = gdn.chunk_fwd(q, k, v, la, b, init_state=S0, cu_seqlens=cu)
    S_inplace = S0.clone()
    o_b, S_b = gdn.chunk_fwd(q, k, v, la, b, init_state=S_inplace, cu_seqlens=cu, final_state=S_inplace)
    torch.cuda.synchronize()
    assert S_b.data_ptr() == S_inplace.data_ptr()
    assert torch.equal(o_a, o_b) and torch.equal(S_a, S_inplace)


@pytest.mark.parametrize("dt", ["bf16", "fp32"])   # checked by G6 itself / by the table pass before G5
@pytest.mark.parametrize("cu,code", [([0, 10, 5, 20], 2), ([1, 10, 20], 1), ([0, 10, 19], 3)])
def test_malformed_cu_seqlens_reported(cu, code, dt):
    T = 20
    inp = W.chunk_inputs(1, T, 2, 64, 32, dt, seed=38)
    q, k, v, la, b = _dev_inputs(inp)
    o = torch.full((1, T, 2, 32), 7.0, device="cuda")
    N = len(cu) - 1
    fin = torch.full((N, 2, 32, 64), 3.0, device="cuda")
    ws = torch.empty(gdn.chunk_fwd_workspace_size(1, T, 2, 64, 32, N, in_dtype=q.dtype), dtype=torch.uint8,
                     device="cuda")
    gdn.chunk_fwd(q, k, v, la, b, cu_seqlens=dev(np.array(cu), torch.int32), o=o, final_state=fin, workspace=ws)
    assert gdn.chunk_fwd_check(ws) == code
    assert bool((o == 7.0).all()) and bool((fin == 3.0).all())    # nothing written


def test_empty_inputs():
    S0 = torch.randn(2, 3, 32, 64, device="cuda")
    z = lambda *s, dt=BF: torch.zeros(*s, dtype=dt, device="cuda")
    o, S = gdn.chunk_fwd(z(2, 0, 3, 64), z(2, 0, 3, 64), z(2, 0, 3, 32), z(2, 0, 3, dt=torch.float32),
                         z(2, 0, 3, dt=torch.float32), init_state=S0)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 3, 32) and torch.equal(S, S0)
    # packed batch whose sequences are all empty
    o, S = gdn.chunk_fwd(z(1, 0, 3, 64), z(1, 0, 3, 64), z(1, 0, 3, 32), z(1, 0, 3, dt=torch.float32),
                         z(1, 0, 3, dt=torch.float32), init_state=S0,
                         cu_seqlens=torch.zeros(3, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(S, S0)
    # decode with N = 0 is a no-op
    st = torch.zeros(0, 2, 32, 32, device="cuda")
    o = gdn.decode_step(st, z(0, 2, 32), z(0, 2, 32), z(0, 2, 32), z(0, 2, dt=torch.float32), z(0, 2, dt=torch.float32))
    assert o.shape == (0, 2, 32)


@pytest.mark.parametrize("odt", [torch.bfloat16, torch.float16])
def test_output_dtypes(odt):
    """16-bit o is the fp32 result rounded once to the output type."""
    inp = W.chunk_inputs(1, 150, 2, 128, 64, "bf16", seed=39, init_std=0.1)
    o32, S32 = run_chunk(inp)
    o16, S16 = run_chunk(inp, out_dtype=odt)
    assert o16.dtype == odt
    assert torch.equal(o16, o32.to(odt))
    assert torch.equal(S16, S32)
    d = W.decode_inputs(4, 2, 128, 64, pool=1, seed=40)
    args = (dev(d.q[0], BF), dev(d.k[0], BF), dev(d.v[0], BF), dev(d.log_alpha[0]), dev(d.beta[0]))
    st_a, st_b = dev(d.state), dev(d.state)
    a = gdn.decode_step(st_a, *args)
    c = gdn.decode_step(st_b, *args, out_dtype=odt)
    torch.cuda.synchronize()
    assert torch.equal(c, a.to(odt))


def test_fp16_inputs():
    inp = W.chunk_inputs(2, 140, 2, 128, 128, "fp16", seed=41, init_std=0.1, name="fp16 inputs")
    o, S = run_chunk(inp)
    check_parity(inp, o, S)


def test_beta_extended_range():
    """Write strength beta in (0, 2) (negative eigenvalues of the transition,
    noted as an extension on the translated paper page): computed as given."""
    inp = W.chunk_inputs(2, 200, 2, 128, 128, "bf16", seed=42, init_std=0.1, name="beta in (0,2)")
    rng = np.random.default_rng(42)
    inp.beta[:] = rng.uniform(0.0, 2.0, size=inp.beta.shape).astype(np.float32)
    o, S = run_chunk(inp)
    check_parity(inp, o, S)
    d = W.decode_inputs(4, 2, 128, 128, pool=1, seed=43)
    d.beta[:] = rng.uniform(1.0, 2.0, size=d.beta.shape).astype(np.float32)
    st = dev(d.state)
    od = gdn.decode_step(st, dev(d.q[0], BF), dev(d.k[0], BF), dev(d.v[0], BF), dev(d.log_alpha[0]), dev(d.beta[0]))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.recurrent(d.q[0][:, None], d.k[0][:, None], d.v[0][:, None], d.log_alpha[0][:, None],
                                    d.beta[0][:, None], init_state=d.state)
    rms = _rms(o_ref)
    assert float(np.abs(od.cpu().numpy() - o_ref[:, 0]).max()) / rms <= TOL["bf16"]
    assert float(np.abs(st.cpu().numpy() - S_ref).max()) / rms <= TOL["bf16"]


# ---- token-serial path (calls averaging at most SHORT_AVG tokens per sequence) ----------

SHORT_CASES = [
    # lengths, H, dk, dv, dtype
    ([1, 16, 5, 0, 9, 2, 3, 7], 2, 128, 128, "fp32"),
    ([4, 4, 4, 4], 3, 32, 96, "fp32"),
    ([40, 0, 0, 1], 2, 64, 48, "bf16"),       # one sequence spans three 16-token batches
    ([3, 12, 1], 1, 256, 208, "fp16"),        # four row groups, the last one ragged
    ([2, 2], 2, 128, 16, "bf16"),
    ([16] * 5, 2, 256, 256, "bf16"),
]


@pytest.mark.parametrize("lens,H,dk,dv,dt", SHORT_CASES, ids=lambda x: str(x))
def test_short_path_parity(lens, H, dk, dv, dt):
    assert sum(lens) <= SHORT_AVG * len(lens)
    inp = W.packed_inputs(lens, H=H, dk=dk, dv=dv, in_dtype=dt, seed=50 + dk + dv, init_std=0.1,
                          name=f"short {lens} H{H} dk{dk} dv{dv} {dt}")
    o, S = run_chunk(inp)
    check_parity(inp, o, S)


def test_short_path_batched():
    """Equal-length batch (no cu_seqlens) of short sequences, with and without
    an initial state."""
    inp = W.chunk_inputs(6, 10, 2, 64, 64, "fp32", seed=57, init_std=0.1, name="short batched")
    o, S = run_chunk(inp)
    check_parity(inp, o, S)
    o0, S0 = run_chunk(inp, init_override=None)
    inp.init_state = None
    check_parity(inp, o0, S0, label="short batched, zero initial state")


@pytest.mark.parametrize("gate", ["-60", "-5", "0", "mixed", "beta2"])
def test_short_path_gates(gate):
    """Decay extremes on the token-serial path: log alpha = -60 or -5 drives
    the running decay scale out of its range every token or every few tokens,
    0 never decays; 'mixed' interleaves -60 with mild decay; 'beta2' takes
    beta in (0, 2)."""
    inp = W.packed_inputs([16, 9, 1, 14], H=2, dk=128, dv=128, in_dtype="fp32", seed=58, init_std=0.1,
                          name=f"short gates {gate}")
    if gate == "mixed":
        inp.log_alpha[:] = -0.5
        inp.log_alpha[:, ::3] = -60.0
    elif gate == "beta2":
        inp.beta[:] = np.random.default_rng(58).uniform(0.0, 2.0, size=inp.beta.shape).astype(np.float32)
    else:
        inp.log_alpha[:] = float(gate)
    o, S = run_chunk(inp)
    check_parity(inp, o, S)


def test_short_path_qk_l2norm():
    inp = W.packed_inputs([5, 11, 0, 16], H=2, dk=128, dv=64, in_dtype="bf16", seed=59, init_std=0.1,
                          name="short l2norm")
    inp.k[:, 3] = 0.0     # an all-zero key row stays zero after normalisation
    o, S = run_chunk(inp, qk_l2norm=True)
    check_parity(inp, o, S, qk_l2norm=True)


# ---- the same calls in 16-token chunks on the matrix cores (16-bit inputs, dk <= 128) ----
# GDN_SMALL_CHUNKS=0 sends them to the token-serial kernel instead: the two
# kernels agree with the oracle and with each other.

SMALL_CASES = [
    # lengths, H, dk, dv, in dtype, out dtype
    ([1, 16, 5, 0, 9, 2, 3, 7], 2, 128, 128, "bf16", "fp32"),
    ([17, 33, 1, 0], 2, 128, 256, "bf16", "bf16"),      # chunks 16 + 1 and 16 + 16 + 1
    ([4, 4, 4, 4], 3, 32, 96, "fp16", "fp16"),
    ([40, 0, 0, 1], 2, 64, 48, "fp16", "fp32"),
    ([2, 2], 2, 128, 16, "bf16", "fp32"),
    ([5, 12, 3, 0, 20], 2, 64, 320, "bf16", "fp32"),   # 20 value slices: two groups of waves
]
_OUT = {"fp32": torch.float32, "bf16": BF, "fp16": torch.float16}


def _small_vs_serial(inp, monkeypatch, label, **kw):
    o, S = run_chunk(inp, **kw)
    check_parity(inp, o, S, label=label, qk_l2norm=kw.get("qk_l2norm", False))
    monkeypatch.setenv("GDN_SMALL_CHUNKS", "0")
    o1, S1 = run_chunk(inp, **kw)
    monkeypatch.delenv("GDN_SMALL_CHUNKS")
    rms = max(float(o1.float().pow(2).mean().sqrt()), 1e-6)
    # a 16-bit o is rounded by each kernel on its own: one unit in the last
    # place of the largest |o| on top of the tolerance
    ulp = {BF: 2.0 ** -7, torch.float16: 2.0 ** -10}.get(o.dtype, 0.0) * float(o1.float().abs().max()) / rms
    e_o = float((o.float() - o1.float()).abs().max()) / rms
    e_s = float((S - S1).abs().max()) / rms if S is not None else 0.0
    log(f"[16-token chunks vs token-serial] {label}: o {e_o:.3e} (ulp {ulp:.1e}) S {e_s:.3e}")
    assert e_o <= TOL[inp.in_dtype] + ulp
    assert e_s <= TOL[inp.in_dtype]


@pytest.mark.parametrize("lens,H,dk,dv,dt,odt", SMALL_CASES, ids=lambda x: str(x))
def test_small_chunks_parity(lens, H, dk, dv, dt, odt, monkeypatch):
    assert sum(lens) <= SHORT_AVG * len(lens)
    inp = W.packed_inputs(lens, H=H, dk=dk, dv=dv, in_dtype=dt, seed=60 + dk + dv, init_std=0.1,
                          name=f"small chunks {lens} H{H} dk{dk} dv{dv} {dt}->{odt}")
    _small_vs_serial(inp, monkeypatch, inp.name, out_dtype=_OUT[odt])


@pytest.mark.parametrize("gate", ["-60", "-5", "0", "mixed", "beta2"])
def test_small_chunks_gates(gate, monkeypatch):
    """Decay extremes in 16-token chunks: every gate product inside a chunk is
    taken relative to the chunk, so -60 per token underflows to zero without
    overflowing anywhere; beta in (0, 2)."""
    inp = W.packed_inputs([16, 9, 1, 14, 31], H=2, dk=128, dv=128, in_dtype="bf16", seed=61, init_std=0.1,
                          name=f"small chunks gates {gate}")
    if gate == "mixed":
        inp.log_alpha[:] = -0.5
        inp.log_alpha[:, ::3] = -60.0
    elif gate == "beta2":
        inp.beta[:] = np.random.default_rng(61).uniform(0.0, 2.0, size=inp.beta.shape).astype(np.float32)
    else:
        inp.log_alpha[:] = float(gate)
    _small_vs_serial(inp, monkeypatch, inp.name)


def test_small_chunks_batched_no_state(monkeypatch):
    """Equal-length batch without cu_seqlens, zero initial state, final state
    not returned; then L2-normalised q and k on a packed batch."""
    inp = W.chunk_inputs(6, 10, 2, 64, 64, "bf16", seed=62, name="small chunks batched")
    inp.init_state = None
    _small_vs_serial(inp, monkeypatch, inp.name, init_override=None)
    o, S = run_chunk(inp, init_override=None, final=False)
    assert S is None
    o_ref, _ = run_chunk(inp, init_override=None)
    assert torch.equal(o, o_ref)
    inp = W.packed_inputs([5, 11, 0, 16, 20], H=2, dk=128, dv=64, in_dtype="fp16", seed=63, init_std=0.1,
                          name="small chunks l2norm")
    inp.k[:, 3] = 0.0
    _small_vs_serial(inp, monkeypatch, inp.name, qk_l2norm=True)


@pytest.mark.parametrize("dk", [32, 64])
def test_small_chunks_l2norm_narrow_keys(dk, monkeypatch):
    """q/k L2 normalisation in 16-token chunks when a key row spans 4 or 8
    staging lanes (the row sums take fewer lane exchanges than at dk = 128)."""
    inp = W.packed_inputs([7, 16, 3, 0, 21], H=3, dk=dk, dv=48, in_dtype="bf16", seed=64 + dk, init_std=0.1,
                          name=f"small chunks l2norm dk{dk}")
    inp.q[:] = inp.q * 2.0        # not unit rows (scaled exactly): the normalisation must act
    inp.k[:] = inp.k * 0.5
    inp.k[:, 5] = 0.0
    _small_vs_serial(inp, monkeypatch, inp.name, qk_l2norm=True)
