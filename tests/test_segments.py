"""GPU tests of the segmented state pass: each sequence's chunks cut into
segments, a transition pass per segment (the segment's affine map S -> S F + G
from a zero state and the identity), a combine pass that walks the maps to
each segment's incoming state, and the output pass per segment.  The split is
forced with GDN_SEG_CHUNKS (read by the library at every call, also by the
workspace-size query) down to one chunk per segment, so short inputs cross
many segment boundaries; every case is checked against the fp64 oracle, and
the segmented result against the unsegmented one of the same call."""
import numpy as np
import pytest
import torch

import gated_delta_rule_24_amd as gdn
import oracle
import workloads as W

from .gpu_util import TOL, check_parity, dev, log, run_chunk

pytestmark = pytest.mark.gpu


def _run(inp, seg, monkeypatch, **kw):
    monkeypatch.setenv("GDN_SEG_CHUNKS", str(seg))
    return run_chunk(inp, **kw)


CASES = [
    # B, T, H, dk, dv, dtype, init_std, seg
    (2, 500, 2, 128, 128, "bf16", 0.1, 2),
    (1, 640, 3, 128, 256, "bf16", None, 3),    # dv + dk = 384: transition tiles of value and F columns
    (1, 300, 2, 64, 48, "fp32", 0.1, 1),       # dv + dk = 112: a transition tile mixes both kinds
    (3, 200, 1, 32, 16, "fp32", 0.1, 1),
    (1, 450, 2, 256, 64, "fp16", 0.1, 2),
    (1, 129, 2, 128, 128, "bf16", 0.1, 1),     # a one-token last segment
    (2, 256, 2, 128, 128, "bf16", 0.1, 4),     # exactly one segment: the split is a no-op
]


@pytest.mark.parametrize("B,T,H,dk,dv,dt,init_std,seg", CASES, ids=lambda x: str(x))
def test_segmented_parity(B, T, H, dk, dv, dt, init_std, seg, monkeypatch):
    inp = W.chunk_inputs(B, T, H, dk, dv, dt, seed=T + dk + seg, init_std=init_std,
                         name=f"segmented B{B} T{T} H{H} dk{dk} dv{dv} {dt} seg{seg}")
    o, S = _run(inp, seg, monkeypatch)
    check_parity(inp, o, S)
    o0, S0 = _run(inp, 0, monkeypatch)
    rms = float(o0.float().pow(2).mean().sqrt())
    e = max(float((o - o0).abs().max()), float((S - S0).abs().max())) / rms
    log(f"[segmented vs whole] {inp.name}: {e:.3e}")
    assert e <= TOL[dt]


def test_segmented_packed(monkeypatch):
    """Packed batch with empty, one-token and partial-chunk sequences: segment
    units come from the device-side table."""
    lens = [5, 0, 64, 1, 130, 200, 333, 65]
    inp = W.packed_inputs(lens, H=2, dk=128, dv=128, in_dtype="bf16", seed=71, name="segmented packed")
    for seg in (1, 2):
        o, S = _run(inp, seg, monkeypatch)
        check_parity(inp, o, S, label=f"segmented packed seg{seg}")


def test_segmented_in_place(monkeypatch):
    """final_state == init_state: the output pass never reads the caller's
    initial state (the combine pass copies it), so the last segment's write
    cannot race with the first segment's read."""
    inp = W.chunk_inputs(2, 700, 2, 128, 128, "bf16", seed=72, init_std=0.1, name="segmented in place")
    monkeypatch.setenv("GDN_SEG_CHUNKS", "2")
    dt = torch.bfloat16
    S = dev(inp.init_state)
    o, S_out = gdn.chunk_fwd(dev(inp.q, dt), dev(inp.k, dt), dev(inp.v, dt), dev(inp.log_alpha), dev(inp.beta),
                             init_state=S, final_state=S)
    torch.cuda.synchronize()
    assert S_out.data_ptr() == S.data_ptr()
    check_parity(inp, o, S)


def test_segmented_gates(monkeypatch):
    """log alpha = -60 (the map F is 0), log alpha = 0 (no decay) and beta up to 2."""
    for name, la_val, beta_scale in (("la=-60", -60.0, 1.0), ("la=0", 0.0, 1.0), ("beta2", None, 2.0)):
        inp = W.chunk_inputs(1, 400, 2, 128, 128, "bf16", seed=73, init_std=0.1, name=f"segmented {name}")
        if la_val is not None:
            inp.log_alpha[:] = la_val
        inp.beta[:] = inp.beta * beta_scale
        o, S = _run(inp, 2, monkeypatch)
        check_parity(inp, o, S)


def test_segmented_malformed_cu(monkeypatch):
    """A malformed cu_seqlens leaves o and the final state untouched on the
    segmented path too, and is reported."""
    monkeypatch.setenv("GDN_SEG_CHUNKS", "1")
    inp = W.packed_inputs([100, 200], H=2, dk=128, dv=128, in_dtype="bf16", seed=74)
    dt = torch.bfloat16
    cu = dev(np.array([0, 250, 290], dtype=np.int32), torch.int32)   # does not end at T
    o = torch.full((1, 300, 2, 128), 7.0, device="cuda")
    fin = torch.full((2, 2, 128, 128), 5.0, device="cuda")
    ws = torch.empty(gdn.chunk_fwd_workspace_size(1, 300, 2, 128, 128, 2), dtype=torch.uint8,
                     device="cuda")
    gdn.chunk_fwd(dev(inp.q, dt), dev(inp.k, dt), dev(inp.v, dt), dev(inp.log_alpha), dev(inp.beta),
                  init_state=dev(inp.init_state), cu_seqlens=cu, o=o, final_state=fin, workspace=ws)
    torch.cuda.synchronize()
    assert gdn.chunk_fwd_check(ws) != 0
    assert bool((o == 7.0).all()) and bool((fin == 5.0).all())
