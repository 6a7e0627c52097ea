"""gdn_chunk_fwd_noalloc (the library's scratch array instead of a workspace)
against gdn_chunk_fwd on the same inputs, through the C ABI: calls in a
row, each smaller than the one before, so each runs on the scratch the
previous one left behind (the last a short call).  Both entry points share their kernels and are
deterministic, so the outputs must match bit for bit; each is also checked
against the fp64 oracle."""
import ctypes

import numpy as np
import pytest
import torch

import gated_delta_rule_24_amd as gdn
import workloads as W

from .gpu_util import check_parity, dev, log

pytestmark = pytest.mark.gpu


def _noalloc_call(inp, o, fin):
    """gdn_chunk_fwd_noalloc through ctypes, on preallocated outputs."""
    lib = gdn.load()
    dt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[inp.in_dtype]
    q, k, v = dev(inp.q, dt), dev(inp.k, dt), dev(inp.v, dt)
    la, b = dev(inp.log_alpha), dev(inp.beta)
    S0 = None if inp.init_state is None else dev(inp.init_state)
    cu = None if inp.cu_seqlens is None else dev(inp.cu_seqlens, torch.int32)
    N = inp.num_seqs
    d = gdn.ChunkDesc(inp.B, inp.T, inp.H, inp.dk, inp.dv, N, gdn.CHUNK, gdn._DT[dt], gdn._DT[o.dtype], 0)
    vp = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = lib.gdn_chunk_fwd_noalloc(ctypes.byref(d), vp(q), vp(k), vp(v), vp(la), vp(b), vp(S0), vp(cu), vp(o),
                                   vp(fin), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.gdn_last_error_message()
    torch.cuda.synchronize()
    return (q, k, v, la, b, S0, cu)


def _reference(args, inp, o_dtype):
    q, k, v, la, b, S0, cu = args
    o, S = gdn.chunk_fwd(q, k, v, la, b, init_state=S0, cu_seqlens=cu, out_dtype=o_dtype)
    torch.cuda.synchronize()
    return o, S


def test_noalloc_matches_workspace_call_twice():
    cases = [
        W.chunk_inputs(4, 1000, 8, 128, 128, "bf16", seed=81, init_std=0.1, name="noalloc first (larger)"),
        W.packed_inputs([70, 0, 129, 5], H=3, dk=64, dv=48, in_dtype="bf16", seed=82, name="noalloc second (smaller)"),
        # a short call (at most 16 tokens per sequence on average: the
        # 16-token-chunk kernel) on the scratch the two before left behind
        W.packed_inputs([5, 12, 0, 9], H=2, dk=128, dv=64, in_dtype="bf16", seed=83, name="noalloc third (short)"),
    ]
    ws_first = gdn.chunk_fwd_workspace_size(4, 1000, 8, 128, 128, 4)
    ws_second = gdn.chunk_fwd_workspace_size(1, 204, 3, 64, 48, 4)
    assert ws_second < ws_first <= gdn.NOALLOC_SCRATCH_BYTES
    for inp in cases:
        o = torch.empty((inp.B, inp.T, inp.H, inp.dv), dtype=torch.float32, device="cuda")
        fin = torch.empty((inp.num_seqs, inp.H, inp.dv, inp.dk), dtype=torch.float32, device="cuda")
        args = _noalloc_call(inp, o, fin)
        o_ref, S_ref = _reference(args, inp, torch.float32)
        same = bool(torch.equal(o, o_ref)) and bool(torch.equal(fin, S_ref))
        log(f"[noalloc] {inp.name}: bitwise equal to gdn_chunk_fwd: {same}")
        assert same
        check_parity(inp, o, fin)


def test_noalloc_rejects_oversized():
    inp_desc = gdn.ChunkDesc(8, 8192, 16, 128, 128, 8, gdn.CHUNK, 1, 0, 0)
    lib = gdn.load()
    x = torch.zeros(16, device="cuda")
    p = ctypes.c_void_p(x.data_ptr())
    st = lib.gdn_chunk_fwd_noalloc(ctypes.byref(inp_desc), p, p, p, p, p, None, None, p, None, None)
    assert st == 6
    log(f"[noalloc] oversized call: {lib.gdn_last_error_message().decode()}")
