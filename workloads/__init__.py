"""Seeded synthetic inputs for the gated delta rule core.

This module only draws numbers: Gaussian and uniform samples from numpy's
PCG64, per-token L2 normalisation of q and k (the token-mixing block of the
Gated DeltaNet paper normalises q and k upstream of the recurrence, section
3.4 "Gated Delta Networks and hybrid models"), a sigmoid to put the write
strength beta in (0, 1), and round-to-nearest-even casts to bf16.  It holds
none of the recurrence's arithmetic.  Both the HIP path's tests and the CPU
oracle consume exactly the arrays built here, so the two sides see the same
input bytes (the oracle widens them to fp64, which is exact).

Workloads (sizes follow the prefill/long/packed/decode shapes the core is
benchmarked on; the paper trains at 4K context and evaluates extrapolation to
20K tokens, and the pages' state-size arithmetic uses 16 heads of 128x128):

  tiny     B=1  H=1  L=256    dk=dv=32   fp32 everything, zero initial state
  prefill  B=4  H=16 L=4096   dk=dv=128  bf16 q,k,v, fp32 gates, zero state
  long     B=1  H=16 L=32768  dk=128 dv=256, heads 0..7 slow-forgetting
  packed   8 sequences, lengths iid U{512..8192}, H=16, dk=dv=128,
           N(0, 0.1^2) fp32 initial states, cu_seqlens offsets
  decode   N=256 H=16 dk=dv=128 resident fp32 states N(0, 0.1^2),
           a pool of 64 single-token step inputs
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

CHUNK = 64

# Draw distributions shared by every workload.
LOG_ALPHA_RANGE = (-0.1, -0.001)
SLOW_LOG_ALPHA_RANGE = (-0.01, -0.0001)
INIT_STATE_STD = 0.1


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32
    arrays whose values are exactly representable in bf16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # Finite inputs only: adding 0x7FFF plus the kept lsb carries into the
    # exponent exactly when rounding up crosses a binade, as it should.
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + (np.uint32(0x7FFF) + lsb)) & np.uint32(0xFFFF0000)
    return r.view(np.float32).reshape(x.shape)


def fp16_round(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


def l2_normalise(x: np.ndarray) -> np.ndarray:
    """Per-token L2 normalisation over the last axis (done in fp64)."""
    x64 = x.astype(np.float64)
    n = np.sqrt((x64 * x64).sum(axis=-1, keepdims=True))
    return (x64 / n).astype(np.float32)


def sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def cast(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_round(x)
    if dtype == "fp16":
        return fp16_round(x)
    raise ValueError(f"unknown dtype {dtype}")


@dataclasses.dataclass
class ChunkInputs:
    """Inputs of one chunked (prefill) call.

    q, k: [B, T, H, dk]; v: [B, T, H, dv] fp32 arrays holding values exactly
    representable in `in_dtype`.  log_alpha, beta: [B, T, H] fp32.
    init_state: [N, H, dv, dk] fp32 or None (zeros).  cu_seqlens: int32 [N+1]
    for a packed batch (then B == 1), else None and N == B.
    """
    name: str
    in_dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    log_alpha: np.ndarray
    beta: np.ndarray
    init_state: Optional[np.ndarray]
    cu_seqlens: Optional[np.ndarray]
    seed: int

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def T(self):
        return self.q.shape[1]

    @property
    def H(self):
        return self.q.shape[2]

    @property
    def dk(self):
        return self.q.shape[3]

    @property
    def dv(self):
        return self.v.shape[3]

    @property
    def num_seqs(self):
        return self.B if self.cu_seqlens is None else len(self.cu_seqlens) - 1

    def seq_bounds(self):
        """(batch row, start, end) per sequence, token indices along T."""
        if self.cu_seqlens is None:
            return [(b, 0, self.T) for b in range(self.B)]
        cu = self.cu_seqlens
        return [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]


def chunk_inputs(B, T, H, dk, dv, in_dtype="bf16", seed=0, *, lengths=None,
                 init_std=None, log_alpha_range=LOG_ALPHA_RANGE,
                 slow_heads=0, name="custom", rng=None) -> ChunkInputs:
    """Draw one chunked-call input set.

    Draw order (fixed): lengths (if packed, drawn by the caller), q, k, v,
    log_alpha, the beta pre-activation, initial states.  With `lengths` the
    batch is packed: B must be 1 and T == sum(lengths).  `slow_heads` heads
    (the first ones) draw log_alpha from the slow-forgetting range.
    """
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    if lengths is not None:
        assert B == 1 and T == int(np.sum(lengths))
    q = l2_normalise(rng.standard_normal((B, T, H, dk), dtype=np.float32))
    k = l2_normalise(rng.standard_normal((B, T, H, dk), dtype=np.float32))
    v = rng.standard_normal((B, T, H, dv), dtype=np.float32)
    la = rng.uniform(*log_alpha_range, size=(B, T, H)).astype(np.float32)
    if slow_heads:
        la[:, :, :slow_heads] = rng.uniform(
            *SLOW_LOG_ALPHA_RANGE, size=(B, T, slow_heads)).astype(np.float32)
    beta = sigmoid(rng.standard_normal((B, T, H), dtype=np.float32))
    cu = None
    N = B
    if lengths is not None:
        cu = np.zeros(len(lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        N = len(lengths)
    init = None
    if init_std is not None:
        init = (init_std * rng.standard_normal((N, H, dv, dk), dtype=np.float32)).astype(np.float32)
    return ChunkInputs(name=name, in_dtype=in_dtype, q=cast(q, in_dtype), k=cast(k, in_dtype),
                       v=cast(v, in_dtype), log_alpha=la, beta=beta, init_state=init,
                       cu_seqlens=cu, seed=seed)


def incoming_grads(inp: ChunkInputs, seed: int, final: bool = True):
    """Seeded gradients of a loss with respect to o ([B,T,H,dv]) and to the
    final state ([N,H,dv,dk], or None), standard normal fp32, for the
    backward pass."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B, T, H, _ = inp.q.shape
    dv, dk = inp.v.shape[-1], inp.q.shape[-1]
    d_o = rng.standard_normal((B, T, H, dv), dtype=np.float32)
    N = B if inp.cu_seqlens is None else len(inp.cu_seqlens) - 1
    d_final = rng.standard_normal((N, H, dv, dk), dtype=np.float32) if final else None
    return d_o, d_final


def packed_lengths(n, lo, hi, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(lo, hi, size=n, endpoint=True).astype(np.int64)


def packed_inputs(lengths, H, dk, dv, in_dtype="bf16", seed=0, init_std=INIT_STATE_STD,
                  name="packed-custom") -> ChunkInputs:
    lengths = [int(x) for x in lengths]
    return chunk_inputs(1, int(sum(lengths)), H, dk, dv, in_dtype, seed, lengths=lengths,
                        init_std=init_std, name=name)


# --- the five benchmark workloads -------------------------------------------

def tiny():
    return chunk_inputs(1, 256, 1, 32, 32, "fp32", seed=1, name="tiny")


def prefill():
    return chunk_inputs(4, 4096, 16, 128, 128, "bf16", seed=2, name="prefill")


def long_context():
    return chunk_inputs(1, 32768, 16, 128, 256, "bf16", seed=3, slow_heads=8, name="long")


def packed():
    # The eight lengths are the first draws of the workload's generator.
    rng = np.random.Generator(np.random.PCG64(4))
    lengths = rng.integers(512, 8192, size=8, endpoint=True)
    return chunk_inputs(1, int(lengths.sum()), 16, 128, 128, "bf16", seed=4,
                        lengths=[int(x) for x in lengths], init_std=INIT_STATE_STD,
                        name="packed", rng=rng)


def continuation():
    """Serving-shape continuation: 256 resident (sequence, head) state sets each
    take 2..16 new tokens in one packed chunked call, the final states written
    over the initial ones.  The lengths are the first draws of the generator."""
    rng = np.random.Generator(np.random.PCG64(6))
    lengths = rng.integers(2, 16, size=256, endpoint=True)
    return chunk_inputs(1, int(lengths.sum()), 16, 128, 128, "bf16", seed=6,
                        lengths=[int(x) for x in lengths], init_std=INIT_STATE_STD,
                        name="continuation", rng=rng)


@dataclasses.dataclass
class DecodeInputs:
    """Resident states plus a pool of single-token step inputs.

    state: [N, H, dv, dk] fp32.  Pool arrays: q, k [P, N, H, dk], v [P, N, H, dv]
    (values representable in in_dtype), log_alpha, beta [P, N, H] fp32.
    Step s uses pool entry s mod P.
    """
    name: str
    in_dtype: str
    state: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    log_alpha: np.ndarray
    beta: np.ndarray
    seed: int

    @property
    def pool(self):
        return self.q.shape[0]


def decode_inputs(N, H, dk, dv, pool=64, in_dtype="bf16", seed=5, name="decode-custom"):
    rng = np.random.Generator(np.random.PCG64(seed))
    state = (INIT_STATE_STD * rng.standard_normal((N, H, dv, dk), dtype=np.float32)).astype(np.float32)
    q = l2_normalise(rng.standard_normal((pool, N, H, dk), dtype=np.float32))
    k = l2_normalise(rng.standard_normal((pool, N, H, dk), dtype=np.float32))
    v = rng.standard_normal((pool, N, H, dv), dtype=np.float32)
    la = rng.uniform(*LOG_ALPHA_RANGE, size=(pool, N, H)).astype(np.float32)
    beta = sigmoid(rng.standard_normal((pool, N, H), dtype=np.float32))
    return DecodeInputs(name=name, in_dtype=in_dtype, state=state, q=cast(q, in_dtype),
                        k=cast(k, in_dtype), v=cast(v, in_dtype), log_alpha=la, beta=beta,
                        seed=seed)


def decode():
    return decode_inputs(256, 16, 128, 128, pool=64, in_dtype="bf16", seed=5, name="decode")


WORKLOADS = {
    "tiny": tiny,
    "prefill": prefill,
    "long": long_context,
    "packed": packed,
    "decode": decode,
    "continuation": continuation,
}
