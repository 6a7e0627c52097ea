"""Benchmark of the gated delta rule core on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
                    [--only prefill|long|packed|decode|continuation|backward|copy]

A step is one chunked prefill over the prefill workload (B=4, H=16, L=4096,
dk=dv=128, C=64, bf16 q/k/v, fp32 gates, fp32 o and states), inputs resident
in HBM.  `value` is prefill tokens/s (mean over K back-to-back steps after W
untimed ones; the median and minimum of K individually timed steps are
reported beside it).  The defaults, K = 50 and W = 400 (about 55 ms of
prefill), let the GPU reach its steady clock before the timed steps: after
the host has spent seconds drawing inputs, the first tens of milliseconds of
GPU work run slower.  The other legs warm up for W steps and at least 50 ms.
The same run times the long-context workload (B=1, H=16, L=32768, dk=128,
dv=256, half the heads slow-forgetting) under "long", the packed batch (eight
sequences of 512..8192 tokens with initial states) under "packed", 1000
in-place decode steps (256 sequences x 16 heads, 128x128 fp32 states) under
"decode", the continuation call (256 resident states take 2..16 tokens each)
under "continuation" and the backward pass over the prefill workload under
"backward".  Each kernel's average duration comes from HIP events the library
records around its launches on the launch stream; the roofline objects use
the algorithmic bytes and flops of the method (counted below) over that
duration.  The CPU baselines are the fp64 oracle on a bounded sample of each
chunked workload, on all host cores.

Prints ONE JSON line.  --only runs a single leg (for profiler runs) and
prints that leg's part of the line.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s (H=16,dk=dv=128,C=64) + decode steps/s; % MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak, TFLOP/s
C = 64


def chunk_flops_per_token_head(dk, dv, c=C):
    # W S^T, Q S^T and V'^T K (6 dk dv); K K^T, Q K^T, W, U and P V' (2C(3dk + 2dv)); the
    # triangular inverse (C^2/3).  Counted dense, as the chunked algorithm computes them.
    return 6 * dk * dv + 2 * c * (3 * dk + 2 * dv) + c * c / 3


def chunk_min_bytes(B, T, H, dk, dv, N, in_bytes, out_bytes, has_init, has_final):
    # q, k, v in; log_alpha and beta in; o out; initial and final states
    th = B * T * H
    b = th * (2 * dk + dv) * in_bytes + th * 2 * 4 + th * dv * out_bytes
    st = N * H * dv * dk * 4
    return b + (st if has_init else 0) + (st if has_final else 0)


MFMA_F32_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix peak, TFLOP/s


def bwd_grad_flops_per_chunk_head(dk, dv, c=C):
    # The gradient kernel's products, triangular ones at their triangular size (t = c(c+1)/2):
    # U = dO S, Z = dY S, W2 = V' dS_next (6 c dk dv); dP = dO V'^T, dM = dV' Y^T (2 * 2 t dv);
    # T^T dT and W T^T (about 2 c^3 / 3); K K^T, Q K^T (2 * 2 t dk); (dP o Gamma) K and
    # (dP o Gamma)^T Q (2 * 2 t dk); (dK o + dK o^T) K (2 c^2 dk).
    t = c * (c + 1) / 2
    return 6 * c * dk * dv + 4 * t * dv + 2 * c ** 3 / 3 + 8 * t * dk + 2 * c * c * dk


def decode_min_bytes(N, H, dk, dv, in_bytes, out_bytes):
    # the fp32 state read and written once, q, k, v and gates in, o out
    nh = N * H
    return nh * dv * dk * 4 * 2 + nh * (2 * dk + dv) * in_bytes + nh * 2 * 4 + nh * dv * out_bytes


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "gated_delta_rule_24_amd", "csrc")


def kernel_sources_digest(files):
    """sha256 over the sources a kernel is built from, to tie counter readings to a kernel version."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed FETCH_SIZE / WRITE_SIZE
    readings, each scaled by what the same counter reads for a copy of known size; None when the
    kernel's sources have changed since the counters were taken (or none were taken)."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except OSError:
        return None
    k = rec.get("kernels", {}).get(f"{kernel}@{workload}")
    if not k or k.get("workload") != workload or kernel_sources_digest(k["sources"]) != k["sources_sha256"]:
        return None
    cal = rec["copy_calibration"]
    return 1024.0 * (k["fetch_kib"] * cal["fetch_scale"] + k["write_kib"] * cal["write_scale"])


def measured_mfma_busy(kernel, workload):
    """Share of all matrix-core cycles `kernel` kept busy on `workload`, from the committed SQ counter
    readings: SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs).  None when the
    kernel's sources have changed since the counters were taken (or none were taken)."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except OSError:
        return None
    k = rec.get("sq", {}).get(f"{kernel}@{workload}")
    if not k or kernel_sources_digest(k["sources"]) != k["sources_sha256"]:
        return None
    return k["SQ_VALU_MFMA_BUSY_CYCLES"] / (k["GRBM_GUI_ACTIVE"] / 8 * 1024)


def _to(x, dev, dt):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev, dt)


def warm_up(step, warmup, min_ms=0.0):
    """`warmup` untimed steps, continued (for the legs after the headline one) until at least
    `min_ms` of device time has passed: after the host has spent seconds drawing a leg's inputs,
    the first tens of milliseconds of GPU work run slower (a long-context call: 0.59 ms per step
    averaged over 20 steps after 5 warm-up steps, 0.50 ms after 50)."""
    import torch
    for _ in range(warmup):
        step()
    if min_ms <= 0:
        return
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(10000):
        step()
        t1.record()
        t1.synchronize()
        if t0.elapsed_time(t1) >= min_ms:
            break


def time_steps(step, steps, warmup, min_warm_ms=0.0):
    """Mean step time over `steps` back-to-back steps bracketed by device synchronisation, then the
    median and minimum of the same number of individually timed steps (events on torch's current
    stream, the one every call here launches on)."""
    import statistics

    import torch
    warm_up(step, warmup, min_warm_ms)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    mean_ms = ev0.elapsed_time(ev1) / steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    each = [a.elapsed_time(b) for a, b in evs]
    return mean_ms, statistics.median(each), min(each)


CHUNK_WORKLOADS = {
    # name: (generator, has_init, description of the shape)
    "prefill": ("prefill", False),
    "long": ("long_context", False),
    "packed": ("packed", True),
}


def run_chunk_workload(args, gdn, W, dev, name, out_dtype="fp32"):
    """One gdn_chunk_fwd call over a whole workload (inputs resident in HBM), timed as in time_steps;
    per-kernel durations from the library's own events on the launch stream."""
    import torch
    gen, has_init = CHUNK_WORKLOADS[name]
    inp = getattr(W, gen)()
    B, T, H, dk, dv, N = inp.B, inp.T, inp.H, inp.dk, inp.dv, inp.num_seqs
    q, k, v = (_to(x, dev, torch.bfloat16) for x in (inp.q, inp.k, inp.v))
    la, be = _to(inp.log_alpha, dev, torch.float32), _to(inp.beta, dev, torch.float32)
    S0 = _to(inp.init_state, dev, torch.float32) if has_init else None
    cu = torch.from_numpy(inp.cu_seqlens).to(dev) if inp.cu_seqlens is not None else None
    odt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[out_dtype]
    o = torch.empty((B, T, H, dv), dtype=odt, device=dev)
    fin = torch.empty((N, H, dv, dk), dtype=torch.float32, device=dev)
    ws = torch.empty(gdn.chunk_fwd_workspace_size(B, T, H, dk, dv, N, out_dtype=odt), dtype=torch.uint8,
                     device=dev)

    def step():
        gdn.chunk_fwd(q, k, v, la, be, init_state=S0, cu_seqlens=cu, o=o, final_state=fin, workspace=ws,
                      out_dtype=odt)

    # the headline prefill leg takes exactly args.warmup warm-up steps; the other legs also warm
    # up for at least 50 ms of device time
    ms_per_step, ms_med, ms_min = time_steps(step, args.steps, args.warmup, 0.0 if name == "prefill" else 50.0)

    # per-kernel durations (events recorded by the library around each launch)
    with gdn.profile() as prof:
        for _ in range(args.steps):
            step()
    torch.cuda.synchronize()
    kernels = {kn: {"launches": n, "avg_us": 1e3 * ms / n} for kn, (n, ms) in prof.results.items()}

    flops = chunk_flops_per_token_head(dk, dv) * B * T * H
    min_bytes = chunk_min_bytes(B, T, H, dk, dv, N, 2, o.element_size(), has_init, True)
    dom = max(kernels, key=lambda n: kernels[n]["avg_us"] * kernels[n]["launches"])
    dom_s = kernels[dom]["avg_us"] * 1e-6
    path_s = ms_per_step * 1e-3
    roofline = {
        "kernel": dom,
        "bound": "hbm",
        "achieved": min_bytes / dom_s / 1e9,
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": min_bytes / dom_s / 1e9 / HBM_PEAK_GBS,
        "traffic": measured_traffic(dom, name),
        "algorithmic_bytes": min_bytes,
        "mfma_tflops": flops / dom_s / 1e12,
        "mfma_frac": flops / dom_s / 1e12 / MFMA_F16_PEAK_TFLOPS,
        "mfma_busy_counter": measured_mfma_busy(dom, name),
        "path_hbm_frac": min_bytes / path_s / 1e9 / HBM_PEAK_GBS,
        "path_mfma_frac": flops / path_s / 1e12 / MFMA_F16_PEAK_TFLOPS,
    }
    cfg = {"workload": name, "B": B, "L": T, "H": H, "dk": dk, "dv": dv, "chunk": C, "in_dtype": "bf16",
           "out_dtype": out_dtype, "init_state": "fp32" if has_init else None, "final_state": "fp32"}
    if inp.cu_seqlens is not None:
        cfg["lengths"] = [int(x) for x in (inp.cu_seqlens[1:] - inp.cu_seqlens[:-1])]
    res = {"value": B * T / path_s, "unit": "tokens/s", "ms_per_step": ms_per_step, "ms_median": ms_med,
           "ms_min": ms_min, "roofline": roofline, "kernels": kernels, "config": cfg}
    del q, k, v, la, be, S0, cu, o, fin, ws
    torch.cuda.empty_cache()
    return res, inp


def run_decode(args, gdn, W, dev):
    import torch
    d = W.decode()
    Nd, Hd, dv, dk = d.state.shape
    state = _to(d.state, dev, torch.float32)
    pool = [tuple(_to(x, dev, torch.bfloat16) for x in (d.q[p], d.k[p], d.v[p]))
            + (_to(d.log_alpha[p], dev, torch.float32), _to(d.beta[p], dev, torch.float32))
            for p in range(d.pool)]
    od = torch.empty((Nd, Hd, dv), dtype=torch.float32, device=dev)
    for s in range(10):
        gdn.decode_step(state, *pool[s % d.pool], o=od)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for s in range(args.decode_steps):
        gdn.decode_step(state, *pool[s % d.pool], o=od)
    ev1.record()
    torch.cuda.synchronize()
    dec_ms = ev0.elapsed_time(ev1) / args.decode_steps
    with gdn.profile() as dprof:
        for s in range(100):
            gdn.decode_step(state, *pool[s % d.pool], o=od)
    n_l, ms_l = dprof.results["gdn_decode_step"]
    dec_kernel_s = ms_l / n_l * 1e-3
    dbytes = decode_min_bytes(Nd, Hd, dk, dv, 2, 4)
    res = {
        "value": 1e3 / dec_ms, "unit": "steps/s", "ms_per_step": dec_ms, "steps": args.decode_steps,
        "config": {"workload": "decode", "N": int(Nd), "H": int(Hd), "dk": int(dk), "dv": int(dv),
                   "in_dtype": "bf16", "state": "fp32 in place"},
        "roofline": {"kernel": "gdn_decode_step", "bound": "hbm", "achieved": dbytes / dec_kernel_s / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dbytes / dec_kernel_s / 1e9 / HBM_PEAK_GBS,
                     "traffic": measured_traffic("gdn_decode_step", "decode"), "algorithmic_bytes": dbytes, "avg_us": dec_kernel_s * 1e6},
    }
    del state, pool, od
    torch.cuda.empty_cache()
    return res


def run_continuation(args, gdn, W, dev):
    """256 resident (sequence, head) state sets take 2..16 tokens each in one packed chunked call,
    final states written over the initial ones; repeated calls keep appending the same tokens."""
    import torch
    inp = W.continuation()
    T, H, dk, dv, N = inp.T, inp.H, inp.dk, inp.dv, inp.num_seqs
    q, k, v = (_to(x, dev, torch.bfloat16) for x in (inp.q, inp.k, inp.v))
    la, be = _to(inp.log_alpha, dev, torch.float32), _to(inp.beta, dev, torch.float32)
    cu = torch.from_numpy(inp.cu_seqlens).to(dev)
    state = _to(inp.init_state, dev, torch.float32)
    o = torch.empty((1, T, H, dv), dtype=torch.float32, device=dev)
    ws = torch.empty(gdn.chunk_fwd_workspace_size(1, T, H, dk, dv, N), dtype=torch.uint8, device=dev)

    def step():
        gdn.chunk_fwd(q, k, v, la, be, init_state=state, cu_seqlens=cu, o=o, final_state=state, workspace=ws)

    warm_up(step, args.warmup, 50.0)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    with gdn.profile() as prof:
        for _ in range(args.steps):
            step()
    torch.cuda.synchronize()
    kernels = {name: {"launches": n, "avg_us": 1e3 * t / n} for name, (n, t) in prof.results.items()}
    nbytes = chunk_min_bytes(1, T, H, dk, dv, N, 2, 4, True, True)
    dom = max(kernels, key=lambda n: kernels[n]["avg_us"] * kernels[n]["launches"])
    dom_s = kernels[dom]["avg_us"] * 1e-6
    lens = inp.cu_seqlens[1:] - inp.cu_seqlens[:-1]
    res = {
        "value": T / (ms * 1e-3), "unit": "tokens/s", "ms_per_call": ms, "calls": args.steps,
        "config": {"workload": "continuation", "N": int(N), "H": int(H), "dk": int(dk), "dv": int(dv),
                   "tokens": int(T), "lengths": f"{int(lens.min())}..{int(lens.max())}", "in_dtype": "bf16",
                   "out_dtype": "fp32", "state": "fp32, initial and final aliased in place"},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": nbytes / dom_s / 1e9, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": nbytes / dom_s / 1e9 / HBM_PEAK_GBS, "traffic": measured_traffic(dom, "continuation"),
                     "algorithmic_bytes": nbytes, "path_hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "kernels": kernels,
    }
    del q, k, v, la, be, cu, state, o, ws
    torch.cuda.empty_cache()
    return res


def run_backward(args, gdn, W, dev):
    """gdn_chunk_bwd on the prefill workload: gradients of o (fp32, standard normal) and of the final
    state flow back to q, k, v, log alpha, beta and the (zero) initial state."""
    import torch
    inp = W.prefill()
    B, T, H, dk, dv = inp.B, inp.T, inp.H, inp.dk, inp.dv
    q, k, v = (_to(x, dev, torch.bfloat16) for x in (inp.q, inp.k, inp.v))
    la, be = _to(inp.log_alpha, dev, torch.float32), _to(inp.beta, dev, torch.float32)
    d_o_np, d_fin_np = W.incoming_grads(inp, seed=12)
    d_o, d_fin = _to(d_o_np, dev, torch.float32), _to(d_fin_np, dev, torch.float32)
    del d_o_np, d_fin_np
    ws = torch.empty(gdn.chunk_bwd_workspace_size(B, T, H, dk, dv, B), dtype=torch.uint8, device=dev)

    def step():
        gdn.chunk_bwd(q, k, v, la, be, d_o, d_final=d_fin, workspace=ws)

    steps = max(1, args.steps // 2)
    warm_up(step, max(1, args.warmup // 2), 50.0)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    with gdn.profile() as prof:
        for _ in range(steps):
            step()
    torch.cuda.synchronize()
    kernels = {name: {"launches": n_, "avg_us": 1e3 * t / n_} for name, (n_, t) in prof.results.items()}
    dom = max(kernels, key=lambda x: kernels[x]["avg_us"] * kernels[x]["launches"])
    items = B * ((T + C - 1) // C) * H
    gflops = bwd_grad_flops_per_chunk_head(dk, dv) * items
    g_s = kernels["gdn_bwd_grad"]["avg_us"] * 1e-6
    res = {
        "value": B * T / (ms * 1e-3), "unit": "tokens/s", "ms_per_call": ms, "calls": steps,
        "config": {"workload": "backward", "B": B, "L": T, "H": H, "dk": dk, "dv": dv, "chunk": C,
                   "in_dtype": "bf16", "grads": "fp32", "d_final": "fp32"},
        "roofline": {"kernel": "gdn_bwd_grad", "bound": "mfma", "achieved": gflops / g_s / 1e12,
                     "peak": MFMA_F32_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": gflops / g_s / 1e12 / MFMA_F32_PEAK_TFLOPS,
                     "traffic": measured_traffic("gdn_bwd_grad", "backward"), "algorithmic_flops": gflops,
                     "mfma_busy_counter": measured_mfma_busy("gdn_bwd_grad", "backward"),
                     "note": "flops priced at the fp32 matrix peak although the bf16-input dQ/dK products run as "
                             "exact three-term bf16 splits on the bf16 instruction; mfma_busy_counter is the "
                             "hardware share of matrix-core cycles, independent of that pricing",
                     "dominant_kernel": dom},
        "kernels": kernels,
    }
    del q, k, v, la, be, d_o, d_fin, ws
    torch.cuda.empty_cache()
    return res


def run_cpu_baseline(inp, seconds):
    """The fp64 oracle on a workload's inputs, on all host cores: a prefix of every sequence, grown until
    one pass takes about `seconds`; once the prefix is the whole workload, whole passes are repeated
    until the total reaches `seconds`.  Packed batches are cut per sequence (the same prefix length of
    each, capped at its own length)."""
    import numpy as np

    import oracle
    threads = oracle.num_threads()
    H = inp.H
    bounds = inp.seq_bounds()
    longest = max(e - s for _, s, e in bounds)

    def one(sl):
        # the sample is cut and widened to fp64 outside the timed region
        if inp.cu_seqlens is None:
            idx, cu = np.arange(sl), None
        else:
            idx = np.concatenate([np.arange(s, min(e, s + sl)) for _, s, e in bounds])
            cu = np.concatenate([[0], np.cumsum([min(e - s, sl) for _, s, e in bounds])])
        args = [np.ascontiguousarray(x[:, idx], dtype=np.float64)
                for x in (inp.q, inp.k, inp.v, inp.log_alpha, inp.beta)]
        t0 = time.perf_counter()
        oracle.recurrent(*args, init_state=inp.init_state, cu_seqlens=cu, threads=threads)
        return time.perf_counter() - t0, inp.B * len(idx)

    sl = 64
    while True:
        el, ntok = one(sl)
        if el >= seconds or sl >= longest:
            break
        sl = min(longest, max(sl * 2, int(sl * seconds / max(el, 1e-3) * 1.1)))
    passes, total = 1, ntok
    while el < seconds:
        dt, n = one(sl)
        el += dt
        total += n
        passes += 1
    what = (f"first {sl} of {inp.T} tokens of each of the {inp.B} sequences" if inp.cu_seqlens is None else
            f"first min({sl}, length) tokens of each of the {len(bounds)} packed sequences ({ntok} of {inp.T})")
    return {"value": total / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{inp.name} workload, {what}, all {H} heads, {passes} pass(es) "
                      f"(fp64 token recurrence, {el:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--out-dtype", choices=["fp32", "bf16", "fp16"], default="fp32",
                    help="prefill output dtype (the state is fp32 either way)")
    ap.add_argument("--only", choices=["prefill", "long", "packed", "decode", "continuation", "backward", "copy"],
                    default=None,
                    help="run one leg only (for profiler runs) and print its part of the line; "
                         "'copy' runs a plain 256 MiB read + 256 MiB write elementwise kernel used to "
                         "calibrate the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the path has no multi-GPU mode; "
              "(sequence, head) pairs are independent and would be sharded with no communication.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_delta_rule_24_amd as gdn
    import workloads as W

    if not os.path.exists(gdn.lib_path()):
        from gated_delta_rule_24_amd import build as gbuild
        gbuild.build()
    gdn.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.only == "decode":
        print(json.dumps({"decode": run_decode(args, gdn, W, dev)}), flush=True)
        return
    if args.only == "continuation":
        print(json.dumps({"continuation": run_continuation(args, gdn, W, dev)}), flush=True)
        return
    if args.only == "backward":
        print(json.dumps({"backward": run_backward(args, gdn, W, dev)}), flush=True)
        return
    if args.only == "copy":
        n = 64 * 1024 * 1024                      # 256 MiB of fp32
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        launches = max(1, args.steps)
        torch.mul(a, 1.0, out=b)                  # warm-up launch
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()                               # torch's current stream, the one the copies run on
        for _ in range(launches):
            torch.mul(a, 1.0, out=b)
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) * 1e3 / launches
        print(json.dumps({"copy": {"bytes_read": 4 * n, "bytes_written": 4 * n, "launches": launches + 1,
                                   "avg_us": us, "GB/s": 8 * n / us / 1e3}}), flush=True)
        return
    legs = {}
    for name in ("prefill", "long", "packed"):
        if args.only not in (None, name):
            continue
        legs[name] = run_chunk_workload(args, gdn, W, dev, name, args.out_dtype)
    if args.only is not None:
        res = legs[args.only][0]
        print(json.dumps({args.only: res}), flush=True)
        return
    pre, inp = legs["prefill"]
    decode = run_decode(args, gdn, W, dev)
    cont = run_continuation(args, gdn, W, dev)
    bwd = run_backward(args, gdn, W, dev)
    cpu = None if args.no_cpu_baseline else run_cpu_baseline(inp, args.cpu_seconds)
    extra = {}
    for name in ("long", "packed"):
        res, winp = legs[name]
        if not args.no_cpu_baseline:
            res["cpu_baseline"] = run_cpu_baseline(winp, args.cpu_seconds / 3)
        extra[name] = res
    del legs, inp
    out = {
        "metric": METRIC,
        "value": pre["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["ms_per_step"],
        "ms_median": pre["ms_median"],
        "ms_min": pre["ms_min"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "compute": "bf16 inputs; fp16 matrix-core operands, fp32 accumulation and fp32 state",
        "data": "synthetic (seeded; q,k L2-normalised, log_alpha~U(-0.1,-0.001), beta=sigmoid(N(0,1)))",
        "config": pre["config"],
        "roofline": pre["roofline"],
        "cpu_baseline": cpu,
        "long": extra["long"],
        "packed": extra["packed"],
        "decode": decode,
        "continuation": cont,
        "backward": bwd,
        "kernels": pre["kernels"],
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
