#!/usr/bin/env python3
"""Benchmark of libgdn on one MI355X.

One step = one pass of the whole hot path: gdn_chunk_fwd over the 64K-token
layer (B=1, T=65536, 16 QK / 48 V heads, head dim 128, chunk 64, bf16
q/k/v, fp32 gates and state, nonzero initial state) and one
gdn_decode_step over the 256-sequence batch (fp32 state 256 x 48 x 128 x 128,
updated in place; the step index advances through successive decode tokens).
The K timed prefills run first, then the K timed decode steps back to back.
Inputs are generated once, moved to HBM, and are resident before timing
starts.

The step's prefill is one gdn_chunk_fwd call, timed with HIP events (torch
events on the stream it is called on). On this shape the library runs kernel
2's later chunks on a second stream beside the scan (the scan's 192
workgroups leave a quarter of the CUs idle), so the kernels overlap and
their durations cannot be told apart inside the step. Each kernel's launch
duration is therefore measured in a second timed region, in which the same
prefill is enqueued one stage at a time through gdn_chunk_fwd_stages (one
whole-sequence launch per kernel, events between them); these launches, and
the windowed ones of the step, carry different kernel names in a trace.
`value` is prefill tokens/s (T / mean prefill time of the step); decode GB/s
is reported beside it. Prints one JSON line.

`roofline` grades the prefill's dominant kernel (the fused scan) as a dense
contraction: its algorithmic flops (6 dk dv + 4 C dv per token and V head:
W S, K^T U, Q S, P U and Ut) over its mean launch time, against bf16 MFMA
peak (2.5 PFLOP/s). `roofline_prefill` does the same for the whole prefill
(7,667,712 flops per token) and splits its bytes into the layer's compulsory
I/O and the design's workspace intermediates. `roofline_decode` grades the
decode step against HBM peak (8 TB/s). `cpu_baseline` times the oracle on
this host's cores before the GPU is touched.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN prefill tokens/s at T=64K (48 V heads, d=128) + decode state GB/s"
PEAK_BF16_FLOPS = 2.5e15      # MI355X dense bf16 MFMA
PEAK_HBM_BYTES = 8.0e12       # MI355X HBM3E
STAGES = ["gdn_k2_inverse_w", "gdn_k3_scan"]
DECODE_KERNEL = "gdn_kd_decode_step"


def algorithmic_work(T, HQ, HV, D, C, N, decode_batch):
    """Per-launch algorithmic flops and HBM bytes of each kernel, from the
    chunkwise method's operation counts (dense C x C in-chunk products, bf16
    q/k/v/o and fragments, fp32 gates and states; the causal C x C operands
    Tinv diag(b) and P count the bytes of their lower triangles), and the
    resource that bounds it (the one whose time at peak is larger); see the
    design notes. Returns ({kernel: (bound, flops, bytes)}, flops per token)."""
    dk = dv = D
    e = 2                                       # bytes per bf16 element
    gates = T * HV * 8                          # log a and b (fp32), or g and b
    tri = (C + 1) / 2.0                         # lower-triangle elements per token of a causal C x C operand
    work = {
        # K K^T and Q K^T per QK head, the triangular inverse and W per V
        # head; reads q, k, log a, b; writes the K^T and Q fragments (once per
        # QK head), Tinv diag(b), W, the masked q.k fragments P and the
        # row-factor table (2C + 4 fp32 per chunk and V head)
        "gdn_k2_inverse_w": (T * (HQ * 4 * C * dk + HV * (C * C / 3.0 + 2 * C * dk)),
                             2 * T * HQ * dk * e + gates + T * HQ * 2 * dk * e
                             + T * HV * (2 * tri + dk) * e + T * HV * (2 * C + 4) * 4 / C),
        # Ut, W S, Q S, K^T U, P U per V head; reads Q, K^T, P, V, Tinv
        # diag(b), W, the row factors and the initial states; writes o and the
        # final states
        "gdn_k3_scan": (T * HV * (6 * dk * dv + 4 * C * dv),
                        T * HQ * 2 * dk * e + T * HV * (dv + 2 * tri + dk) * e + T * HV * (2 * C + 4) * 4 / C
                        + T * HV * dv * e + 2 * N * HV * dk * dv * 4),
    }
    per_token = HV * (6 * dk * dv + 2 * C * dk + 4 * C * dv + C * C / 3.0) + HQ * 4 * C * dk
    total_flops = sum(f for f, _ in work.values())
    assert abs(total_flops - per_token * T) < 1e-6 * total_flops
    out = {}
    for k, (f, b) in work.items():
        out[k] = ("mfma" if f / PEAK_BF16_FLOPS > b / PEAK_HBM_BYTES else "hbm", float(f), float(b))
    state = decode_batch * HV * dk * dv * 4
    dec_bytes = 2 * state + decode_batch * (2 * HQ * dk * 2 + 2 * HV * dv * 2 + 2 * HV * 4)
    out[DECODE_KERNEL] = ("hbm", 0.0, float(dec_bytes))
    return out, per_token


BWD_STAGES = ["gdn_k1_chunk_prep", "gdn_k2_inverse_w [bwd]", "gdn_k3_scan [save]", "gdn_kb_dstate",
              "gdn_kb_grad"]


def algorithmic_work_bwd(T, HQ, HV, D, C, N):
    """Per-launch algorithmic flops and HBM bytes of the backward pass's
    kernels (gdn_chunk_bwd's five launches), counted as for the forward:
    dense C x C in-chunk products, compulsory reads and writes of each
    launch (bf16 rows and fragments, fp32 gates and states; Tinv diag(b)
    counts its lower triangle). Returns
    {kernel: (bound, flops, bytes)}."""
    dk = dv = D
    e = 2
    gates = T * HV * 8
    tri = (C + 1) / 2.0                         # lower-triangle elements per token of a causal C x C operand
    dtab = T * HV * (2 * C + 4) * 4 / C
    states = N * HV * dk * dv * 4
    chunk_states = T / C * HV * dk * dv * e     # one dk x dv matrix per chunk and V head
    work = {
        # Q K^T (query-indexed) per QK head; reads q, k, log a, b; writes g, b,
        # K^T, K and Q^T fragments, the query-indexed q.k fragments
        "gdn_k1_chunk_prep": (T * HQ * 2 * C * dk,
                              2 * T * HQ * dk * e + 2 * gates + 3 * T * HQ * dk * e + T * HQ * C * e),
        # K K^T, the inverse, W and W^T; reads k, q.k, g, b; writes Tinv
        # diag(b), W, the row factors, P^T, W^T and Tinv^T
        "gdn_k2_inverse_w [bwd]": (T * (HQ * 2 * C * dk + HV * (C * C / 3.0 + 4 * C * dk)),
                                   T * HQ * (dk + C) * e + gates
                                   + T * HV * (2 * C + tri + 2 * dk) * e + dtab),
        # Ut, W S, K^T U; reads K^T, V, Tinv diag(b), W, the row factors and
        # the initial states; writes the chunk-start states and U
        "gdn_k3_scan [save]": (T * HV * (4 * dk * dv + 2 * C * dv),
                               T * HQ * dk * e + T * HV * (dv + tri + dk) * e + dtab + states
                               + chunk_states + T * HV * dv * e),
        # K dS, P^T dO, Q^T dO, W^T dU; reads K and Q^T, P^T and W^T
        # fragments, the row factors, dL/do, dL/dS_final; writes dL/dS_end per
        # chunk, dL/dU, dL/dS_0
        "gdn_kb_dstate": (T * HV * (6 * dk * dv + 2 * C * dv),
                          2 * T * HQ * dk * e + T * HV * (C + dk + dv) * e + dtab + states
                          + chunk_states + T * HV * dv * e + states),
        # dO S0^T, U dS^T, dU S0^T, dO U^T, dPm K, dPm^T Q, dT, K K^T,
        # (B + B^T) K, Tinv^T dU, Tinv^T dW (and the fp32 C^3 products of dA);
        # reads q, k, their fragments, dL/do, v, U, dL/dU, Tinv^T, P^T, the
        # states, g, b, the row factors; writes dq, dk, dv, dlog a, db
        "gdn_kb_grad": (T * HV * (6 * dk * dv + 4 * C * dv + 10 * C * dk + 4 * C * C),
                        4 * T * HQ * dk * e + 4 * T * HV * dv * e + 2 * T * HV * C * e + 2 * chunk_states
                        + gates + dtab + 2 * T * HQ * dk * e + T * HV * dv * e + gates),
    }
    return {k: ("mfma" if f / PEAK_BF16_FLOPS > b / PEAK_HBM_BYTES else "hbm", float(f), float(b))
            for k, (f, b) in work.items()}


def backward_bench(gdn, I, inp, dev, stream, T, HQ, HV, D, C, reps=3):
    """The backward pass of the same 64K-token layer (seeded dL/do and
    dL/dS_final), per launch, with events between its five stages."""
    import torch
    seeds = I.make_backward_seeds(31, [T], HV, D, "bf16")
    d_o, dfin = seeds["d_o"].to(dev), seeds["d_final"].to(dev)
    dims = gdn.make_dims(1, T, HQ, HV, D, D, C, torch.bfloat16)
    ws = torch.empty(gdn.gdn_chunk_bwd_workspace_bytes(dims), dtype=torch.uint8, device=dev)
    grads = dict(dq=torch.empty_like(inp["q"]), dk=torch.empty_like(inp["k"]), dv=torch.empty_like(inp["v"]),
                 dlog_alpha=torch.empty_like(inp["log_alpha"]), dbeta=torch.empty_like(inp["beta"]),
                 d_init_state=torch.empty_like(inp["init_state"]))

    def stage(s):
        gdn.gdn_chunk_bwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], d_o, inp["init_state"],
                          None, dfin, chunk=C, workspace=ws, grads=grads, stages=(s, s))
    n = len(BWD_STAGES)
    for s in range(1, n + 1):
        stage(s)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(reps)]
    for i in range(reps):
        for s in range(n):
            ev[i][s].record(stream)
            stage(s + 1)
        ev[i][n].record(stream)
    torch.cuda.synchronize()
    ms = {name: sum(ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(reps)) / reps
          for j, name in enumerate(BWD_STAGES)}
    total = sum(ms.values())
    work = algorithmic_work_bwd(T, HQ, HV, D, C, 1)
    kernels = {}
    for name in BWD_STAGES:
        bound, flops, nbytes = work[name]
        amount = flops if bound == "mfma" else nbytes
        rate = amount / (ms[name] * 1e-3)
        peak = PEAK_BF16_FLOPS if bound == "mfma" else PEAK_HBM_BYTES
        kernels[name] = {"ms": round(ms[name], 4), "bound": bound,
                         "achieved": round(rate / (1e12 if bound == "mfma" else 1e9), 3),
                         "unit": "TFLOP/s" if bound == "mfma" else "GB/s", "frac": round(rate / peak, 4),
                         "mfma_frac": round(flops / (ms[name] * 1e-3) / PEAK_BF16_FLOPS, 4),
                         "hbm_frac": round(nbytes / (ms[name] * 1e-3) / PEAK_HBM_BYTES, 4)}
    del ws
    return {"ms": round(total, 4), "tokens_per_s": round(T / (total * 1e-3), 1),
            "mfma_frac": round(sum(work[k][1] for k in BWD_STAGES) / (total * 1e-3) / PEAK_BF16_FLOPS, 4),
            "kernels": kernels}


def load_traffic(kernel):
    """Measured HBM bytes per launch of `kernel` from the committed counter
    summary (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a plain copy), or
    None when there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel)
    if not rec:
        return None
    src = os.path.join(ROOT, "linear_attention_recurrence_delta_amd", "csrc", rec["source"])
    with open(src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec["source_sha256"]:
            return None
    return rec["bytes_per_launch"]


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _pool_unit(args):
    """One (sequence, V head) unit of the pool leg: the NumPy form-1
    recurrence over the unit's tokens, one thread."""
    from threadpoolctl import threadpool_limits
    from oracle import gdn_oracle as O
    with threadpool_limits(limits=1):
        _, fin = O.recurrent_form1(*args)
    return float(fin.sum())


def cpu_baseline(inp, seconds):
    """The fp64 oracle as it stands, on bounded samples of the same 64K-token
    input (all 48 V heads), on this host's cores, in three legs of about
    `seconds` / 3 each: the NumPy form-1 recurrence in one process
    (vectorised over heads, one thread); the same recurrence over
    independent (sequence, V head) units in a process pool with one worker
    per core; and the C writing of the same recurrence with one thread per
    core. Returns (headline leg, all legs); rates are oracle tokens/s (every
    head of a token counted once)."""
    import multiprocessing as mp
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import c_ref as CR
    from oracle import gdn_oracle as O
    cores = len(os.sched_getaffinity(0))
    f64 = {x: inp[x].double().numpy() for x in ("q", "k", "v", "log_alpha", "beta")}
    state = inp["init_state"].double().numpy()
    hv, group = f64["v"].shape[1], f64["v"].shape[1] // f64["q"].shape[1]
    legs = {}
    # one process, tokens in blocks of 32 until the time share is used
    block, done, budget = 32, 0, seconds / 3.0
    st = state
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while time.perf_counter() - t0 < budget and done + block <= f64["q"].shape[0]:
            s = slice(done, done + block)
            _, st = O.recurrent_form1(*(f64[x][s] for x in ("q", "k", "v", "log_alpha", "beta")), st)
            done += block
    dt = time.perf_counter() - t0
    assert np.isfinite(st).all()
    legs["numpy_one_process"] = {"value": round(done / dt, 2), "cores": 1, "tokens": done,
                                 "seconds": round(dt, 2)}
    # process pool over (sequence, V head) units, sized from the one-process rate
    n_pool = int(min(f64["q"].shape[0], max(256, budget * cores * done / dt / 1.5)))
    units = [(f64["q"][:n_pool, h // group:h // group + 1], f64["k"][:n_pool, h // group:h // group + 1],
              f64["v"][:n_pool, h:h + 1], f64["log_alpha"][:n_pool, h:h + 1], f64["beta"][:n_pool, h:h + 1],
              state[:, h:h + 1]) for h in range(hv)]
    ctx = mp.get_context("spawn")
    with ctx.Pool(cores) as pool:
        pool.map(_pool_unit, units[:cores])            # workers started and warm
        t0 = time.perf_counter()
        sums = pool.map(_pool_unit, units, chunksize=1)
        dt = time.perf_counter() - t0
    assert np.isfinite(sums).all()
    legs["numpy_pool"] = {"value": round(n_pool / dt, 2), "cores": cores, "tokens": n_pool,
                          "seconds": round(dt, 2)}
    # the C recurrence, one thread per core, sized from the first calibration
    f32 = {x: inp[x].float().numpy() for x in ("q", "k", "v", "log_alpha", "beta")}
    n_c = 1024
    CR.recurrent_form1(*(f32[x][:n_c] for x in ("q", "k", "v", "log_alpha", "beta")), state, None, cores)
    while True:
        t0 = time.perf_counter()
        _, fin = CR.recurrent_form1(*(f32[x][:n_c] for x in ("q", "k", "v", "log_alpha", "beta")), state, None,
                                    cores)
        dt = time.perf_counter() - t0
        if dt >= budget / 4 or n_c >= f32["q"].shape[0]:
            break
        n_c = int(min(f32["q"].shape[0], n_c * max(2.0, budget / max(dt, 1e-3))))
    assert np.isfinite(fin).all()
    legs["c_threads"] = {"value": round(n_c / dt, 2), "cores": cores, "tokens": n_c, "seconds": round(dt, 2)}
    best = max(legs, key=lambda k: legs[k]["value"])
    return best, legs


def verify_bench(gdn, I, dev, decode_ms, kt=4, reps=5):
    """Speculative verify of `kt` drafted tokens for the 256-sequence batch in
    one gdn_decode_multi pass: with per-token snapshots (state read once,
    kt states written) and committing in place (state read and written
    once). Timed outside the prefill region; HBM bytes are the state traffic
    plus the per-token inputs and outputs."""
    import torch
    spec = I.WORKLOADS["decode_256"]
    dec = I.workload_inputs("decode_256", steps=kt)
    args = [dec[x].to(dev) for x in ("q", "k", "v", "log_alpha", "beta")]
    state = dec["state0"].to(dev)
    snaps = torch.empty((kt,) + tuple(state.shape), dtype=torch.float32, device=dev)
    o = torch.empty_like(args[2])
    nb, hq, hv, d = spec["batch"], spec["h_qk"], spec["h_v"], spec["d"]
    sbytes = nb * hv * d * d * 4
    io = kt * nb * (2 * hq * d * 2 + 2 * hv * d * 2 + 2 * hv * 4)
    out = {"tokens_per_seq": kt, "sequences": nb}
    for name, snap, nbytes in (("snapshots", snaps, sbytes * (1 + kt) + io), ("commit", None, 2 * sbytes + io)):
        gdn.gdn_decode_multi(*args, state, o=o, snapshots=snap)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(torch.cuda.current_stream(dev))
        for _ in range(reps):
            gdn.gdn_decode_multi(*args, state, o=o, snapshots=snap)
        e1.record(torch.cuda.current_stream(dev))
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"ms": round(ms, 4), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "hbm_frac": round(nbytes / (ms * 1e-3) / PEAK_HBM_BYTES, 4),
                     "tokens_per_s": round(kt * nb / (ms * 1e-3), 1)}
    out["commit_vs_single_steps"] = round(kt * decode_ms / out["commit"]["ms"], 3)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (read BYTES, write BYTES) a few "
                         "times, as the reference for scaling HBM byte counters")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    import linear_attention_recurrence_delta_amd as gdn
    from linear_attention_recurrence_delta_amd import inputs as I

    spec = I.WORKLOADS["long_64k"]
    dspec = I.WORKLOADS["decode_256"]
    T, HQ, HV, D, C = spec["seq_lens"][0], spec["h_qk"], spec["h_v"], spec["d"], spec["chunk"]
    NB = dspec["batch"]
    n_dec = min(dspec["steps"], args.warmup + args.steps)

    inp_cpu = I.workload_inputs("long_64k")
    # the CPU baseline runs first, before this process touches the GPU (its
    # pool leg starts worker processes)
    cpu_line = None
    if not args.no_cpu_baseline:
        best, legs = cpu_baseline(inp_cpu, args.cpu_seconds)
        descr = {"numpy_one_process": "NumPy form-1 recurrence, one process, one thread",
                 "numpy_pool": "NumPy form-1 recurrence over (sequence, V head) units, one worker process per core",
                 "c_threads": "C form-1 recurrence (oracle/gdn_ref.c), one thread per (sequence, V head) unit"}
        cpu_line = {
            "value": legs[best]["value"], "unit": "tokens/s", "cores": legs[best]["cores"], "kind": "oracle",
            "sample": f"first {legs[best]['tokens']} tokens of the same 64K-token input, all 48 V heads, fp64; "
                      f"{descr[best]}; {legs[best]['seconds']} s",
            "cpu_model": cpu_model(), "affinity_cores": len(os.sched_getaffinity(0)),
            "legs": legs}
    gdn.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp_cpu.items()}
    dec = I.workload_inputs("decode_256", steps=n_dec)
    dec = {k: v.to(dev) for k, v in dec.items()}
    state = dec["state0"].clone()
    dims = gdn.make_dims(1, T, HQ, HV, D, D, C, torch.bfloat16)
    ws = torch.empty(gdn.gdn_chunk_fwd_workspace_bytes(dims), dtype=torch.uint8, device=dev)
    o = torch.empty_like(inp["v"])
    fin = torch.empty_like(inp["init_state"])
    o_dec = torch.empty_like(dec["v"][0])
    stream = torch.cuda.current_stream(dev)

    def prefill(stages=None):
        gdn.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                          inp["init_state"], None, chunk=C, workspace=ws, o=o, final_state=fin,
                          stages=stages)

    def decode(i):
        j = i % n_dec
        gdn.gdn_decode_step(dec["q"][j], dec["k"][j], dec["v"][j], dec["log_alpha"][j],
                            dec["beta"][j], state, o=o_dec)

    for i in range(args.warmup):
        prefill()
        for s in range(1, len(STAGES) + 1):
            prefill((s, s))
        decode(i)
    torch.cuda.synchronize()

    K = args.steps
    NST = len(STAGES)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    dev_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        prefill()
        ev[i][1].record(stream)
    # the K decode steps run back to back after the K prefills, as a serving
    # loop runs them: a step enqueued right behind a 64K-token prefill also
    # absorbs the write-back of that prefill's outputs from the caches
    for i in range(K):
        dev_ev[i][0].record(stream)
        decode(args.warmup + i)
        dev_ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # each kernel's launch duration: the same prefill, one stage at a time
    kev = [[torch.cuda.Event(enable_timing=True) for _ in range(NST + 1)] for _ in range(K)]
    for i in range(K):
        for s in range(NST):
            kev[i][s].record(stream)
            prefill((s + 1, s + 1))
        kev[i][NST].record(stream)
    torch.cuda.synchronize()

    names = STAGES + [DECODE_KERNEL]
    ms = {n: sum(kev[i][j].elapsed_time(kev[i][j + 1]) for i in range(K)) / K
          for j, n in enumerate(STAGES)}
    ms[DECODE_KERNEL] = sum(dev_ev[i][0].elapsed_time(dev_ev[i][1]) for i in range(K)) / K
    prefill_ms = sum(ev[i][0].elapsed_time(ev[i][1]) for i in range(K)) / K
    stagewise_ms = sum(kev[i][0].elapsed_time(kev[i][NST]) for i in range(K)) / K
    decode_ms = ms[DECODE_KERNEL]
    work, per_token = algorithmic_work(T, HQ, HV, D, C, 1, NB)
    kernels = {}
    for n in names:
        bound, flops, nbytes = work[n]
        amount = flops if bound == "mfma" else nbytes
        rate = amount / (ms[n] * 1e-3)
        peak = PEAK_BF16_FLOPS if bound == "mfma" else PEAK_HBM_BYTES
        kernels[n] = {"ms": round(ms[n], 4), "bound": bound,
                      "achieved": round(rate / (1e12 if bound == "mfma" else 1e9), 3),
                      "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
                      "frac": round(rate / peak, 4),
                      "mfma_frac": round(flops / (ms[n] * 1e-3) / PEAK_BF16_FLOPS, 4),
                      "hbm_frac": round(nbytes / (ms[n] * 1e-3) / PEAK_HBM_BYTES, 4)}
    # The headline roofline grades the prefill's dominant kernel (the scan)
    # as the method's dense contraction: its share of the method's flops
    # (W S, K^T U, Q S, P U and Ut per V head) against bf16 MFMA peak.
    dominant = max(STAGES, key=lambda n: ms[n])
    d_flops = work[dominant][1]
    roofline = {"kernel": dominant, "bound": "mfma",
                "achieved": round(d_flops / (ms[dominant] * 1e-3) / 1e12, 3), "peak": 2500.0, "unit": "TFLOP/s",
                "frac": round(d_flops / (ms[dominant] * 1e-3) / PEAK_BF16_FLOPS, 4),
                "traffic": load_traffic(dominant),
                "flops_per_launch": d_flops, "flops_per_token": d_flops / T}
    # the whole prefill: the method's flops against MFMA peak; its bytes
    # split into the layer's compulsory I/O (q, k, v, o, gates, states) and
    # what this design adds (the workspace intermediates kernel 2 writes
    # and the scan reads)
    compulsory = T * (2 * HQ * D * 2 + 2 * HV * D * 2 + 2 * HV * 4) + 2 * HV * D * D * 4
    design = sum(work[n][2] for n in STAGES)
    measured = [load_traffic(n) for n in STAGES]
    sec = prefill_ms * 1e-3
    roofline_prefill = {
        "flops": per_token * T, "mfma_achieved_TFLOPs": round(per_token * T / sec / 1e12, 3),
        "mfma_frac": round(per_token * T / sec / PEAK_BF16_FLOPS, 4),
        "compulsory_bytes": compulsory, "compulsory_hbm_frac": round(compulsory / sec / PEAK_HBM_BYTES, 4),
        "design_bytes": round(design), "intermediate_bytes": round(design - compulsory),
        "measured_bytes": None if None in measured else sum(measured)}
    dec_bytes = work[DECODE_KERNEL][2]
    tokens_per_s = T / (prefill_ms * 1e-3)

    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "64K-token GDN layer prefill (B=1, T=65536, 16 QK / 48 V heads, "
                               "d=128, chunk 64, bf16 q/k/v, fp32 gates/state, N(0,0.02^2) "
                               "init) + one batched decode step (256 sequences, fp32 state "
                               "256x48x128x128 in place)",
                   "tokens": T, "chunk": C, "decode_batch": NB},
        "prefill_ms": round(prefill_ms, 4),
        "prefill_stagewise_ms": round(stagewise_ms, 4),
        "prefill_mfma_frac": round(per_token * T / (prefill_ms * 1e-3) / PEAK_BF16_FLOPS, 4),
        "decode_ms": round(decode_ms, 4),
        "decode_GBps": round(dec_bytes / (decode_ms * 1e-3) / 1e9, 1),
        "decode_hbm_frac": round(dec_bytes / (decode_ms * 1e-3) / PEAK_HBM_BYTES, 4),
        "roofline": roofline,
        "roofline_prefill": roofline_prefill,
        "roofline_decode": {"kernel": DECODE_KERNEL, "bound": "hbm",
                            "achieved": kernels[DECODE_KERNEL]["achieved"], "peak": 8000.0,
                            "unit": "GB/s", "frac": kernels[DECODE_KERNEL]["frac"],
                            "traffic": load_traffic(DECODE_KERNEL)},
        "kernels": kernels,
        "cpu_baseline": None,
    }
    line["cpu_baseline"] = cpu_line
    line["decode_verify"] = verify_bench(gdn, I, dev, decode_ms)
    # fused input preparation (raw q, k and gate logits): the same workload
    # with the flag set; the kernels' work does not depend on the values
    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps
    pf_prep = timed(lambda: gdn.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                                              inp["init_state"], None, chunk=C, workspace=ws, o=o,
                                              final_state=fin, prepare_inputs=True))
    dec_prep = timed(lambda: gdn.gdn_decode_step(dec["q"][0], dec["k"][0], dec["v"][0], dec["log_alpha"][0],
                                                 dec["beta"][0], state, o=o_dec, prepare_inputs=True))
    line["prepare_inputs"] = {"prefill_ms": round(pf_prep, 4), "prefill_tokens_per_s": round(T / (pf_prep * 1e-3), 1),
                              "decode_ms": round(dec_prep, 4),
                              "decode_GBps": round(dec_bytes / (dec_prep * 1e-3) / 1e9, 1)}
    # the gate-only variant (S <- a S + b k v^T) on the same inputs, per
    # kernel; DeltaNet (log a = 0) runs the kernels timed above unchanged
    def gate_only_stage(s):
        gdn.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                          inp["init_state"], None, chunk=C, workspace=ws, o=o, final_state=fin,
                          stages=(s, s), delta_rule=False)
    go_ms = [timed(lambda s=s: gate_only_stage(s)) for s in range(1, NST + 1)]
    dec_go = timed(lambda: gdn.gdn_decode_step(dec["q"][0], dec["k"][0], dec["v"][0], dec["log_alpha"][0],
                                               dec["beta"][0], state, o=o_dec, delta_rule=False))
    line["backward"] = backward_bench(gdn, I, inp, dev, stream, T, HQ, HV, D, C)
    line["gate_only"] = {"prefill_ms": round(sum(go_ms), 4), "prefill_tokens_per_s": round(T / (sum(go_ms) * 1e-3), 1),
                         "kernel_ms": {n: round(t, 4) for n, t in zip(STAGES, go_ms)},
                         "decode_ms": round(dec_go, 4),
                         "decode_GBps": round(dec_bytes / (dec_go * 1e-3) / 1e9, 1)}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
