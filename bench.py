"""Benchmark of the SSD hot path on one MI355X.

One step = one pass of the whole path over one batch: ssd_fwd over the prefill batch
(chunk_state with the dt' cumsum and, for fp32, C B^T once per group -> state_passing ->
chunk_scan; for large bf16 batches chunk_state_seq, one pass over the chunks with the state
carried in registers, in place of the first two), writing final_state, then one ssd_step
decode token per sequence continuing
from that state.  Other workloads (--workload): the backward (ssd_bwd), the decode loop and
the conv1d + SiLU in front of the scan.  Workload: the fp32
forward of batch 4 x 1024 tokens, 24 heads, headdim 64, dstate 64, 1 group, chunk 256
(plus its decode token).  Inputs are seeded synthetic tensors resident in HBM before the
timed region.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--workload NAME]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import torch  # noqa: E402

from state_space_sequence_mamba_amd import inputs as I  # noqa: E402
from state_space_sequence_mamba_amd import ssd  # noqa: E402
from state_space_sequence_mamba_amd.profiling import load_traffic, workload_slug  # noqa: E402
from state_space_sequence_mamba_amd.timing import HipEvents  # noqa: E402

HBM_PEAK_GBS = 8000.0                         # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0}   # dense matrix peaks, TFLOP/s
DEFAULT_WORKLOAD = "ssd_fwd f32 B4 L1024 H24 P64 N64 G1 Q256"
KERNELS = ["chunk_state", "state_passing", "chunk_scan", "ssd_step"]


def algorithmic_cost(w):
    """Bytes each kernel must move (its inputs once, its outputs once) and the flops it must
    do (causal half of the in-chunk products, C B^T once per group), per launch."""
    e = 4 if w.dtype == "f32" else 2
    B, L, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    nc = (L + Q - 1) // Q
    lens = [min(Q, L - c * Q) for c in range(nc)]
    cum = 2 * B * H * nc * Q * 4                       # dt' and its cumsum, fp32
    st = B * nc * H * P * N * 4                        # chunk states, fp32
    fin = B * H * P * N * 4
    x = B * L * H * P * e
    bc = B * L * G * N * e
    tri = sum(n * (n + 1) // 2 for n in lens)           # causal (i, j) pairs per (b, h) sequence
    pre = w.dtype == "f32"
    nrb = Q // 64
    cbw = B * nc * G * (nrb * (nrb + 1) // 2) * 16 * 1024     # C B^T blocks written (16 KB each)
    cbr = cbw * (H // G)                                        # ... and read once per head
    cost = {
        # dt' and its cumsum (dt in, both out), the chunk states; fp32 adds C B^T once per group
        # (C in, 16 KB blocks out, one per row block and causal column block)
        "chunk_state": dict(bytes=B * L * H * e + 8 * H + cum + x + bc + st + ((bc + cbw) if pre else 0),
                            flops=2 * B * H * L * P * N + (2 * B * G * N * tri if pre else 0)),
        # one pass over the chunks: dt in, dt' and its cumsum out, x and B once, the entering
        # states out once (bf16: rounded to bf16) and the final state; fp32 adds C B^T as above
        "chunk_state_seq": dict(bytes=B * L * H * e + 8 * H + cum + x + bc + (st if pre else st // 2) + fin
                                + ((bc + cbw) if pre else 0),
                                flops=2 * B * H * L * P * N + (2 * B * G * N * tri if pre else 0)),
        # bf16 writes the entering states once, rounded to bf16, for the scan
        "state_passing": dict(bytes=st + (st // 2 if not pre else st) + fin + B * H * nc * 4,
                              flops=2 * B * nc * H * P * N),
        # fp32 reads the C B^T blocks back once per head; bf16 forms C B^T inside chunk_scan
        "chunk_scan": dict(bytes=2 * x + (cbr if pre else 2 * bc) + cum + (st if pre else st // 2) + H * P * 4,
                           flops=2 * B * H * P * tri + 2 * B * H * L * N * P + (0 if pre else 2 * B * G * N * tri)),
        # decode: state read + write, x, y, dt, B, C
        "ssd_step": dict(bytes=2 * fin + 2 * B * H * P * e + B * H * e + 2 * B * G * N * e,
                         flops=4 * B * H * P * N),
    }
    for k, v in cost.items():
        peak_f = MFMA_PEAK_TFLOPS[w.dtype] * 1e12
        t_f = v["flops"] / peak_f if k in ("chunk_state", "chunk_state_seq", "chunk_scan") else 0.0
        t_b = v["bytes"] / (HBM_PEAK_GBS * 1e9)
        v["bound"] = "mfma" if t_f > t_b else "hbm"
    return cost


def cpu_baseline(w, inp, dec, budget_s):
    """The float64 oracle (as it stands) on a bounded sample of the same step, single thread."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import ssd_recurrence

    f64 = lambda t: t.detach().cpu().double().numpy()  # noqa: E731
    rows = w.batch
    with threadpool_limits(1):
        # one pass over as many whole sequences as fit the budget, then repeat passes until
        # the budget is spent (or a cap of 30 s), so the rate rests on 10-30 s of work
        while True:
            x = np.concatenate([f64(inp["x"][:rows]), f64(dec["x"][0, :rows])[:, None]], axis=1)
            dt = np.concatenate([f64(inp["dt"][:rows]), f64(dec["dt"][0, :rows])[:, None]], axis=1)
            Bm = np.concatenate([f64(inp["B"][:rows]), f64(dec["B"][0, :rows])[:, None]], axis=1)
            Cm = np.concatenate([f64(inp["C"][:rows]), f64(dec["C"][0, :rows])[:, None]], axis=1)
            t0 = time.perf_counter()
            ssd_recurrence(x, dt, f64(inp["dt_bias"]), f64(inp["A"]), Bm, Cm, f64(inp["D"]))
            secs = time.perf_counter() - t0
            if secs <= budget_s or rows == 1:
                break
            rows = max(1, rows // 2)
        passes = 1
        while secs < budget_s and secs * (passes + 1) / passes < 30.0:
            t0 = time.perf_counter()
            ssd_recurrence(x, dt, f64(inp["dt_bias"]), f64(inp["A"]), Bm, Cm, f64(inp["D"]))
            secs += time.perf_counter() - t0
            passes += 1
    tokens = passes * rows * (w.seqlen + 1)
    return {"value": tokens / secs, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"float64 sequential recurrence over {rows} of {w.batch} sequences x "
                      f"{w.seqlen + 1} tokens (prefill + decode token), {passes} passes, {secs:.2f} s, "
                      f"numpy, 1 thread"}


def run_decode(w, args, dev):
    """The decode workload: `w.steps` consecutive ssd_step calls from a random state (one token
    per sequence per call), timed as one region; inputs for every step are resident in HBM."""
    inp = I.make_step_inputs(w.batch, w.nheads, w.headdim, w.dstate, w.ngroups, w.steps, w.dtype, w.seed,
                             w.d_init, device=dev)
    state = inp["state0"].clone()
    y = torch.empty_like(inp["x"][0])
    W = min(args.warmup, w.steps)
    for t in range(W):
        ssd.ssd_step(state, inp["x"][t], inp["dt"][t], inp["dt_bias"], inp["A"], inp["B"][t], inp["C"][t],
                     inp["D"], y=y)
    state.copy_(inp["state0"])
    torch.cuda.synchronize()
    hev = HipEvents()
    t0, t1 = hev.create(), hev.create()
    wall0 = time.perf_counter()
    hev.record(t0)
    for t in range(w.steps):
        ssd.ssd_step(state, inp["x"][t], inp["dt"][t], inp["dt_bias"], inp["A"], inp["B"][t], inp["C"][t],
                     inp["D"], y=y)
    hev.record(t1)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = hev.elapsed_ms(t0, t1)
    e = 2 if w.dtype == "bf16" else 4
    B, H, P, N, G = w.batch, w.nheads, w.headdim, w.dstate, w.ngroups
    alg_bytes = 8 * B * H * P * N + 2 * B * H * P * e + B * H * e + 2 * B * G * N * e
    per_step_s = ms * 1e-3 / w.steps
    ach = alg_bytes / per_step_s / 1e9
    out = {
        "metric": "SSD decode tokens/sec at 1 MI355X + % of HBM roofline", "value": round(B * w.steps / (ms * 1e-3), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": w.steps, "warmup": W, "ms_per_step": round(ms / w.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) state/x/B/C/dt per step)",
        "config": {"workload": w.name, "batch": B, "nheads": H, "headdim": P, "dstate": N, "ngroups": G},
        "roofline": {"kernel": "ssd_step", "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(workload_slug(w.name), "ssd_step"),
                     "alg_bytes_per_launch": alg_bytes},
        "wall_s_timed_region": round(wall, 4),
    }
    hev.close()
    emit(args, dev, out)


BWD_STAGES = ["chunk_state", "state_passing", "gate_fwd", "gate_bwd", "chunk_state_grad",
              "state_passing_rev", "bwd_dxdb", "bwd_dc", "bwd_finalize", "bwd_reduce"]


def backward_cost(w):
    """Algorithmic bytes and flops of each backward kernel per launch.  C B^T and dy x^T are
    counted once (in bwd_dxdb; bwd_dc recomputes them, which is not algorithmic work)."""
    e = 4 if w.dtype == "f32" else 2
    B, L, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    nc = (L + Q - 1) // Q
    lens = [min(Q, L - c * Q) for c in range(nc)]
    tri = sum(n * (n + 1) // 2 for n in lens)
    cum = B * H * nc * Q * 4
    st = B * nc * H * P * N * 4
    fin = B * H * P * N * 4
    x = B * L * H * P * e
    bc = B * L * G * N * e
    perh = B * L * H * N * 4
    cost = {
        "chunk_state": dict(bytes=B * L * H * e + 8 * H + cum + x + bc + st, flops=2 * B * H * L * P * N),
        "state_passing": dict(bytes=2 * st + B * H * nc * 4, flops=2 * B * nc * H * P * N),
        "gate_fwd": dict(bytes=0, flops=0),
        "gate_bwd": dict(bytes=0, flops=0),
        "chunk_state_grad": dict(bytes=x + bc + cum + st, flops=2 * B * H * L * P * N),
        "state_passing_rev": dict(bytes=2 * st + 2 * fin + B * H * nc * 4, flops=2 * B * nc * H * P * N),
        # C B^T, dy x^T and the weighted products contract tiles of the input dtype (MFMA in
        # that dtype); the carried terms through the fp32 state gradients run on fp32 MFMA
        "bwd_dxdb": dict(bytes=2 * x + 2 * bc + 2 * cum + st + x + perh + 3 * B * H * L * 4,
                         flops=2 * N * tri * B * G + 2 * P * tri * B * H * 2 + 2 * N * tri * B * H
                         + 4 * B * H * L * P * N,
                         flops_in=2 * N * tri * B * G + 2 * P * tri * B * H * 2 + 2 * N * tri * B * H),
        "bwd_dc": dict(bytes=2 * x + 2 * bc + 2 * cum + st + perh + B * H * L * 4,
                       flops=2 * N * tri * B * H + 2 * B * H * L * P * N,
                       flops_in=2 * N * tri * B * H),
        "bwd_finalize": dict(bytes=2 * st + 5 * cum + B * L * H * e * 2, flops=2 * B * nc * H * P * N),
        "bwd_reduce": dict(bytes=2 * perh + 2 * bc, flops=2 * B * L * H * N),
    }
    for k, v in cost.items():
        # chunk_state contracts on MFMA in the input dtype; the backward kernels' products run
        # on fp32 MFMA except the flops_in share (input-dtype MFMA): the peak is the blend that
        # the split implies, flops / (flops_in / peak_in + rest / peak_f32)
        p_in, p_32 = MFMA_PEAK_TFLOPS[w.dtype], MFMA_PEAK_TFLOPS["f32"]
        if k.startswith("chunk_state"):
            v["peak"] = p_in
        else:
            f_in = v.pop("flops_in", 0)
            t = f_in / p_in + (v["flops"] - f_in) / p_32
            v["peak"] = round(v["flops"] / t, 1) if t > 0 else p_32
        t_f = v["flops"] / (v["peak"] * 1e12)
        t_b = v["bytes"] / (HBM_PEAK_GBS * 1e9)
        v["bound"] = "mfma" if t_f > t_b else "hbm"
    return cost


def run_bwd(w, args, dev):
    """The backward workload: K ssd_bwd calls over one resident batch (HIP graph replay);
    per-kernel durations from an eager pass with the library's stage events."""
    inp = {k: v.to(dev) for k, v in I.make_workload_inputs(w).items()}
    dout, dfin = I.make_upstream_grads(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.dtype,
                                       seed=500 + w.seed, device=dev)
    out = ssd.ssd_bwd(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"], dout, D=inp["D"],
                      chunk_size=w.chunk, dfinal_state=dfin)
    dims = ssd.make_dims(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, inp["x"].dtype)
    ws = torch.empty(ssd.ssd_bwd_workspace_size(dims, w.chunk), dtype=torch.uint8, device=dev)
    # rotating copies of the per-token inputs and of the outputs, as in the forward benchmark
    per_copy = sum(t.numel() * t.element_size() for t in (inp["x"], inp["dt"], inp["B"], inp["C"], dout))
    per_copy += sum(t.numel() * t.element_size() for t in out.values() if t is not None)
    R = max(1, -(-2 * args.rotate_mb * 2**20 // per_copy)) if args.rotate_mb > 0 else 1
    copies = [(inp, dout, out)] + [({**inp, **{k: inp[k].clone() for k in ("x", "dt", "B", "C")}}, dout.clone(),
                                    {k: (None if t is None else torch.empty_like(t)) for k, t in out.items()})
                                   for _ in range(R - 1)]

    def step(i, evs=None):
        c, dy, o = copies[i % R]
        ssd.ssd_bwd(c["x"], c["dt"], c["dt_bias"], c["A"], c["B"], c["C"], dy, D=c["D"],
                    chunk_size=w.chunk, dfinal_state=dfin, workspace=ws, out=o, stage_events=evs)

    K, W = args.steps, args.warmup
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    use_graph = not args.no_graph
    if use_graph:
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(graph, stream=cap):
            for i in range(K):
                step(W + i)
        torch.cuda.synchronize()
    hev = HipEvents()
    t0, t1 = hev.create(), hev.create()
    wall0 = time.perf_counter()
    hev.record(t0)
    if use_graph:
        graph.replay()
    else:
        for i in range(K):
            step(W + i)
    hev.record(t1)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = hev.elapsed_ms(t0, t1) / K
    events = [[hev.create() for _ in range(20)] for _ in range(K)]
    for i in range(K):
        step(W + i, events[i])
    torch.cuda.synchronize()
    per_kernel_ms = {k: sum(hev.elapsed_ms(ev[2 * i], ev[2 * i + 1]) for ev in events) / K
                     for i, k in enumerate(BWD_STAGES)}
    cost = backward_cost(w)
    kernels = {}
    for k in BWD_STAGES:
        if k.startswith("gate"):
            continue
        t = per_kernel_ms[k] * 1e-3
        c = cost[k]
        if c["bound"] == "mfma":
            ach, peak, unit = c["flops"] / t / 1e12, c["peak"], "TFLOP/s"
        else:
            ach, peak, unit = c["bytes"] / t / 1e9, HBM_PEAK_GBS, "GB/s"
        kernels[k] = {"us": round(per_kernel_ms[k] * 1e3, 3), "bound": c["bound"], "achieved": round(ach, 2),
                      "peak": peak, "unit": unit, "frac": round(ach / peak, 4), "alg_bytes": c["bytes"],
                      "alg_flops": c["flops"]}
    dom = max(kernels, key=lambda k: kernels[k]["us"])
    kd = kernels[dom]
    res = {
        "metric": "SSD backward tokens/sec at 1 MI355X + % of MFMA/HBM roofline",
        "value": round(w.batch * w.seqlen / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) x/B/C/dt/dout/dfinal, log-uniform dt bias, A=-U[1,16])",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "nheads": w.nheads,
                   "headdim": w.headdim, "dstate": w.dstate, "ngroups": w.ngroups, "chunk_size": w.chunk},
        "roofline": {"kernel": dom, "bound": kd["bound"], "achieved": kd["achieved"], "peak": kd["peak"],
                     "unit": kd["unit"], "frac": kd["frac"], "traffic": load_traffic(workload_slug(w.name), dom)},
        "kernels": kernels,
        "launch": ("hip_graph (per-kernel times from an eager pass of the same K steps)" if use_graph
                   else "eager"),
        "input_copies": R,
        "wall_s_timed_region": round(wall, 4),
    }
    hev.close()
    emit(args, dev, res)


def peak_probe(dev):
    """Attainable rates measured on this GPU, to set beside the published peaks the rooflines use:
    register-resident MFMA loops (libssd_peak.so) for the two matrix shapes the kernels issue,
    and a 1 GiB device-to-device copy (read + write bytes per second)."""
    import ctypes
    from state_space_sequence_mamba_amd import build as B
    if not os.path.exists(B.LIB_PEAK):
        raise RuntimeError(f"{B.LIB_PEAK} not found: build it with `python -m state_space_sequence_mamba_amd.build`")
    lib = ctypes.CDLL(B.LIB_PEAK)
    lib.ssd_peak_mfma_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.ssd_peak_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.ssd_peak_mfma_flops.restype = ctypes.c_double
    blocks = 2048
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    res = {}
    for kind, name, iters in ((0, "fp32_mfma_16x16x4_tflops", 10000), (1, "bf16_mfma_16x16x32_tflops", 20000)):
        best = None
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            rc = lib.ssd_peak_mfma_launch(kind, blocks, iters, ctypes.c_void_p(out.data_ptr()),
                                          ctypes.c_void_p(stream))
            e1.record()
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"ssd_peak_mfma_launch({kind}) failed: {rc}")
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        res[name] = round(lib.ssd_peak_mfma_flops(kind, blocks, iters) / (best * 1e-3) / 1e12, 1)
    n = 1024 * 1024 * 1024
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = None
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        best = e0.elapsed_time(e1) if best is None else min(best, e0.elapsed_time(e1))
    res["copy_1gib_gbs"] = round(2 * n / (best * 1e-3) / 1e9, 1)
    del src, dst
    return res


def emit(args, dev, out):
    copy_probe(args, dev)
    if args.peak_probe:
        out["measured_peaks"] = peak_probe(dev)
    print(json.dumps(out), flush=True)


def copy_probe(args, dev):
    """A plain device copy of --copy-probe-mb MiB: the known-size reference of counter runs."""
    if args.copy_probe_mb:
        n = args.copy_probe_mb * 1024 * 1024
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()


def run_conv(w, args, dev):
    """The conv workload: K launches of conv1d_silu over one resident batch (HIP graph replay),
    the carried conv state written every launch."""
    c = I.make_conv_inputs(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.width, w.dtype,
                           w.seed, with_state=True, device=dev)
    H, P, N, G = w.nheads, w.headdim, w.dstate, w.ngroups
    x, B, C, st_out = ssd.conv1d_silu(c["xbc"], c["weight"], c["bias"], H, P, N, G, conv_state=c["conv_state"])

    def step():
        ssd.conv1d_silu(c["xbc"], c["weight"], c["bias"], H, P, N, G, conv_state=c["conv_state"],
                        conv_state_out=st_out, x=x, B=B, C=C)

    K, W = args.steps, args.warmup
    for _ in range(W):
        step()
    torch.cuda.synchronize()
    use_graph = not args.no_graph
    if use_graph:
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(graph, stream=cap):
            for _ in range(K):
                step()
        torch.cuda.synchronize()
    hev = HipEvents()
    t0, t1 = hev.create(), hev.create()
    wall0 = time.perf_counter()
    hev.record(t0)
    if use_graph:
        graph.replay()
    else:
        for _ in range(K):
            step()
    hev.record(t1)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = hev.elapsed_ms(t0, t1) / K
    hev.close()
    e = 2 if w.dtype == "bf16" else 4
    Dc = H * P + 2 * G * N
    KH = w.width - 1
    # input and output once, the state in and out, taps and bias
    alg_bytes = 2 * w.batch * w.seqlen * Dc * e + 2 * w.batch * KH * Dc * e + Dc * (w.width + 1) * 4
    ach = alg_bytes / (ms * 1e-3) / 1e9
    out = {
        "metric": "conv1d+SiLU tokens/sec at 1 MI355X + % of HBM roofline",
        "value": round(w.batch * w.seqlen / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) xBC and state, U(+-1/sqrt(K)) taps and bias)",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "channels": Dc, "width": w.width},
        "roofline": {"kernel": "conv1d_silu", "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(workload_slug(w.name), "conv1d_silu"),
                     "alg_bytes_per_launch": alg_bytes},
        "launch": "hip_graph" if use_graph else "eager",
        "wall_s_timed_region": round(wall, 4),
    }
    emit(args, dev, out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch the timed steps eagerly, not as a HIP graph")
    ap.add_argument("--rotate-mb", type=int, default=256,
                    help="forward steps rotate over copies of x, dt, B, C, y totalling at least twice "
                         "this many MiB, so inputs come from HBM, not the last-level cache (0 = one copy)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="after timing, run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--peak-probe", action="store_true",
                    help="after timing, measure attainable MFMA rates and copy bandwidth (measured_peaks)")
    ap.add_argument("--heads-per-block", type=int, default=0, help="chunk_scan launch shape (0 = built-in)")
    ap.add_argument("--scan-variant", type=int, default=0,
                    help="chunk_scan decomposition: 1 = 64-row blocks, 2 = whole chunks, 0 = built-in")
    ap.add_argument("--rows-group", type=int, default=0,
                    help="chunk_scan row blocks: units per dispatch group on an XCD (0 = built-in, 16)")
    ap.add_argument("--state-path", type=int, default=0,
                    help="chunk states: 1 = chunk_state + state_passing, 2 = one pass over the chunks, "
                         "0 = built-in")
    ap.add_argument("--state-slice", type=int, default=0,
                    help="one-pass chunk states: headdim rows per workgroup (0 = built-in)")
    ap.add_argument("--conv-tokens", type=int, default=0,
                    help="conv1d_silu tokens per thread, a multiple of 4 (0 = built-in)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(see the sharding design for more GPUs)", file=sys.stderr)
        sys.exit(2)
    w = I.workload(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if w.entry == "step":
        run_decode(w, args, dev)
        return
    if w.entry == "bwd":
        run_bwd(w, args, dev)
        return
    if w.entry == "conv":
        if args.conv_tokens:
            ssd.tune_set(3, args.conv_tokens)
        run_conv(w, args, dev)
        return
    if args.heads_per_block:
        ssd.tune_set(0, args.heads_per_block)
    if args.scan_variant:
        ssd.tune_set(2, args.scan_variant)
    if args.rows_group:
        ssd.tune_set(4, args.rows_group)
    if args.state_path:
        ssd.tune_set(5, args.state_path)
    if args.state_slice:
        ssd.tune_set(6, args.state_slice)

    inp = I.make_workload_inputs(w)
    dec = I.make_step_inputs(w.batch, w.nheads, w.headdim, w.dstate, w.ngroups, 1, w.dtype,
                             seed=1000 + w.seed, d_init=w.d_init, device="cpu")
    d = {k: v.to(dev) for k, v in inp.items()}
    dd = {k: v[0].contiguous().to(dev) for k, v in dec.items() if k in ("x", "dt", "B", "C")}
    y = torch.empty_like(d["x"])
    # Consecutive steps read and write rotating copies of the per-token tensors (x, dt, B, C,
    # y), enough of them to exceed the 256 MB last-level cache twice, so that every step reads
    # its inputs from HBM as a fresh batch would
    per_copy = sum(d[k].numel() * d[k].element_size() for k in ("x", "dt", "B", "C")) + y.numel() * y.element_size()
    R = max(1, -(-2 * args.rotate_mb * 2**20 // per_copy)) if args.rotate_mb > 0 else 1
    copies = [{**d, "y": y}] + [{**d, **{k: d[k].clone() for k in ("x", "dt", "B", "C")}, "y": torch.empty_like(y)}
                               for _ in range(R - 1)]
    state = torch.empty(w.batch, w.nheads, w.headdim, w.dstate, dtype=torch.float32, device=dev)
    y_dec = torch.empty_like(dd["x"])
    dims = ssd.make_dims(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, d["x"].dtype)
    ws = torch.empty(ssd.ssd_fwd_workspace_size(dims, w.chunk), dtype=torch.uint8, device=dev)

    K, W = args.steps, args.warmup
    use_graph = not args.no_graph
    hev = HipEvents()
    nev = 8   # start / stop of the forward's three kernels (from their dispatches), 2 around ssd_step
    events = [[hev.create() for _ in range(nev)] for _ in range(max(K, 1))]
    t_start, t_end = hev.create(), hev.create()

    def step(i, evs=None):
        # launches go to the current stream (the capture stream while a graph is captured)
        c = copies[i % R]
        ssd.ssd_fwd(c["x"], c["dt"], c["dt_bias"], c["A"], c["B"], c["C"], c["D"], chunk_size=w.chunk,
                    y=c["y"], final_state=state, workspace=ws, stage_events=None if evs is None else evs[:6])
        if evs is not None:
            hev.record(evs[6])
        ssd.ssd_step(state, dd["x"], dd["dt"], d["dt_bias"], d["A"], dd["B"], dd["C"], d["D"], y=y_dec)
        if evs is not None:
            hev.record(evs[7])

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    if use_graph:
        # the K steps are captured once into a HIP graph; the timed region is one replay
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(graph, stream=cap):
            for i in range(K):
                step(W + i)
        torch.cuda.synchronize()
    wall0 = time.perf_counter()
    hev.record(t_start)
    if use_graph:
        graph.replay()
    else:
        for i in range(K):
            step(W + i)
    hev.record(t_end)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = hev.elapsed_ms(t_start, t_end)
    ms_per_step = total_ms / K

    # Per-kernel durations: the same K steps launched eagerly, each forward kernel timed by a
    # start / stop event pair recorded by its own dispatch (ssd_fwd_timed); ssd_step between
    # two stream events.  Timing events cannot live inside a captured graph on this runtime.
    for i in range(K):
        step(W + i, events[i])
    torch.cuda.synchronize()

    # the one-pass chunk-state path launches no state_passing (its event pair brackets nothing)
    one_pass = ssd.fwd_state_path(dims, w.chunk) == 2
    names = ["chunk_state_seq", None, "chunk_scan", "ssd_step"] if one_pass else KERNELS
    per_kernel_ms = {k: 0.0 for k in names if k}
    pairs = [(0, 1), (2, 3), (4, 5), (6, 7)]
    for evs in events[:K]:
        for k, (a, b) in zip(names, pairs):
            if k:
                per_kernel_ms[k] += hev.elapsed_ms(evs[a], evs[b]) / K

    cost = algorithmic_cost(w)
    kernels = {}
    for k in per_kernel_ms:
        t = per_kernel_ms[k] * 1e-3
        c = cost[k]
        if c["bytes"] == 0 and c["flops"] == 0:       # not launched for this dtype
            continue
        if c["bound"] == "mfma":
            ach, peak, unit = c["flops"] / t / 1e12, MFMA_PEAK_TFLOPS[w.dtype], "TFLOP/s"
        else:
            ach, peak, unit = c["bytes"] / t / 1e9, HBM_PEAK_GBS, "GB/s"
        kernels[k] = {"us": round(per_kernel_ms[k] * 1e3, 3), "bound": c["bound"], "achieved": round(ach, 2),
                      "peak": peak, "unit": unit, "frac": round(ach / peak, 4),
                      "alg_bytes": c["bytes"], "alg_flops": c["flops"]}
    dom = max(kernels, key=lambda k: per_kernel_ms[k])
    kd = kernels[dom]
    # measured HBM bytes per launch of the dominant kernel (FETCH_SIZE + WRITE_SIZE runs,
    # calibrated on a plain copy); None when absent or taken on different kernel sources
    roofline = {"kernel": dom, "bound": kd["bound"], "achieved": kd["achieved"], "peak": kd["peak"],
                "unit": kd["unit"], "frac": kd["frac"], "traffic": load_traffic(workload_slug(w.name), dom)}

    tokens = w.batch * (w.seqlen + 1)
    out = {
        "metric": "SSD scan tokens/sec at 1 MI355X + % of MFMA/HBM roofline",
        "value": round(tokens / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) x/B/C/dt, log-uniform dt bias, A=-U[1,16])",
        "config": {"workload": w.name + " + 1 decode token", "batch": w.batch, "seqlen": w.seqlen,
                   "nheads": w.nheads, "headdim": w.headdim, "dstate": w.dstate, "ngroups": w.ngroups,
                   "chunk_size": w.chunk, "tokens_per_step": tokens},
        "roofline": roofline,
        "kernels": kernels,
        "launch": ("hip_graph (per-kernel times from an eager pass of the same K steps)" if use_graph
                   else "eager"),
        "input_copies": R,
        "wall_s_timed_region": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp, dec, args.cpu_budget)
    emit(args, dev, out)


if __name__ == "__main__":
    main()
