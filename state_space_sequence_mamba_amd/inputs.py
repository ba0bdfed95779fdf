"""Seeded synthetic inputs for the SSD scan and the named workloads.

This module draws random numbers and nothing else: it holds none of the
scan's arithmetic, so both the GPU path's tests and the CPU oracle consume
exactly the same tensors.

Distributions (from the Mamba-2 notes' parameter defaults):
  x, B, C, dt_raw ~ N(0, 1)
  dt_bias[h] = the bias that makes softplus(dt_bias) equal to a step drawn
               log-uniformly in [1e-3, 1e-1]  ("Agent 228: MAMBA-2
               Implementation Gaps", Gap 3, dt initialisation; dt_min / dt_max
               defaults in section 5.1 of the reference-comparison page)
  A[h] = -(1 + 15 u), u ~ U[0, 1)   one negative scalar per head
  D    = 1 (skip weight initialised to ones, Gap 4) or N(1, 0.1) per (h, p)

Draw order for a forward workload (CPU generator, fp32 unless stated):
x, B, C, dt_raw, u_dt (f64), u_A (f64), [D noise].  bf16 workloads then round
x, B, C and dt_raw to bf16 (nearest-even, torch's cast).  dt_bias, A and D stay
fp32.
"""
from dataclasses import dataclass
import math

import torch

DT_MIN = 1e-3
DT_MAX = 1e-1


@dataclass(frozen=True)
class Workload:
    name: str
    entry: str            # "fwd", "bwd", "step", "conv" or "norm"
    dtype: str            # "f32" or "bf16" (x, dt, B, C, y)
    batch: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    seed: int
    d_init: str           # "ones" or "normal"
    seqlen: int = 0       # fwd and conv
    chunk: int = 0        # fwd only
    steps: int = 0        # step only
    width: int = 0        # conv only (kernel width)

    @property
    def tokens(self):
        return self.batch * (self.steps if self.entry == "step" else self.seqlen)


# The five workloads the scan is specified on: three forward sizes in the two
# input precisions, a long multi-group sequence, and a 1000-token decode loop.
WORKLOADS = {w.name: w for w in [
    Workload("ssd_fwd f32 B1 L256 H4 P16 N16 G1 Q64", "fwd", "f32", 1, 4, 16, 16, 1, 0, "ones",
             seqlen=256, chunk=64),
    Workload("ssd_fwd f32 B4 L1024 H24 P64 N64 G1 Q256", "fwd", "f32", 4, 24, 64, 64, 1, 1, "ones",
             seqlen=1024, chunk=256),
    Workload("ssd_fwd bf16 B8 L4096 H32 P64 N128 G1 Q256", "fwd", "bf16", 8, 32, 64, 128, 1, 2, "normal",
             seqlen=4096, chunk=256),
    Workload("ssd_step bf16 B256 H80 P64 N128 G1 x1000", "step", "bf16", 256, 80, 64, 128, 1, 3, "ones",
             steps=1000),
    Workload("ssd_fwd bf16 B2 L16384 H80 P64 N128 G8 Q256", "fwd", "bf16", 2, 80, 64, 128, 8, 4, "normal",
             seqlen=16384, chunk=256),
    # the backward of the two forward workloads above (same inputs, seeded upstream gradients)
    Workload("ssd_bwd f32 B4 L1024 H24 P64 N64 G1 Q256", "bwd", "f32", 4, 24, 64, 64, 1, 1, "ones",
             seqlen=1024, chunk=256),
    Workload("ssd_bwd bf16 B8 L4096 H32 P64 N128 G1 Q256", "bwd", "bf16", 8, 32, 64, 128, 1, 2, "normal",
             seqlen=4096, chunk=256),
    # the conv in front of the scan, on the channels of the B8 L4096 bf16 forward (Dc 2304)
    Workload("conv1d_silu bf16 B8 L4096 H32 P64 N128 G1 K4", "conv", "bf16", 8, 32, 64, 128, 1, 5, "ones",
             seqlen=4096, width=4),
    # the gated RMSNorm after the scan, over the B2 L16384 H80 bf16 forward's output (all 80 heads
    # of a token normalised together)
    Workload("gated_rmsnorm bf16 B2 L16384 H80 P64", "norm", "bf16", 2, 80, 64, 128, 1, 6, "ones",
             seqlen=16384),
]}
WORKLOAD_LIST = list(WORKLOADS.values())


def workload(name):
    """One of WORKLOADS, or a forward / backward of another size named the same way, e.g.
    "ssd_fwd bf16 B4 L4096 H32 P64 N128 G1 Q256" (seed 0; D ones for f32, normal for bf16)."""
    if name in WORKLOADS:
        return WORKLOADS[name]
    parts = name.split()
    if len(parts) != 9 or parts[0] not in ("ssd_fwd", "ssd_bwd") or parts[1] not in ("f32", "bf16"):
        raise KeyError(f"unknown workload {name!r}")
    try:
        v = {p[0]: int(p[1:]) for p in parts[2:]}
        return Workload(name, parts[0][4:], parts[1], v["B"], v["H"], v["P"], v["N"], v["G"], 0,
                        "ones" if parts[1] == "f32" else "normal", seqlen=v["L"], chunk=v["Q"])
    except (KeyError, ValueError):
        raise KeyError(f"unknown workload {name!r}") from None


def _torch_dtype(dtype):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def _dt_bias_and_A(u_dt, u_A):
    """dt_bias from a log-uniform step (inverse of softplus), A = -(1 + 15 u)."""
    d = torch.exp(math.log(DT_MIN) + u_dt * (math.log(DT_MAX) - math.log(DT_MIN)))
    dt_bias = d + torch.log(-torch.expm1(-d))
    A = -(1.0 + 15.0 * u_A)
    return dt_bias.float(), A.float()


def make_fwd_inputs(batch, seqlen, nheads, headdim, dstate, ngroups, dtype="f32", seed=0,
                    d_init="ones", device="cpu"):
    """Inputs of one ssd_fwd call, drawn on the CPU and moved to `device`.

    Returns a dict with x (B,L,H,P), dt (B,L,H), dt_bias (H), A (H),
    B and C (B,L,G,N), D (H,P).  x, dt, B, C in `dtype`; the rest fp32.
    """
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn(batch, seqlen, nheads, headdim, generator=g)
    Bm = torch.randn(batch, seqlen, ngroups, dstate, generator=g)
    Cm = torch.randn(batch, seqlen, ngroups, dstate, generator=g)
    dt = torch.randn(batch, seqlen, nheads, generator=g)
    u_dt = torch.rand(nheads, generator=g, dtype=torch.float64)
    u_A = torch.rand(nheads, generator=g, dtype=torch.float64)
    if d_init == "ones":
        D = torch.ones(nheads, headdim)
    elif d_init == "normal":
        D = 1.0 + 0.1 * torch.randn(nheads, headdim, generator=g)
    else:
        raise ValueError(d_init)
    dt_bias, A = _dt_bias_and_A(u_dt, u_A)
    td = _torch_dtype(dtype)
    out = dict(x=x.to(td), dt=dt.to(td), dt_bias=dt_bias, A=A, B=Bm.to(td), C=Cm.to(td), D=D.float())
    return {k: v.to(device) for k, v in out.items()}


def make_gate(shape, dtype="f32", seed=0, device="cpu"):
    """Output-gate input z ~ N(0, 1) of `shape`, from its own CPU generator."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn(*shape, generator=g).to(_torch_dtype(dtype)).to(device)


def make_norm_inputs(batch, seqlen, nheads, headdim, dtype="f32", seed=0, device="cpu"):
    """Inputs of one gated_rmsnorm call: y and z (B,L,H,P) ~ N(0, 1) in `dtype` (the scale of a
    scan output and its gate), weight (H*P,) fp32 ~ 1 + 0.1 N(0, 1) (norm weights near one)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    y = torch.randn(batch, seqlen, nheads, headdim, generator=g)
    z = torch.randn(batch, seqlen, nheads, headdim, generator=g)
    w = 1.0 + 0.1 * torch.randn(nheads * headdim, generator=g)
    td = _torch_dtype(dtype)
    return {"y": y.to(td).to(device), "z": z.to(td).to(device), "weight": w.float().to(device)}


def make_conv_inputs(batch, seqlen, nheads, headdim, dstate, ngroups, width=4, dtype="f32", seed=0,
                     with_state=False, device="cpu"):
    """Inputs of one conv1d_silu call, drawn on the CPU and moved to `device`.

    xbc (B, L, H*P + 2*G*N) ~ N(0, 1) in `dtype`; weight (Dc, K) and bias (Dc) fp32 ~
    U(-1/sqrt(K), 1/sqrt(K)) (the default initialisation of a depthwise conv layer, fan-in K);
    conv_state (B, K-1, Dc) ~ N(0, 1) in `dtype` when asked for, else None.
    """
    g = torch.Generator(device="cpu").manual_seed(seed)
    Dc = nheads * headdim + 2 * ngroups * dstate
    td = _torch_dtype(dtype)
    bound = 1.0 / math.sqrt(width)
    xbc = torch.randn(batch, seqlen, Dc, generator=g).to(td)
    weight = (2.0 * torch.rand(Dc, width, generator=g) - 1.0) * bound
    bias = (2.0 * torch.rand(Dc, generator=g) - 1.0) * bound
    state = torch.randn(batch, width - 1, Dc, generator=g).to(td) if with_state else None
    out = dict(xbc=xbc, weight=weight.float(), bias=bias.float(), conv_state=state)
    return {k: (None if v is None else v.to(device)) for k, v in out.items()}


def make_upstream_grads(batch, seqlen, nheads, headdim, dstate, dtype="f32", seed=0, device="cpu"):
    """Upstream gradients of one ssd_fwd call: dout (B, L, H, P) in `dtype` and dfinal
    (B, H, P, N) fp32, both N(0, 1), from their own CPU generator."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    dout = torch.randn(batch, seqlen, nheads, headdim, generator=g).to(_torch_dtype(dtype))
    dfin = torch.randn(batch, nheads, headdim, dstate, generator=g)
    return dout.to(device), dfin.to(device)


def make_workload_inputs(w, device="cpu"):
    if w.entry not in ("fwd", "bwd"):
        raise ValueError("use make_step_inputs for decode workloads")
    return make_fwd_inputs(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups,
                           w.dtype, w.seed, w.d_init, device)


def make_step_inputs(batch, nheads, headdim, dstate, ngroups, steps, dtype="bf16", seed=3,
                     d_init="ones", device="cpu"):
    """Inputs of a decode loop of `steps` ssd_step calls, drawn with a generator on `device`.

    Returns state0 (B,H,P,N) fp32 ~ N(0,1) and per-step stacks
    x (T,B,H,P), dt (T,B,H), B and C (T,B,G,N) in `dtype`, plus dt_bias, A (H)
    and D (H,P) fp32.  Draw order: state0, then per step x, B, C, dt_raw;
    then u_dt, u_A, [D noise].  Per-step drawing keeps the fp32 transient small.
    """
    dev = torch.device(device)
    g = torch.Generator(device=dev).manual_seed(seed)
    td = _torch_dtype(dtype)
    state0 = torch.randn(batch, nheads, headdim, dstate, generator=g, device=dev)
    xs = torch.empty(steps, batch, nheads, headdim, dtype=td, device=dev)
    Bs = torch.empty(steps, batch, ngroups, dstate, dtype=td, device=dev)
    Cs = torch.empty(steps, batch, ngroups, dstate, dtype=td, device=dev)
    dts = torch.empty(steps, batch, nheads, dtype=td, device=dev)
    for t in range(steps):
        xs[t] = torch.randn(batch, nheads, headdim, generator=g, device=dev).to(td)
        Bs[t] = torch.randn(batch, ngroups, dstate, generator=g, device=dev).to(td)
        Cs[t] = torch.randn(batch, ngroups, dstate, generator=g, device=dev).to(td)
        dts[t] = torch.randn(batch, nheads, generator=g, device=dev).to(td)
    u_dt = torch.rand(nheads, generator=g, dtype=torch.float64, device=dev)
    u_A = torch.rand(nheads, generator=g, dtype=torch.float64, device=dev)
    if d_init == "ones":
        D = torch.ones(nheads, headdim, device=dev)
    else:
        D = 1.0 + 0.1 * torch.randn(nheads, headdim, generator=g, device=dev)
    dt_bias, A = _dt_bias_and_A(u_dt, u_A)
    return dict(state0=state0, x=xs, dt=dts, B=Bs, C=Cs, dt_bias=dt_bias, A=A, D=D.float())
