"""Shared helpers of the tests: error metric, tolerances, oracle calls on sampled slices."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from oracle import ssd_recurrence, ssd_step_ref

# Tolerances on rel_err = max|gpu - oracle| / max|oracle| per output tensor.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.max(np.abs(ref))
    if scale == 0.0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - ref)) / scale)


def p999_rel_err(got, ref, floor=1e-3):
    """99.9th percentile of the elementwise relative error |got - ref| / (|ref| + floor max|ref|)
    (the floor keeps near-zero reference values from dominating); a diagnostic beside rel_err."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref) + floor * max(float(np.max(np.abs(ref))), np.finfo(np.float64).tiny)
    return float(np.percentile(np.abs(got - ref) / den, 99.9))


def to64(t):
    return t.detach().float().cpu().double().numpy()


def dtype_name(t):
    return {torch.float32: "f32", torch.bfloat16: "bf16"}[t.dtype]


def _gather_slices(inp, pairs, initial_state=None):
    """The listed (b, h) slices as the heads of one batch row, each its own group: the oracle
    treats heads (and groups) independently, so one call evaluates every slice exactly."""
    H = inp["x"].shape[2]
    G = inp["B"].shape[2]
    bs = [b for b, _ in pairs]
    hs = [h for _, h in pairs]
    gs = [h // (H // G) for h in hs]
    x = np.stack([to64(inp["x"][b, :, h]) for b, h in pairs], axis=1)[None]           # (1, L, S, P)
    dt = np.stack([to64(inp["dt"][b, :, h]) for b, h in pairs], axis=1)[None]         # (1, L, S)
    Bm = np.stack([to64(inp["B"][b, :, g]) for b, g in zip(bs, gs)], axis=1)[None]    # (1, L, S, N)
    Cm = np.stack([to64(inp["C"][b, :, g]) for b, g in zip(bs, gs)], axis=1)[None]
    bias = to64(inp["dt_bias"])[hs]
    A = to64(inp["A"])[hs]
    D = None if inp.get("D") is None else to64(inp["D"])[hs]
    init = None
    if initial_state is not None:
        init = np.stack([to64(initial_state[b, h]) for b, h in pairs], axis=0)[None]
    return x, dt, bias, A, Bm, Cm, D, init


def oracle_slices(inp, pairs, initial_state=None, workers=4):
    """Oracle y[b, :, h, :] and final_state[b, h] for the listed (b, h) pairs only.

    Each (b, h) depends only on its own x, dt, and its group's B and C (pinned by
    test_batch_and_head_independence), so slicing gives the exact oracle values.  The slices
    are evaluated as the heads of one oracle call per worker thread (numpy releases the GIL
    inside its array operations).
    """
    pairs = list(pairs)
    parts = [pairs[i::workers] for i in range(min(workers, len(pairs)))]

    def run(part):
        x, dt, bias, A, Bm, Cm, D, init = _gather_slices(inp, part, initial_state)
        y, fin = ssd_recurrence(x, dt, bias, A, Bm, Cm, D, initial_state=init)
        return {pr: (y[0, :, k], fin[0, k]) for k, pr in enumerate(part)}

    out = {}
    with ThreadPoolExecutor(len(parts)) as ex:
        for res in ex.map(run, parts):
            out.update(res)
    return out


def oracle_step_slices(inp, pairs, steps, record):
    """Oracle decode loop on sampled (b, h): y at the recorded step indices and the last state."""
    H = inp["x"].shape[2]
    G = inp["B"].shape[2]
    out = {}
    for b, h in pairs:
        g = h // (H // G)
        st = to64(inp["state0"][b:b + 1, h:h + 1])
        ys = {}
        bias = to64(inp["dt_bias"][h:h + 1])
        A = to64(inp["A"][h:h + 1])
        D = to64(inp["D"][h:h + 1])
        xs = to64(inp["x"][:steps, b:b + 1, h:h + 1])
        dts = to64(inp["dt"][:steps, b:b + 1, h:h + 1])
        Bs = to64(inp["B"][:steps, b:b + 1, g:g + 1])
        Cs = to64(inp["C"][:steps, b:b + 1, g:g + 1])
        for t in range(steps):
            y, st = ssd_step_ref(st, xs[t], dts[t], bias, A, Bs[t], Cs[t], D)
            if t in record:
                ys[t] = y[0, 0]
        out[(b, h)] = (ys, st[0, 0])
    return out
