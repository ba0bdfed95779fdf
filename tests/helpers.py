"""Shared helpers of the tests: error metric, tolerances, oracle calls on sampled slices."""
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


def to64(t):
    return t.detach().float().cpu().double().numpy()


def dtype_name(t):
    return {torch.float32: "f32", torch.bfloat16: "bf16"}[t.dtype]


def oracle_slices(inp, pairs, initial_state=None):
    """Oracle y[b, :, h, :] and final_state[b, h] for the listed (b, h) pairs only.

    Each (b, h) depends only on its own x, dt, and its group's B and C (pinned by
    test_batch_and_head_independence), so slicing gives the exact oracle values.
    """
    H = inp["x"].shape[2]
    G = inp["B"].shape[2]
    out = {}
    for b, h in pairs:
        g = h // (H // G)
        init = None
        if initial_state is not None:
            init = to64(initial_state[b:b + 1, h:h + 1])
        y, fin = ssd_recurrence(
            to64(inp["x"][b:b + 1, :, h:h + 1]), to64(inp["dt"][b:b + 1, :, h:h + 1]),
            to64(inp["dt_bias"][h:h + 1]), to64(inp["A"][h:h + 1]),
            to64(inp["B"][b:b + 1, :, g:g + 1]), to64(inp["C"][b:b + 1, :, g:g + 1]),
            None if inp.get("D") is None else to64(inp["D"][h:h + 1]), initial_state=init)
        out[(b, h)] = (y[0, :, 0], fin[0, 0])
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
