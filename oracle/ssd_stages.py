"""Float64 staged form of the chunked SSD evaluation (test infrastructure only).

The chunked algorithm of "Agent 228: MAMBA-2 Implementation Gaps", Gap 1
(diagonal block per chunk, off-diagonal block from the carried state, last
state of a chunk carried to the next) and of "Agent 228: MAMBA-2 Reference
Implementations Comparison", section 3.2, split into the four stages the GPU
path also has.  Each stage is written as its defining sum, in float64, with
no blocking beyond the chunking itself.  The tests pin this staged form to
the sequential recurrence in ssd_oracle, and use it to read the GPU
workspace (dt', segment cumsum, chunk states) stage by stage.

Conventions (Q = chunk size, nc = ceil(L / Q); positions past L in the last
chunk are padding):
  dtp  (Bt, H, nc, Q)   softplus(dt + dt_bias), clamped if asked; 0 on padding
  dAcs (Bt, H, nc, Q)   inclusive in-chunk cumsum of dtp * A (flat on padding)
  S    (Bt, nc, H, P, N) state contributed by chunk c alone, decayed to its end
  prev (Bt, nc, H, P, N) state entering chunk c;  final (Bt, H, P, N)
"""
import numpy as np

from .ssd_oracle import _f64, _step_size, head_groups, silu

__all__ = ["chunk_cumsum", "chunk_state", "state_passing", "chunk_scan", "ssd_chunked"]


def _nchunks(L, Q):
    return (L + Q - 1) // Q


def chunk_cumsum(dt, dt_bias, A, Q, dt_limit=None):
    dt, dt_bias, A = map(_f64, (dt, dt_bias, A))
    Bt, L, H = dt.shape
    nc = _nchunks(L, Q)
    dtp = np.zeros((Bt, H, nc, Q))
    dAcs = np.zeros((Bt, H, nc, Q))
    for c in range(nc):
        n = min(Q, L - c * Q)
        d = _step_size(dt[:, c * Q:c * Q + n, :], dt_bias[None, None, :], dt_limit)   # (Bt, n, H)
        dtp[:, :, c, :n] = d.transpose(0, 2, 1)
        run = np.zeros((Bt, H))
        for i in range(Q):
            run = run + dtp[:, :, c, i] * A[None, :]
            dAcs[:, :, c, i] = run
    return dtp, dAcs


def chunk_state(x, B, dtp, dAcs):
    x, B = _f64(x), _f64(B)
    Bt, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    nc, Q = dtp.shape[2], dtp.shape[3]
    g = head_groups(H, G)
    S = np.zeros((Bt, nc, H, P, N))
    for c in range(nc):
        n = min(Q, L - c * Q)
        for i in range(n):
            t = c * Q + i
            w = np.exp(dAcs[:, :, c, Q - 1] - dAcs[:, :, c, i]) * dtp[:, :, c, i]   # (Bt, H)
            S[:, c] += (w[:, :, None] * x[:, t])[:, :, :, None] * B[:, t][:, g, None, :]
    return S


def state_passing(S, dAcs, initial_state=None):
    Bt, nc, H, P, N = S.shape
    Q = dAcs.shape[3]
    h = np.zeros((Bt, H, P, N)) if initial_state is None else _f64(initial_state).copy()
    prev = np.zeros_like(S)
    for c in range(nc):
        prev[:, c] = h
        h = np.exp(dAcs[:, :, c, Q - 1])[:, :, None, None] * h + S[:, c]
    return prev, h


def chunk_scan(x, B, C, dtp, dAcs, prev, D=None, z=None):
    x, B, C = map(_f64, (x, B, C))
    D, z = _f64(D), _f64(z)
    Bt, L, H, P = x.shape
    G = B.shape[2]
    nc, Q = dtp.shape[2], dtp.shape[3]
    g = head_groups(H, G)
    y = np.zeros((Bt, L, H, P))
    for c in range(nc):
        n = min(Q, L - c * Q)
        for i in range(n):
            t = c * Q + i
            Ci = C[:, t][:, g, :]                                           # (Bt, H, N)
            # carried state, decayed to position i
            acc = np.exp(dAcs[:, :, c, i])[:, :, None] * (prev[:, c] * Ci[:, :, None, :]).sum(-1)
            # diagonal block: causal masked "attention" within the chunk
            for j in range(i + 1):
                s = c * Q + j
                cb = (Ci * B[:, s][:, g, :]).sum(-1)                         # (Bt, H)
                w = cb * np.exp(dAcs[:, :, c, i] - dAcs[:, :, c, j]) * dtp[:, :, c, j]
                acc = acc + w[:, :, None] * x[:, s]
            if D is not None:
                acc = acc + D[None] * x[:, t]
            if z is not None:
                acc = acc * silu(z[:, t])
            y[:, t] = acc
    return y


def ssd_chunked(x, dt, dt_bias, A, B, C, D=None, chunk_size=64, initial_state=None, z=None, dt_limit=None):
    """All four stages in order; returns (y, final_state, intermediates dict)."""
    dtp, dAcs = chunk_cumsum(dt, dt_bias, A, chunk_size, dt_limit)
    S = chunk_state(x, B, dtp, dAcs)
    prev, final = state_passing(S, dAcs, initial_state)
    y = chunk_scan(x, B, C, dtp, dAcs, prev, D, z)
    return y, final, {"dtp": dtp, "dAcs": dAcs, "S": S, "prev": prev}
