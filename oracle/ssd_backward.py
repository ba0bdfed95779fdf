"""Plain float64 CPU oracle of the SSD scan's gradients (reverse mode).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module; only the test-suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

The pages only gesture at training (the reference-comparison page's training
notes, sections 6-7 of the comprehensive comparison); they give no backward
formulas.  The reading taken: the backward of the scan is the exact gradient of
the forward that ssd_oracle.ssd_recurrence computes (the recurrence of section
3.2 of "Agent 228: MAMBA-2 Reference Implementations Comparison", with the D skip
of Gap 4 and the optional gate and clamp), obtained by running that recurrence
backwards in time.  With the upstream gradients dout = dL/dy (y already gated) and
dfinal = dL/dh_{L-1}, per batch row b and head h (group g):

    dy_t   = dout_t * silu(z_t)                  (dout_t if there is no gate)
    dz_t   = dout_t * y~_t * silu'(z_t)          y~_t: the output before the gate
    G      = dfinal (or 0), then for t = L-1 .. 0:
        G      += dy_t^T C_t                     adjoint of h_t   (P x N)
        dC_t   += dy_t h_t                       (summed over the heads of the group)
        dx_t    = D * dy_t + d_t * G B_t^T
        dB_t   += d_t * x_t G                    (summed over the heads of the group)
        dd_t    = sum(G * (A a_t h_{t-1} + x_t^T B_t))
        dA     += sum(G * d_t a_t h_{t-1})
        dD     += dy_t * x_t
        G       = a_t G                          adjoint of h_{t-1}
    d initial_state = G
    d dt_t    = dd_t * sigmoid(dt_t + dt_bias) * [lo <= d_t <= hi]   (clamp derivative)
    d dt_bias = sum over b, t of d dt_t

with d_t the step, a_t = exp(d_t A) and h_t the forward states (recomputed and kept).
Pinned against central finite differences of ssd_recurrence.
"""
import numpy as np

from .ssd_oracle import _f64, head_groups, silu, softplus

__all__ = ["ssd_recurrence_bwd"]


def _sigmoid(v):
    return 0.5 * (1.0 + np.tanh(0.5 * v))


def ssd_recurrence_bwd(x, dt, dt_bias, A, B, C, dout, D=None, initial_state=None, z=None, dt_limit=None,
                       dfinal=None):
    """Gradients of (y, final_state) of ssd_recurrence against every input.

    dout (Bt, L, H, P): dL/dy;  dfinal (Bt, H, P, N) or None: dL/dfinal_state.
    Returns a dict with dx, ddt, ddt_bias, dA, dB, dC, dD (None without D),
    dinitial_state, dz (None without z); all float64, shaped like their inputs.
    """
    x, dt, dt_bias, A, B, C, dout = map(_f64, (x, dt, dt_bias, A, B, C, dout))
    D, z, dfinal = _f64(D), _f64(z), _f64(dfinal)
    Bt, L, H, P = x.shape
    G_, N = B.shape[2], B.shape[3]
    g = head_groups(H, G_)

    # forward again, keeping every state and the pre-gate output
    raw = dt + dt_bias[None, None, :]                       # (Bt, L, H)
    d = softplus(raw)
    inside = np.ones_like(d)
    if dt_limit is not None:
        inside = ((d >= dt_limit[0]) & (d <= dt_limit[1])).astype(np.float64)
        d = np.clip(d, dt_limit[0], dt_limit[1])
    a = np.exp(d * A[None, None, :])                         # (Bt, L, H)
    hs = np.zeros((L + 1, Bt, H, P, N))                      # hs[t + 1] = h_t, hs[0] = h_{-1}
    if initial_state is not None:
        hs[0] = _f64(initial_state)
    ypre = np.zeros((Bt, L, H, P))
    for t in range(L):
        Bh, Ch = B[:, t][:, g, :], C[:, t][:, g, :]
        hs[t + 1] = a[:, t, :, None, None] * hs[t] + (d[:, t, :, None] * x[:, t])[..., None] * Bh[:, :, None, :]
        ypre[:, t] = (hs[t + 1] * Ch[:, :, None, :]).sum(-1)
        if D is not None:
            ypre[:, t] += D[None] * x[:, t]

    if z is None:
        dy, dz = dout, None
    else:
        s = _sigmoid(z)
        dy = dout * silu(z)
        dz = dout * ypre * s * (1.0 + z * (1.0 - s))

    dx = np.zeros_like(x)
    dd = np.zeros((Bt, L, H))
    dA = np.zeros(H)
    dB = np.zeros_like(B)
    dC = np.zeros_like(C)
    dD = None if D is None else np.zeros_like(D)
    Gs = np.zeros((Bt, H, P, N)) if dfinal is None else dfinal.copy()
    for t in range(L - 1, -1, -1):
        Bh, Ch = B[:, t][:, g, :], C[:, t][:, g, :]         # (Bt, H, N)
        Gs = Gs + dy[:, t][..., None] * Ch[:, :, None, :]   # adjoint of h_t
        dC_h = (dy[:, t][..., None] * hs[t + 1]).sum(axis=2)            # (Bt, H, N)
        GB = (Gs * Bh[:, :, None, :]).sum(-1)                            # (Bt, H, P)
        dx[:, t] = d[:, t, :, None] * GB
        if D is not None:
            dx[:, t] += D[None] * dy[:, t]
            dD += (dy[:, t] * x[:, t]).sum(axis=0)
        xG = (x[:, t][..., None] * Gs).sum(axis=2)                       # (Bt, H, N)
        dB_h = d[:, t, :, None] * xG
        Gh = (Gs * hs[t]).sum(axis=(2, 3))                               # <G, h_{t-1}>  (Bt, H)
        dd[:, t] = A[None, :] * a[:, t] * Gh + (GB * x[:, t]).sum(-1)
        dA += (d[:, t] * a[:, t] * Gh).sum(axis=0)
        for gg in range(G_):
            heads = g == gg
            dB[:, t, gg] += dB_h[:, heads].sum(axis=1)
            dC[:, t, gg] += dC_h[:, heads].sum(axis=1)
        Gs = a[:, t, :, None, None] * Gs                                 # adjoint of h_{t-1}

    ddt = dd * _sigmoid(raw) * inside
    return {"dx": dx, "ddt": ddt, "ddt_bias": ddt.sum(axis=(0, 1)), "dA": dA, "dB": dB, "dC": dC, "dD": dD,
            "dinitial_state": Gs, "dz": dz}
