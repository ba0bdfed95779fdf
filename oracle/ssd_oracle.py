"""Plain float64 CPU oracle for the Mamba-2 SSD scan.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module; only the test-suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

What it computes (per batch row b and head h, with g = g(h) the head's group):

    d_t   = softplus(dt[b,t,h] + dt_bias[h])                 discretised step
    a_t   = exp(d_t * A[h])                                    scalar decay
    h_t   = a_t * h_{t-1} + d_t * x[b,t,h,:]^T B[b,t,g,:]      (P x N) state
    y_t   = h_t C[b,t,g,:]^T + D[h,:] * x[b,t,h,:]             uses the NEW state
    final = h_{L-1},   h_{-1} = initial_state (zeros if not given)

Sources (the five pages of the foxhunt Mamba-2 notes):
  * "Agent 228: MAMBA-2 Reference Implementations Comparison", section 3.2
    "Selective Scan Algorithm": dt' = softplus(dt + dt_bias), decay exp(A*dt'),
    input term B*dt'; section 2.2 "SSD Mathematical Formulation": A is a
    scalar times identity per head, Y = diag(p) M diag(q) X with M a
    1-semiseparable causal mask.
  * "Agent 228: MAMBA-2 Implementation Gaps", Gap 3 (softplus is
    log(1 + e^x), bias added before it), Gap 4 (skip term D * x added to the
    SSM output), Gap 1 (the chunked diagonal / off-diagonal evaluation).
  * "MAMBA2 Inference Optimization Report", Step 4: the last state is kept as
    the hidden state for stateful inference (here: final_state / ssd_step).

Optional terms: an output gate y * silu(z) ("Agent 228: MAMBA-2 Reference
Implementations Comparison", section 3.1 forward pass and section 6.1, output
gating, applied to the scan output including the D term), and a clamp of dt' to
[dt_min, dt_max] after the softplus (section 5.2 of the same page; Gap 3).

Readings taken where the pages are silent or disagree (each listed in the
design notes): no dt clamp unless asked for; the bias is always added; A is used exactly as
given (callers pass negative values); B is discretised by Euler (B * dt'),
not exact zero-order hold; D has one value per (head, channel); head h uses
group h // (H / G); the partial last chunk is processed; C is per token.

Shapes (row-major):
  x (Bt, L, H, P)   dt (Bt, L, H)   dt_bias (H)   A (H)
  B, C (Bt, L, G, N)   D (H, P) or None   initial_state (Bt, H, P, N) or None
"""
import numpy as np

__all__ = [
    "softplus",
    "silu",
    "head_groups",
    "ssd_recurrence",
    "ssd_step_ref",
    "ssd_quadratic",
]


def _f64(a):
    """Upcast any array-like (numpy or CPU torch tensor, bf16 included) to float64 exactly."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor: bf16 -> f32 is exact, f32 -> f64 is exact
        a = a.detach().cpu().float().numpy()
    return np.asarray(a, dtype=np.float64)


def softplus(v):
    """log(1 + e^v) in float64 (Gap 3 of the implementation-gaps page).

    np.logaddexp(0, v) evaluates exactly this without overflow for large v.
    """
    return np.logaddexp(0.0, v)


def silu(v):
    """v * sigmoid(v) = v / (1 + e^-v), the gate nonlinearity (float64)."""
    return v / (1.0 + np.exp(-v))


def _step_size(dt_raw, bias, dt_limit):
    d = softplus(dt_raw + bias)
    if dt_limit is not None:
        d = np.clip(d, dt_limit[0], dt_limit[1])
    return d


def head_groups(H, G):
    """Group index of each head: contiguous blocks of H/G heads share B and C."""
    if G < 1 or H % G != 0:
        raise ValueError("nheads must be a multiple of ngroups")
    return np.arange(H) // (H // G)


def ssd_recurrence(x, dt, dt_bias, A, B, C, D=None, initial_state=None, z=None, dt_limit=None):
    """Sequential float64 evaluation of the SSD recurrence, one time step at a time.

    z (Bt,L,H,P) or None: output gate, y <- y * silu(z).  dt_limit (lo, hi) or None: clamp of dt'.
    Returns (y (Bt,L,H,P), final_state (Bt,H,P,N)), both float64.
    """
    x, dt, dt_bias, A, B, C = map(_f64, (x, dt, dt_bias, A, B, C))
    D, z = _f64(D), _f64(z)
    Bt, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    g = head_groups(H, G)
    if initial_state is None:
        h = np.zeros((Bt, H, P, N))
    else:
        h = _f64(initial_state).copy()
    y = np.zeros((Bt, L, H, P))
    for t in range(L):
        d = _step_size(dt[:, t, :], dt_bias[None, :], dt_limit)  # (Bt, H)
        a = np.exp(d * A[None, :])                              # (Bt, H)
        Bt_h = B[:, t][:, g, :]                                 # (Bt, H, N)
        Ct_h = C[:, t][:, g, :]                                 # (Bt, H, N)
        xt = x[:, t]                                            # (Bt, H, P)
        h = a[:, :, None, None] * h + (d[:, :, None] * xt)[:, :, :, None] * Bt_h[:, :, None, :]
        yt = (h * Ct_h[:, :, None, :]).sum(axis=-1)             # (Bt, H, P)
        if D is not None:
            yt = yt + D[None, :, :] * xt
        if z is not None:
            yt = yt * silu(z[:, t])
        y[:, t] = yt
    return y, h


def ssd_step_ref(state, x, dt, dt_bias, A, B, C, D=None, z=None, dt_limit=None):
    """One step of the recurrence on a given state (single-token decode).

    state (Bt,H,P,N), x (Bt,H,P), dt (Bt,H), B and C (Bt,G,N), z (Bt,H,P) or None.
    Returns (y (Bt,H,P), new_state (Bt,H,P,N)), float64; y reads the updated state.
    """
    y, new_state = ssd_recurrence(
        _f64(x)[:, None], _f64(dt)[:, None], dt_bias, A,
        _f64(B)[:, None], _f64(C)[:, None], D, initial_state=state,
        z=None if z is None else _f64(z)[:, None], dt_limit=dt_limit,
    )
    return y[:, 0], new_state


def ssd_quadratic(x, dt, dt_bias, A, B, C, D=None, z=None, dt_limit=None):
    """Brute-force materialised form y = ((L o C B^T) X + D x) * silu(z), zero initial state.

    For every (b, h) it builds the L x L matrix
        M[t, s] = (C_t . B_s) * exp(sum_{k=s+1..t} d_k A) * d_s   for s <= t, else 0
    (the 1-semiseparable causal mask of section 2.2 of the reference-comparison
    page, times the C B^T "attention" scores) and multiplies it by X.
    The decay exponent is summed term by term, not taken as a cumsum difference.
    Small inputs only: O(L^2 (N + P + L)) per head.
    """
    x, dt, dt_bias, A, B, C = map(_f64, (x, dt, dt_bias, A, B, C))
    D, z = _f64(D), _f64(z)
    Bt, L, H, P = x.shape
    G = B.shape[2]
    g = head_groups(H, G)
    y = np.zeros((Bt, L, H, P))
    for b in range(Bt):
        for hh in range(H):
            d = _step_size(dt[b, :, hh], dt_bias[hh], dt_limit)    # (L,)
            dA = d * A[hh]
            M = np.zeros((L, L))
            for t in range(L):
                for s in range(t + 1):
                    decay = np.exp(np.sum(dA[s + 1:t + 1]))
                    M[t, s] = np.dot(C[b, t, g[hh]], B[b, s, g[hh]]) * decay * d[s]
            y[b, :, hh, :] = M @ x[b, :, hh, :]
            if D is not None:
                y[b, :, hh, :] += D[hh][None, :] * x[b, :, hh, :]
            if z is not None:
                y[b, :, hh, :] *= silu(z[b, :, hh, :])
    return y
