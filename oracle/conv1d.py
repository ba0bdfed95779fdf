"""Plain float64 CPU oracle of the causal depthwise conv1d + SiLU in front of the scan.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module; only the test-suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

What it computes (sources: "Agent 228: MAMBA-2 Implementation Gaps", Gap 2, and
"Agent 228: MAMBA-2 Reference Implementations Comparison", sections 3.1 and 5.2:
a depthwise conv1d with kernel width K = d_conv = 4, one filter per channel
(groups = channels), padded by K - 1 and cut back to the first L outputs so that
no output sees a later input, followed by SiLU):

    u[t, c]   = bias[c] + sum_{k=0..K-1} w[c, k] * v[t - (K - 1) + k, c]
    out[t, c] = silu(u[t, c]) = u / (1 + exp(-u))

where v[s, c] for s < 0 comes from the carried conv state (the K - 1 inputs before
the sequence; zeros when none is given).  This is cross-correlation in the
framework convention of the pages' conv layers: w[c, K-1] multiplies the current
input.

Readings (listed in the design notes): the conv runs over the channels of
xBC = [x | B | C] (H*P + 2*G*N channels, in that order) and its SiLU output is
split back into x, B and C, as in the data flow of the Mamba-2 block the pages
describe (conv1d -> SiLU -> (x, B, C) -> SSD); the carried conv state holds the
last K - 1 *inputs* (pre-conv, pre-SiLU), oldest first, so that decoding one
token at a time continues the prefill exactly.

Shapes (row-major):
  xbc (Bt, L, Dc)   weight (Dc, K)   bias (Dc) or None
  conv_state (Bt, K-1, Dc) or None   (row j is the input at time j - (K - 1))
"""
import numpy as np

from .ssd_oracle import _f64, silu

__all__ = ["causal_conv1d", "causal_conv1d_silu", "conv1d_silu_step_ref", "split_xbc"]


def _history(conv_state, Bt, K, Dc):
    if conv_state is None:
        return np.zeros((Bt, K - 1, Dc))
    return _f64(conv_state)


def causal_conv1d(xbc, weight, bias=None, conv_state=None):
    """The pre-activation u of the module doc, and the conv state after the last token.

    Written as the defining sum over taps, one output position at a time.
    """
    v, w = _f64(xbc), _f64(weight)
    b = None if bias is None else _f64(bias)
    Bt, L, Dc = v.shape
    K = w.shape[1]
    # inputs at times -(K-1) .. L-1: the carried history, then the sequence
    full = np.concatenate([_history(conv_state, Bt, K, Dc), v], axis=1)
    u = np.zeros((Bt, L, Dc))
    for t in range(L):
        acc = np.zeros((Bt, Dc)) if b is None else np.broadcast_to(b, (Bt, Dc)).copy()
        for k in range(K):
            # input time t - (K - 1) + k sits at index t + k of `full`
            acc = acc + w[None, :, k] * full[:, t + k, :]
        u[:, t] = acc
    new_state = full[:, L:L + K - 1, :].copy()     # inputs at times L-(K-1) .. L-1
    return u, new_state


def causal_conv1d_silu(xbc, weight, bias=None, conv_state=None):
    """silu(causal_conv1d(...)); returns (out (Bt, L, Dc), new conv state (Bt, K-1, Dc))."""
    u, new_state = causal_conv1d(xbc, weight, bias, conv_state)
    return silu(u), new_state


def conv1d_silu_step_ref(conv_state, xbc_t, weight, bias=None):
    """One decode token: out (Bt, Dc) and the shifted conv state (Bt, K-1, Dc)."""
    out, new_state = causal_conv1d_silu(_f64(xbc_t)[:, None, :], weight, bias, conv_state)
    return out[:, 0], new_state


def split_xbc(out, H, P, G, N):
    """Split the conv output's channels into x (.., H, P), B (.., G, N), C (.., G, N)."""
    out = _f64(out)
    lead = out.shape[:-1]
    d_x, d_bc = H * P, G * N
    assert out.shape[-1] == d_x + 2 * d_bc
    x = out[..., :d_x].reshape(*lead, H, P)
    B = out[..., d_x:d_x + d_bc].reshape(*lead, G, N)
    C = out[..., d_x + d_bc:].reshape(*lead, G, N)
    return x, B, C
