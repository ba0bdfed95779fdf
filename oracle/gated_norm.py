"""Plain float64 CPU oracle of the gated RMSNorm after the scan.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module; only the test-suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

What it computes (sources: "Agent 228: MAMBA-2 Reference Implementations
Comparison", section 7.3, item 9 -- the output gate y * silu(z) -- and item 11 --
an RMSNorm in front of the final projection, as the reference model has): the
gated scan output is normalised by its root mean square over each token's
channels and scaled per channel,

    g[t, c]   = y[t, c] * silu(z[t, c])            (g = y without a gate)
    rms[t]    = sqrt( mean_{c in the group} g[t, c]^2 + eps )
    out[t, c] = g[t, c] / rms[t] * weight[c]

Readings (listed in the design notes): the pages name the norm but not its
extent; the plain reading is one RMSNorm over the token's d_inner = H * P
channels (norm_heads = H).  norm_heads < H normalises groups of norm_heads
consecutive heads (norm_heads * P channels) separately, the grouped form a
model with several B/C groups may use; the gate is applied before the norm.

Shapes (row-major): y, z (Bt, L, H, P); weight (H * P,); out (Bt, L, H, P).
"""
import numpy as np

from .ssd_oracle import _f64, silu

__all__ = ["gated_rmsnorm"]


def gated_rmsnorm(y, z, weight, eps=1e-5, norm_heads=None):
    """out = g / sqrt(mean(g^2) + eps) * weight over groups of norm_heads heads, g = y silu(z)."""
    y = _f64(y)
    Bt, L, H, P = y.shape
    nh = H if norm_heads is None else int(norm_heads)
    assert 1 <= nh <= H and H % nh == 0, "norm_heads must divide the number of heads"
    g = y if z is None else y * silu(_f64(z))
    w = _f64(weight).reshape(H, P)
    out = np.empty_like(g)
    for b in range(Bt):
        for t in range(L):
            for h0 in range(0, H, nh):
                v = g[b, t, h0:h0 + nh]                      # (nh, P): one group of channels
                rms = np.sqrt(np.mean(v * v) + eps)
                out[b, t, h0:h0 + nh] = v / rms * w[h0:h0 + nh]
    return out
