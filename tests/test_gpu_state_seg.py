"""GPU parity of the segmented chunk-state path (chunk_state_seg: each segment of consecutive
chunks from a zero state per (batch, group, slice of heads), state_passing over the segments, the
scan adding each segment's incoming state), through the C ABI, against the float64 oracle and
against the two-launch path (the same sums in another order: agreement to rounding).

The path is forced with launch options (state_path = 3, state_heads, state_chunks) on bf16
chunk-256 P64 N128 shapes that span several segments, 64-token tiles and ragged last chunks.
Bar: rel_err <= 2e-2 (bf16 inputs, fp32 accumulation).
"""
import sys

import numpy as np
import pytest
import torch

from helpers import TOL, oracle_slices, rel_err, to64
from oracle import ssd_recurrence, ssd_stages
from state_space_sequence_mamba_amd import inputs as I
from state_space_sequence_mamba_amd import ssd

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _run(d, opts, init=None, z=None, dt_limit=None):
    y, fin = ssd.ssd_fwd(d["x"], d["dt"], d["dt_bias"], d["A"], d["B"], d["C"], d.get("D"), chunk_size=256,
                         initial_state=init, z=z, dt_limit=dt_limit, opts=opts)
    torch.cuda.synchronize()
    return y, fin


def _seg(hs, sl):
    return {"state_path": 3, "state_heads": hs, "state_chunks": sl}


CASES = [
    # (B, L, H, G, heads per workgroup, chunks per segment)
    (1, 768, 4, 1, 4, 2), (2, 1000, 4, 2, 2, 2), (1, 1300, 5, 1, 5, 2), (2, 2048, 8, 2, 4, 3),
    (1, 2900, 10, 2, 5, 4), (1, 3000, 2, 1, 1, 2), (2, 4096, 8, 1, 2, 4),
]


@pytest.mark.parametrize("Bt,L,H,G,hs,sl", CASES)
def test_segmented_states_match_oracle_and_two_launch_path(Bt, L, H, G, hs, sl):
    _say(f"segmented states B{Bt} L{L} H{H} G{G} hs{hs} SL{sl}")
    inp = I.make_fwd_inputs(Bt, L, H, 64, 128, G, "bf16", seed=500 + L + H, d_init="normal")
    d = {k: v.to(DEV) for k, v in inp.items()}
    dims = ssd.make_dims(Bt, L, H, 64, 128, G, torch.bfloat16)
    assert ssd.fwd_state_path(dims, 256, _seg(hs, sl)) == 3
    y3, f3 = _run(d, _seg(hs, sl))
    y1, f1 = _run(d, {"state_path": 1})
    yr, fr = ssd_recurrence(*(to64(inp[k]) for k in ("x", "dt", "dt_bias", "A", "B", "C", "D")))
    assert np.all(np.isfinite(to64(y3))) and np.all(np.isfinite(to64(f3)))
    assert rel_err(to64(y3), yr) <= TOL["bf16"]
    assert rel_err(to64(f3), fr) <= TOL["bf16"]
    # another order of the same sums (and one more bf16 rounding of the entering states)
    assert rel_err(to64(y3), to64(y1)) <= 1e-2
    assert rel_err(to64(f3), to64(f1)) <= 1e-4


@pytest.mark.parametrize("gate,init,clamp", [(True, False, False), (False, True, False), (True, True, True)])
def test_segmented_states_gate_initial_state_clamp(gate, init, clamp):
    _say(f"segmented states gate={gate} init={init} clamp={clamp}")
    Bt, L, H, G = 2, 1500, 4, 2
    inp = I.make_fwd_inputs(Bt, L, H, 64, 128, G, "bf16", seed=520, d_init="normal")
    d = {k: v.to(DEV) for k, v in inp.items()}
    z = I.make_gate((Bt, L, H, 64), "bf16", seed=521) if gate else None
    h0 = torch.randn(Bt, H, 64, 128, generator=torch.Generator().manual_seed(522)) if init else None
    lim = (0.01, 0.05) if clamp else None
    y, fin = _run(d, _seg(2, 2), init=None if h0 is None else h0.to(DEV), z=None if z is None else z.to(DEV),
                  dt_limit=lim)
    yr, fr = ssd_recurrence(*(to64(inp[k]) for k in ("x", "dt", "dt_bias", "A", "B", "C", "D")),
                            initial_state=None if h0 is None else to64(h0), z=None if z is None else to64(z),
                            dt_limit=lim)
    assert rel_err(to64(y), yr) <= TOL["bf16"]
    assert rel_err(to64(fin), fr) <= TOL["bf16"]


@pytest.mark.parametrize("Aval", [0.0, -1e-3])
def test_segmented_states_weak_decay_long_chain(Aval):
    """The B2 L16384 H80 G8 launch with weak decay: the states carried across all 16 segments of 4
    chunks survive, so an error in any segment's incoming state or decay would show."""
    _say(f"segmented states weak decay A={Aval}")
    Bt, L, H, G = 2, 16384 - 33, 80, 8
    inp = I.make_fwd_inputs(Bt, L, H, 64, 128, G, "bf16", seed=530, d_init="normal")
    inp["A"] = torch.full_like(inp["A"], Aval)
    d = {k: v.to(DEV) for k, v in inp.items()}
    y, fin = _run(d, _seg(5, 4))
    yc, fc = to64(y), to64(fin)
    pairs = [(b, g * 10 + (3 * b + g) % 10) for b in range(Bt) for g in range(G) if (b + g) % 2 == 0]
    for (b, h), (yr, fr) in oracle_slices(inp, pairs).items():
        assert rel_err(yc[b, :, h], yr) <= TOL["bf16"], (b, h)
        assert rel_err(fc[b, h], fr) <= TOL["bf16"], (b, h)


def test_segmented_path_host_choice():
    """Sizes the segmented path cannot take (a single chunk, other shapes, a slice size
    that does not divide the group) keep another path."""
    bf, f32 = torch.bfloat16, torch.float32
    assert ssd.fwd_state_path(ssd.make_dims(2, 256, 8, 64, 128, 1, bf), 256, _seg(4, 2)) != 3     # nc = 1
    assert ssd.fwd_state_path(ssd.make_dims(2, 4096, 8, 64, 64, 1, bf), 256, _seg(4, 2)) != 3     # N = 64
    assert ssd.fwd_state_path(ssd.make_dims(2, 4096, 8, 64, 64, 1, f32), 256, _seg(4, 2)) != 3
    assert ssd.fwd_state_path(ssd.make_dims(2, 4096, 6, 64, 128, 1, bf), 256, _seg(4, 2)) != 3    # 6 % 4
    assert ssd.fwd_state_path(ssd.make_dims(2, 4096, 6, 64, 128, 1, bf), 256, _seg(2, 2)) == 3


def test_segment_intermediates_match_staged_oracle():
    """The workspace after a segmented call: each segment's carried states (bf16, from its own zero
    start), end states (fp32) and exponents, and the states entering the segments, against the
    staged oracle's chunk states run over each segment alone."""
    _say("segment intermediates")
    Bt, L, H, P, N, G, Q, hs, SL = 1, 1500, 4, 64, 128, 2, 256, 2, 2
    inp = I.make_fwd_inputs(Bt, L, H, P, N, G, "bf16", seed=540, d_init="normal")
    d = {k: v.to(DEV) for k, v in inp.items()}
    dims = ssd.make_dims(Bt, L, H, P, N, G, torch.bfloat16)
    ws = torch.zeros(ssd.ssd_fwd_workspace_size(dims, Q), dtype=torch.uint8, device=DEV)
    ssd.ssd_fwd(d["x"], d["dt"], d["dt_bias"], d["A"], d["B"], d["C"], d["D"], chunk_size=Q, workspace=ws,
                opts=_seg(hs, SL))
    torch.cuda.synchronize()
    al = lambda n: (n + 255) // 256 * 256  # noqa: E731
    nc = (L + Q - 1) // Q
    nseg = (nc + SL - 1) // SL
    cum = Bt * H * nc * Q * 4
    n_st = Bt * nc * H * P * N
    n_seg = Bt * nseg * H * P * N
    st_off = 2 * al(cum)
    E = ws[st_off: st_off + n_seg * 4].view(torch.float32).view(Bt, nseg, H, P, N)
    hin = ws[st_off + al(n_seg * 4): st_off + al(n_seg * 4) + n_seg * 2].view(torch.bfloat16).view(Bt, nseg, H, P, N)
    p16_off = st_off + al(n_st * 4)                    # (no C B^T blocks: 2 heads per group)
    prev16 = ws[p16_off: p16_off + n_st * 2].view(torch.bfloat16).view(Bt, nc, H, P, N)
    sg_off = p16_off + al(n_st * 2)
    segdec = ws[sg_off: sg_off + Bt * H * nseg * 4].view(torch.float32).view(Bt, H, nseg)
    cd_off = sg_off + al(Bt * H * nc * 4)
    cdec = ws[cd_off: cd_off + Bt * H * nc * 4].view(torch.float32).view(Bt, H, nc)

    r_dtp, r_dacs = ssd_stages.chunk_cumsum(to64(inp["dt"]), to64(inp["dt_bias"]), to64(inp["A"]), Q)
    S = ssd_stages.chunk_state(to64(inp["x"]), to64(inp["B"]), r_dtp, r_dacs)
    r_prev, _ = ssd_stages.state_passing(S, r_dacs)
    for s in range(nseg):
        c0, c1 = s * SL, min(nc, (s + 1) * SL)
        loc, end = ssd_stages.state_passing(S[:, c0:c1], r_dacs[:, :, c0:c1])
        lasts = r_dacs[:, :, c0:c1, Q - 1]
        assert rel_err(to64(E[:, s]), end) <= TOL["bf16"], s        # (x w rounded to bf16, as on every bf16 path)
        assert abs(float(segdec[0, 0, s]) - float(lasts[0, 0].sum())) <= 1e-4 * max(1.0, abs(float(lasts[0, 0].sum())))
        assert rel_err(to64(segdec[:, :, s]), lasts.sum(axis=2)) <= 1e-5, s
        for c in range(c0, c1):
            assert rel_err(to64(cdec[:, :, c]), lasts[:, :, :c - c0].sum(axis=2)) <= 1e-5 if c > c0 else \
                float(cdec[:, :, c].abs().max()) == 0.0, (s, c)
            if c > c0:
                assert rel_err(to64(prev16[:, c]), loc[:, c - c0]) <= TOL["bf16"], (s, c)
        assert rel_err(to64(hin[:, s]), r_prev[:, c0]) <= TOL["bf16"], s
