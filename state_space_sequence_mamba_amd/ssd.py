"""Thin Python binding of libssd.so (include/ssd.h).

Argument marshalling only: torch supplies device memory and the stream; every step of
the scan runs in the library's HIP kernels.  There is no fallback: if libssd.so is
missing or cannot be loaded, every call raises.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SSD_LIBRARY names another build of the same library (the host-sanitized one the CPU tests load)
LIB_PATH = os.environ.get("SSD_LIBRARY") or os.path.join(_HERE, "libssd.so")

(SSD_OK, SSD_ERR_INVALID_ARG, SSD_ERR_UNSUPPORTED, SSD_ERR_DEVICE_PTR, SSD_ERR_WORKSPACE, SSD_ERR_HIP,
 SSD_ERR_SCRATCH_LIMIT) = range(7)
NOALLOC_SCRATCH_BYTES = 64 << 20      # SSD_FWD_NOALLOC_SCRATCH_BYTES of include/ssd.h
SSD_F32, SSD_BF16 = 0, 1

_DTYPES = {torch.float32: SSD_F32, torch.bfloat16: SSD_BF16}


class ssd_dims_t(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("dt_min", ctypes.c_float), ("dt_max", ctypes.c_float)]


class ssd_launch_opts_t(ctypes.Structure):
    """Launch-shape options of the measurement entry points (include/ssd_tuning.h); 0 = built-in."""
    _fields_ = [("scan_variant", ctypes.c_int32), ("heads_per_block", ctypes.c_int32),
                ("min_blocks", ctypes.c_int32), ("rows_group", ctypes.c_int32), ("state_path", ctypes.c_int32),
                ("state_slice", ctypes.c_int32), ("conv_tokens", ctypes.c_int32), ("state_heads", ctypes.c_int32),
                ("state_chunks", ctypes.c_int32), ("bwd_heads", ctypes.c_int32)]


def launch_opts(**fields):
    """An ssd_launch_opts_t with the named fields set (every other field 0 = built-in)."""
    o = ssd_launch_opts_t()
    for k, v in fields.items():
        if k not in dict(ssd_launch_opts_t._fields_):
            raise KeyError(f"unknown launch option {k!r}")
        setattr(o, k, int(v))
    return o


def _opts_ref(opts):
    if opts is None:
        return None
    if isinstance(opts, dict):
        opts = launch_opts(**opts)
    return ctypes.byref(opts)


class SsdError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {ssd_status_string(status)} (status {status})")


_lib = None


def load_library():
    """Load libssd.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} not found: build it with `python -m state_space_sequence_mamba_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, f32p, i32, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    dims_p = ctypes.POINTER(ssd_dims_t)
    norm_args = [dims_p, vp, vp, f32p, ctypes.c_float, i32, vp, vp]
    lib.ssd_gated_rmsnorm.argtypes = norm_args
    lib.ssd_gated_rmsnorm.restype = i32
    lib.ssd_gated_rmsnorm_ex.argtypes = norm_args + [vp]
    lib.ssd_gated_rmsnorm_ex.restype = i32
    lib.ssd_fwd_workspace_size.argtypes = [dims_p, i32]
    lib.ssd_fwd_workspace_size.restype = sz
    fwd_args = [dims_p, vp, vp, f32p, f32p, vp, vp, f32p, vp, i32, f32p, vp, f32p, vp, sz, vp]
    lib.ssd_fwd.argtypes = fwd_args
    lib.ssd_fwd.restype = i32
    lib.ssd_fwd_noalloc.argtypes = [dims_p, vp, vp, f32p, f32p, vp, vp, f32p, vp, i32, f32p, vp, f32p, vp]
    lib.ssd_fwd_noalloc.restype = i32
    opts_p = ctypes.POINTER(ssd_launch_opts_t)
    lib.ssd_fwd_ex.argtypes = fwd_args + [opts_p, vp]
    lib.ssd_fwd_ex.restype = i32
    step_args = [dims_p, f32p, vp, vp, f32p, f32p, vp, vp, f32p, vp, vp, vp]
    lib.ssd_step.argtypes = step_args
    lib.ssd_step.restype = i32
    lib.ssd_step_ex.argtypes = step_args + [vp]
    lib.ssd_step_ex.restype = i32
    lib.ssd_bwd_workspace_size.argtypes = [dims_p, i32, i32]
    lib.ssd_bwd_workspace_size.restype = sz
    bwd_args = [dims_p, vp, vp, f32p, f32p, vp, vp, f32p, vp, i32, f32p, vp, f32p,
                vp, vp, f32p, f32p, vp, vp, f32p, vp, f32p, vp, sz, vp]
    lib.ssd_bwd.argtypes = bwd_args
    lib.ssd_bwd.restype = i32
    lib.ssd_bwd_ex.argtypes = bwd_args + [opts_p, vp]
    lib.ssd_bwd_ex.restype = i32
    conv_args = [dims_p, i32, vp, f32p, f32p, vp, vp, vp, vp, vp, vp]
    lib.ssd_conv1d_silu.argtypes = conv_args
    lib.ssd_conv1d_silu.restype = i32
    lib.ssd_conv1d_silu_ex.argtypes = conv_args + [opts_p]
    lib.ssd_conv1d_silu_ex.restype = i32
    lib.ssd_conv1d_silu_step.argtypes = [dims_p, i32, vp, vp, f32p, f32p, vp, vp, vp, vp]
    lib.ssd_conv1d_silu_step.restype = i32
    lib.ssd_status_string.argtypes = [i32]
    lib.ssd_status_string.restype = ctypes.c_char_p
    lib.ssd_fwd_state_path.argtypes = [dims_p, i32, opts_p]
    lib.ssd_fwd_state_segment_chunks.argtypes = [dims_p, i32, opts_p]
    lib.ssd_fwd_state_segment_chunks.restype = i32
    lib.ssd_fwd_state_path.restype = i32
    lib.ssd_bwd_heads.argtypes = lib.ssd_fwd_state_path.argtypes
    lib.ssd_bwd_heads.restype = i32
    _lib = lib
    return lib


def ssd_status_string(status):
    return load_library().ssd_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def make_dims(batch, seqlen, nheads, headdim, dstate, ngroups, dtype, dt_limit=None):
    """dt_limit = (dt_min, dt_max) clamps dt' = softplus(dt + dt_bias); None = no clamp."""
    code = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    lo, hi = (0.0, 0.0) if dt_limit is None else (float(dt_limit[0]), float(dt_limit[1]))
    return ssd_dims_t(batch, seqlen, nheads, headdim, dstate, ngroups, code, lo, hi)


def ssd_fwd_workspace_size(dims, chunk_size):
    return int(load_library().ssd_fwd_workspace_size(ctypes.byref(dims), int(chunk_size)))


def _check_fwd_shapes(x, dt, dt_bias, A, B, C, D, initial_state, z=None):
    if x.dim() != 4 or dt.dim() != 3 or B.dim() != 4 or C.dim() != 4:
        raise ValueError("x (B,L,H,P), dt (B,L,H), B and C (B,L,G,N) expected")
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if tuple(dt.shape) != (b, L, H) or tuple(B.shape) != (b, L, G, N) or tuple(C.shape) != (b, L, G, N):
        raise ValueError("inconsistent x / dt / B / C shapes")
    if tuple(dt_bias.shape) != (H,) or tuple(A.shape) != (H,):
        raise ValueError("dt_bias and A must have shape (H,)")
    if D is not None and tuple(D.shape) != (H, P):
        raise ValueError("D must have shape (H, P)")
    if initial_state is not None and tuple(initial_state.shape) != (b, H, P, N):
        raise ValueError("initial_state must have shape (B, H, P, N)")
    if z is not None and tuple(z.shape) != tuple(x.shape):
        raise ValueError("z must have the shape of x")
    for t in (dt, B, C, z):
        if t is not None and t.dtype != x.dtype:
            raise ValueError("x, dt, B, C and z must share one dtype")
    for t in (dt_bias, A, D, initial_state):
        if t is not None and t.dtype != torch.float32:
            raise ValueError("dt_bias, A, D and initial_state must be float32")
    for t in (x, dt, dt_bias, A, B, C, D, initial_state, z):
        if t is not None and not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    return b, L, H, P, N, G


def ssd_fwd(x, dt, dt_bias, A, B, C, D=None, chunk_size=256, initial_state=None, y=None,
            final_state=None, return_final_state=True, workspace=None, stream=None, stage_events=None,
            z=None, dt_limit=None, opts=None):
    """Chunked SSD forward.  Returns (y, final_state) (final_state is None if not requested).

    `z` (shape of x) gates the output, y * silu(z); `dt_limit` = (dt_min, dt_max) clamps dt'.
    Output and workspace tensors are allocated with torch when not given.  `stage_events`
    (6 raw hipEvent_t handles as ints: start and stop of each of the three kernels) and `opts`
    (launch options: a dict of ssd_launch_opts_t fields or the struct) select ssd_fwd_ex.
    """
    b, L, H, P, N, G = _check_fwd_shapes(x, dt, dt_bias, A, B, C, D, initial_state, z)
    dims = make_dims(b, L, H, P, N, G, x.dtype, dt_limit)
    lib = load_library()
    if y is None:
        y = torch.empty_like(x)
    if final_state is None and return_final_state:
        final_state = torch.empty(b, H, P, N, dtype=torch.float32, device=x.device)
    ws_bytes = ssd_fwd_workspace_size(dims, chunk_size)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    args = [ctypes.byref(dims), _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
            _ptr(z), int(chunk_size), _ptr(initial_state), _ptr(y), _ptr(final_state), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream)]
    if stage_events is None and opts is None:
        st = lib.ssd_fwd(*args)
    else:
        arr = None if stage_events is None else (ctypes.c_void_p * 6)(*stage_events)
        st = lib.ssd_fwd_ex(*args, _opts_ref(opts), arr)
    if st != SSD_OK:
        raise SsdError(st, "ssd_fwd")
    return y, final_state


def ssd_fwd_noalloc(x, dt, dt_bias, A, B, C, D=None, chunk_size=256, initial_state=None, y=None, final_state=None,
                    stream=None, z=None, dt_limit=None):
    """ssd_fwd with the library's fixed scratch as its workspace (ssd_fwd_noalloc: no device
    allocation in the call).  y and final_state must be given (the binding allocates nothing
    either); returns (y, final_state)."""
    b, L, H, P, N, G = _check_fwd_shapes(x, dt, dt_bias, A, B, C, D, initial_state, z)
    if y is None:
        raise ValueError("ssd_fwd_noalloc: pass y (the call allocates nothing)")
    dims = make_dims(b, L, H, P, N, G, x.dtype, dt_limit)
    st = load_library().ssd_fwd_noalloc(ctypes.byref(dims), _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(B),
                                        _ptr(C), _ptr(D), _ptr(z), int(chunk_size), _ptr(initial_state), _ptr(y),
                                        _ptr(final_state), _stream(stream))
    if st != SSD_OK:
        raise SsdError(st, "ssd_fwd_noalloc")
    return y, final_state


def ssd_step(state, x, dt, dt_bias, A, B, C, D=None, y=None, stream=None, z=None, dt_limit=None, events=None):
    """One decode step: updates `state` (B,H,P,N) fp32 in place and returns y (B,H,P).

    `z` (B,H,P) gates the output, y * silu(z); `dt_limit` = (dt_min, dt_max) clamps dt'.
    `events` (2 raw hipEvent_t handles: start and stop of the step's kernel) selects ssd_step_ex.
    """
    if state.dim() != 4 or x.dim() != 3 or dt.dim() != 2 or B.dim() != 3 or C.dim() != 3:
        raise ValueError("state (B,H,P,N), x (B,H,P), dt (B,H), B and C (B,G,N) expected")
    b, H, P, N = state.shape
    G = B.shape[1]
    if tuple(x.shape) != (b, H, P) or tuple(dt.shape) != (b, H) or tuple(B.shape) != (b, G, N) \
            or tuple(C.shape) != (b, G, N):
        raise ValueError("inconsistent state / x / dt / B / C shapes")
    if z is not None and tuple(z.shape) != (b, H, P):
        raise ValueError("z must have the shape of x")
    if state.dtype != torch.float32:
        raise ValueError("state must be float32")
    for t in (dt, B, C, z):
        if t is not None and t.dtype != x.dtype:
            raise ValueError("x, dt, B, C and z must share one dtype")
    for t in (state, x, dt, dt_bias, A, B, C, D, z):
        if t is not None and not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    dims = make_dims(b, 1, H, P, N, G, x.dtype, dt_limit)
    if y is None:
        y = torch.empty_like(x)
    args = [ctypes.byref(dims), _ptr(state), _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
            _ptr(z), _ptr(y), _stream(stream)]
    lib = load_library()
    if events is None:
        st = lib.ssd_step(*args)
    else:
        st = lib.ssd_step_ex(*args, (ctypes.c_void_p * 2)(*events))
    if st != SSD_OK:
        raise SsdError(st, "ssd_step")
    return y


def gated_rmsnorm(y, weight, z=None, eps=1e-5, norm_heads=None, out=None, stream=None, events=None):
    """out = g / sqrt(mean(g^2) + eps) * weight, g = y * silu(z) (g = y without z), over each token's
    channels in groups of `norm_heads` heads (default: all H heads).

    y, z, out: (B, L, H, P) or, for one decode token, (B, H, P), one dtype; weight (H*P,) float32.
    `out` may be `y` itself.  `events` (2 raw hipEvent_t handles) selects ssd_gated_rmsnorm_ex.
    """
    if y.dim() not in (3, 4):
        raise ValueError("y (B, L, H, P) or (B, H, P) expected")
    b, L, H, P = (y.shape[0], 1, y.shape[1], y.shape[2]) if y.dim() == 3 else tuple(y.shape)
    if z is not None and (z.shape != y.shape or z.dtype != y.dtype):
        raise ValueError("z must have y's shape and dtype")
    if weight.dtype != torch.float32 or weight.numel() != H * P:
        raise ValueError("weight (H*P,) float32 expected")
    for t in (y, z, weight, out):
        if t is not None and not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if out is None:
        out = torch.empty_like(y)
    elif out.shape != y.shape or out.dtype != y.dtype:
        raise ValueError("out must have y's shape and dtype")
    N = 64 if y.dtype == torch.float32 else 128            # (not used by the norm; any supported size)
    dims = make_dims(b, L, H, P, N, 1, y.dtype)
    args = [ctypes.byref(dims), _ptr(y), _ptr(z), _ptr(weight), ctypes.c_float(eps),
            int(H if norm_heads is None else norm_heads), _ptr(out), _stream(stream)]
    lib = load_library()
    st = lib.ssd_gated_rmsnorm(*args) if events is None else \
        lib.ssd_gated_rmsnorm_ex(*args, (ctypes.c_void_p * 2)(*events))
    if st != SSD_OK:
        raise SsdError(st, "ssd_gated_rmsnorm")
    return out


def ssd_bwd_workspace_size(dims, chunk_size, with_gate=False):
    return int(load_library().ssd_bwd_workspace_size(ctypes.byref(dims), int(chunk_size), int(bool(with_gate))))


def ssd_bwd(x, dt, dt_bias, A, B, C, dout, D=None, chunk_size=256, initial_state=None, dfinal_state=None,
            z=None, dt_limit=None, want_dD=True, want_dinitial_state=True, workspace=None, stream=None,
            out=None, stage_events=None, opts=None):
    """Gradients of ssd_fwd.  Returns a dict: dx, ddt, ddt_bias, dA, dB, dC, dD, dz, dinitial_state
    (dD / dz / dinitial_state are None when not requested or not applicable).  `out` reuses a
    previous call's dict as the output buffers; `stage_events` (20 raw hipEvent_t handles as
    ints: start and stop of each of the ten stages) selects the timed entry point."""
    b, L, H, P, N, G = _check_fwd_shapes(x, dt, dt_bias, A, B, C, D, initial_state, z)
    if tuple(dout.shape) != tuple(x.shape) or dout.dtype != x.dtype or not dout.is_contiguous():
        raise ValueError("dout must be a contiguous tensor shaped and typed like x")
    if dfinal_state is not None and (tuple(dfinal_state.shape) != (b, H, P, N) or
                                     dfinal_state.dtype != torch.float32 or not dfinal_state.is_contiguous()):
        raise ValueError("dfinal_state must be a contiguous (B, H, P, N) float32 tensor")
    dims = make_dims(b, L, H, P, N, G, x.dtype, dt_limit)
    f32 = dict(dtype=torch.float32, device=x.device)
    if out is None:
        out = {"dx": torch.empty_like(x), "ddt": torch.empty_like(dt), "ddt_bias": torch.empty(H, **f32),
               "dA": torch.empty(H, **f32), "dB": torch.empty_like(B), "dC": torch.empty_like(C),
               "dD": torch.empty(H, P, **f32) if want_dD else None,
               "dz": torch.empty_like(z) if z is not None else None,
               "dinitial_state": torch.empty(b, H, P, N, **f32) if want_dinitial_state else None}
    ws_bytes = ssd_bwd_workspace_size(dims, chunk_size, z is not None)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    lib = load_library()
    args = [
        ctypes.byref(dims), _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
        int(chunk_size), _ptr(initial_state), _ptr(dout), _ptr(dfinal_state), _ptr(out["dx"]), _ptr(out["ddt"]),
        _ptr(out["ddt_bias"]), _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dz"]),
        _ptr(out["dinitial_state"]), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)]
    if stage_events is None and opts is None:
        st = lib.ssd_bwd(*args)
    else:
        arr = None if stage_events is None else (ctypes.c_void_p * 20)(*stage_events)
        st = lib.ssd_bwd_ex(*args, _opts_ref(opts), arr)
    if st != SSD_OK:
        raise SsdError(st, "ssd_bwd")
    return out


def _check_conv(xbc, weight, bias, lead, nheads, headdim, dstate, ngroups):
    Dc = nheads * headdim + 2 * ngroups * dstate
    if xbc.shape[-1] != Dc:
        raise ValueError(f"xbc has {xbc.shape[-1]} channels, H*P + 2*G*N = {Dc}")
    if weight.dim() != 2 or weight.shape[0] != Dc:
        raise ValueError("weight must have shape (Dc, K)")
    if bias is not None and tuple(bias.shape) != (Dc,):
        raise ValueError("bias must have shape (Dc,)")
    for t in (weight, bias):
        if t is not None and t.dtype != torch.float32:
            raise ValueError("weight and bias must be float32")
    for t in (xbc, weight, bias):
        if t is not None and not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    return Dc, weight.shape[1]


def _conv_outputs(xbc, lead, nheads, headdim, dstate, ngroups, x, B, C):
    kw = dict(dtype=xbc.dtype, device=xbc.device)
    if x is None:
        x = torch.empty(*lead, nheads, headdim, **kw)
    if B is None:
        B = torch.empty(*lead, ngroups, dstate, **kw)
    if C is None:
        C = torch.empty(*lead, ngroups, dstate, **kw)
    for t, shp in ((x, (*lead, nheads, headdim)), (B, (*lead, ngroups, dstate)), (C, (*lead, ngroups, dstate))):
        if tuple(t.shape) != shp or t.dtype != xbc.dtype or not t.is_contiguous():
            raise ValueError("x / B / C outputs: wrong shape, dtype or layout")
    return x, B, C


def conv1d_silu(xbc, weight, bias, nheads, headdim, dstate, ngroups, conv_state=None, conv_state_out=None,
                return_conv_state=True, x=None, B=None, C=None, stream=None, opts=None):
    """Causal depthwise conv1d + SiLU over xbc (B, L, H*P + 2*G*N), split into x, B, C.

    weight (Dc, K) and bias (Dc,) are float32; conv_state (B, K-1, Dc) in xbc's dtype holds the
    K-1 inputs before the sequence.  Returns (x, B, C, conv_state_out); conv_state_out may be
    `conv_state` itself (in-place update).
    """
    if xbc.dim() != 3:
        raise ValueError("xbc (B, L, Dc) expected")
    b, L, _ = xbc.shape
    Dc, K = _check_conv(xbc, weight, bias, (b, L), nheads, headdim, dstate, ngroups)
    for t in (conv_state, conv_state_out):
        if t is not None and (tuple(t.shape) != (b, K - 1, Dc) or t.dtype != xbc.dtype or not t.is_contiguous()):
            raise ValueError("conv state must be a contiguous (B, K-1, Dc) tensor of xbc's dtype")
    x, B, C = _conv_outputs(xbc, (b, L), nheads, headdim, dstate, ngroups, x, B, C)
    if conv_state_out is None and return_conv_state:
        conv_state_out = torch.empty(b, K - 1, Dc, dtype=xbc.dtype, device=xbc.device)
    dims = make_dims(b, L, nheads, headdim, dstate, ngroups, xbc.dtype)
    args = [ctypes.byref(dims), int(K), _ptr(xbc), _ptr(weight), _ptr(bias), _ptr(conv_state),
            _ptr(conv_state_out), _ptr(x), _ptr(B), _ptr(C), _stream(stream)]
    lib = load_library()
    st = lib.ssd_conv1d_silu(*args) if opts is None else lib.ssd_conv1d_silu_ex(*args, _opts_ref(opts))
    if st != SSD_OK:
        raise SsdError(st, "ssd_conv1d_silu")
    return x, B, C, conv_state_out


def conv1d_silu_step(conv_state, xbc, weight, bias, nheads, headdim, dstate, ngroups, x=None, B=None, C=None,
                     stream=None):
    """One decode token: xbc (B, Dc); conv_state (B, K-1, Dc) is shifted in place.  Returns (x, B, C)."""
    if xbc.dim() != 2:
        raise ValueError("xbc (B, Dc) expected")
    b = xbc.shape[0]
    Dc, K = _check_conv(xbc, weight, bias, (b,), nheads, headdim, dstate, ngroups)
    if tuple(conv_state.shape) != (b, K - 1, Dc) or conv_state.dtype != xbc.dtype or not conv_state.is_contiguous():
        raise ValueError("conv state must be a contiguous (B, K-1, Dc) tensor of xbc's dtype")
    x, B, C = _conv_outputs(xbc, (b,), nheads, headdim, dstate, ngroups, x, B, C)
    dims = make_dims(b, 1, nheads, headdim, dstate, ngroups, xbc.dtype)
    st = load_library().ssd_conv1d_silu_step(ctypes.byref(dims), int(K), _ptr(conv_state), _ptr(xbc), _ptr(weight),
                                             _ptr(bias), _ptr(x), _ptr(B), _ptr(C), _stream(stream))
    if st != SSD_OK:
        raise SsdError(st, "ssd_conv1d_silu_step")
    return x, B, C


def bwd_heads(dims, chunk_size, opts=None):
    """Heads per bwd_dxdb workgroup ssd_bwd takes (1, or 4: dB summed over four heads on chip)."""
    return int(load_library().ssd_bwd_heads(ctypes.byref(dims), int(chunk_size), _opts_ref(opts)))


def fwd_state_path(dims, chunk_size, opts=None):
    """1: chunk_state then state_passing; 2: one pass over the chunks; 3: segmented chunk states;
    0: invalid or empty."""
    return int(load_library().ssd_fwd_state_path(ctypes.byref(dims), int(chunk_size), _opts_ref(opts)))


def fwd_state_segment_chunks(dims, chunk_size, opts=None):
    """Chunks per segment on the segmented chunk-state path, 0 on the other paths."""
    return int(load_library().ssd_fwd_state_segment_chunks(ctypes.byref(dims), int(chunk_size), _opts_ref(opts)))
