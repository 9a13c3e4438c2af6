"""MI355X (gfx950) selective scan: Python binding of the C ABI in include/ssm66.h.

This module only marshals arguments: it checks tensor device, dtype, shape and
contiguity, allocates outputs with torch and passes raw device pointers and the
current HIP stream to the library.  Every step of the computation runs in the
library's HIP kernels.  There is no CPU or PyTorch fallback: if the library is
missing, every call raises.

    y, last_state = scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                             softplus=True, dt_mode="zoh",
                             h0=None, seq_lens=None, reset=None)
    y = step(state, u, delta, A, B, C, D=None, z=None, delta_bias=None,
             softplus=True, dt_mode="zoh")     # state updated in place
    grads = scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None,
                     softplus=True, dt_mode="zoh", h0=None, dlast=None)
    y, last_state = ssd_fwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, softplus=True,
                            dt_mode="euler", h0=None)          # Mamba-2 / SSD
    out, window = conv1d_fwd(x, weight, bias=None, silu=True, window_in=None,
                             seq_lens=None, reset=None)
    out = conv1d_step(window, x, weight, bias=None, silu=True)   # window updated in place
"""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libssm66_hip.so")

SSM_F32, SSM_BF16 = 0, 1
SSM_DT_ZOH, SSM_DT_EULER = 0, 1
_MODES = {"zoh": SSM_DT_ZOH, "euler": SSM_DT_EULER}
# scan kernel choices (SSM_SCAN_KERNEL_*): the library's own, the sequential
# kernel with 1, 2 or 4 states per lane, the time-parallel kernels with four
# waves, one wave or 16 lanes per (batch, channel) row
SCAN_KERNELS = {"auto": 0, "seq1": 1, "seq2": 2, "seq4": 3, "tpar": 4, "wave": 5, "wave4": 6}

_lib = None


class SsmError(RuntimeError):
    def __init__(self, status, where):
        super().__init__(f"{where}: status {status} ({status_string(status)})")
        self.status = status


def load_library():
    """Load the built HIP library (build it with selective_state_space_66_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"HIP library not built: {LIB_PATH} is missing "
                          "(run `python -m selective_state_space_66_amd.build`)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.ssm_scan_fwd.restype = ci
    lib.ssm_scan_fwd.argtypes = [vp] * 8 + [ci, ci, vp, vp, i64, i64, i64, i64, ci, vp]
    lib.ssm_scan_fwd_ex.restype = ci
    lib.ssm_scan_fwd_ex.argtypes = [vp] * 8 + [ci, ci] + [vp] * 5 + [i64, i64, i64, i64, ci, vp]
    lib.ssm_scan_bwd_workspace_size.restype = ctypes.c_size_t
    lib.ssm_scan_bwd_workspace_size.argtypes = [i64] * 4
    lib.ssm_scan_ckpt_size.restype = ctypes.c_size_t
    lib.ssm_scan_ckpt_size.argtypes = [i64] * 4
    lib.ssm_scan_kernel_name.restype = ctypes.c_char_p
    lib.ssm_scan_kernel_name.argtypes = [i64] * 4
    lib.ssm_scan_fwd_kernel.restype = ci
    lib.ssm_scan_fwd_kernel.argtypes = [ci] + [vp] * 8 + [ci, ci] + [vp] * 6 + [i64] * 4 + [ci, vp]
    lib.ssm_scan_fwd_ckpt.restype = ci
    lib.ssm_scan_fwd_ckpt.argtypes = [vp] * 8 + [ci, ci] + [vp] * 4 + [i64] * 4 + [ci, vp]
    lib.ssm_scan_bwd_ex.restype = ci
    lib.ssm_scan_bwd_ex.argtypes = [vp] * 8 + [ci, ci] + [vp] * 16 + [ctypes.c_size_t] + \
        [i64] * 4 + [ci, vp]
    lib.ssm_scan_bwd_noalloc.restype = ci
    lib.ssm_scan_bwd_noalloc.argtypes = [vp] * 8 + [ci, ci] + [vp] * 15 + [i64] * 4 + [ci, vp]
    lib.ssm_conv1d_bwd_workspace_size.restype = ctypes.c_size_t
    lib.ssm_conv1d_bwd_workspace_size.argtypes = [i64] * 4
    lib.ssm_conv1d_bwd.restype = ci
    lib.ssm_conv1d_bwd.argtypes = [vp] * 3 + [ci] + [vp] * 10 + [ctypes.c_size_t] + [i64] * 4 + \
        [ci, vp]
    lib.ssm_scan_bwd.restype = ci
    lib.ssm_scan_bwd.argtypes = [vp] * 8 + [ci, ci] + [vp] * 13 + [ctypes.c_size_t] + \
        [i64] * 4 + [ci, vp]
    lib.ssm_ssd_fwd.restype = ci
    lib.ssm_ssd_fwd.argtypes = [vp] * 8 + [ci, ci, vp, vp, vp] + [i64] * 5 + [ci, vp]
    lib.ssm_conv1d_fwd.restype = ci
    lib.ssm_conv1d_fwd.argtypes = [vp] * 3 + [ci] + [vp] * 5 + [i64] * 4 + [ci, vp]
    lib.ssm_conv1d_step.restype = ci
    lib.ssm_conv1d_step.argtypes = [vp] * 4 + [ci, vp] + [i64] * 3 + [ci, vp]
    lib.ssm_step.restype = ci
    lib.ssm_step.argtypes = [vp] * 9 + [ci, ci, vp, i64, i64, i64, ci, vp]
    lib.ssm_alu_probe.restype = ci
    lib.ssm_alu_probe.argtypes = [ci, vp, i64, i64, vp]
    lib.ssm_status_string.restype = ctypes.c_char_p
    lib.ssm_status_string.argtypes = [ci]
    lib.ssm_abi_version.restype = ci
    lib.ssm_abi_version.argtypes = []
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().ssm_status_string(int(status)).decode()


def abi_version() -> int:
    return load_library().ssm_abi_version()


def _io_code(t):
    import torch
    if t.dtype == torch.float32:
        return SSM_F32
    if t.dtype == torch.bfloat16:
        return SSM_BF16
    raise TypeError(f"io tensors must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, shape, dtype, device):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True, dt_mode="zoh",
             y=None, last_state=None, return_last_state=True, h0=None, seq_lens=None, reset=None,
             kernel=None):
    """Selective scan over whole sequences on the GPU.

    u, delta, z: (batch, L, dim); B, C: (batch, L, N) -- all float32 or all bfloat16.
    A: (dim, N) float32; D, delta_bias: (dim,) float32.
    h0: optional (batch, dim, N) float32 initial state (last_state may be h0: in place);
    seq_lens: optional (batch,) int32 real lengths (padding after them: y = 0, state kept);
    reset: optional (batch, L) bool or uint8, state zeroed before each flagged token.
    kernel: None (the library's choice) or a key of SCAN_KERNELS to force one kernel.
    Returns (y, last_state): y like u; last_state (batch, dim, N) float32 (None if not requested).
    """
    import torch
    lib = load_library()
    if u.dim() != 3:
        raise ValueError("u must be (batch, L, dim)")
    batch, L, dim = u.shape
    N = A.shape[-1]
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on the GPU")
    io = u.dtype
    _io_code(u)
    _check(u, "u", (batch, L, dim), io, dev)
    _check(delta, "delta", (batch, L, dim), io, dev)
    _check(A, "A", (dim, N), torch.float32, dev)
    _check(B, "B", (batch, L, N), io, dev)
    _check(C, "C", (batch, L, N), io, dev)
    _check(D, "D", (dim,), torch.float32, dev)
    _check(z, "z", (batch, L, dim), io, dev)
    _check(delta_bias, "delta_bias", (dim,), torch.float32, dev)
    if y is None:
        y = torch.empty_like(u)
    _check(y, "y", (batch, L, dim), io, dev)
    if last_state is None and return_last_state:
        last_state = torch.empty((batch, dim, N), dtype=torch.float32, device=dev)
    _check(last_state, "last_state", (batch, dim, N), torch.float32, dev)
    if h0 is None and seq_lens is None and reset is None and kernel is None:
        st = lib.ssm_scan_fwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                              _ptr(delta_bias), int(bool(softplus)), _MODES[dt_mode], _ptr(y),
                              _ptr(last_state), batch, L, dim, N, _io_code(u), _stream(dev))
        if st != 0:
            raise SsmError(st, "ssm_scan_fwd")
        return y, last_state
    _check(h0, "h0", (batch, dim, N), torch.float32, dev)
    _check(seq_lens, "seq_lens", (batch,), torch.int32, dev)
    if reset is not None and reset.dtype == torch.bool:
        reset = reset.view(torch.uint8)
    _check(reset, "reset", (batch, L), torch.uint8, dev)
    if kernel is not None:
        st = lib.ssm_scan_fwd_kernel(SCAN_KERNELS[kernel], _ptr(u), _ptr(delta), _ptr(A), _ptr(B),
                                     _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                                     int(bool(softplus)), _MODES[dt_mode], _ptr(h0),
                                     _ptr(seq_lens), _ptr(reset), _ptr(y), _ptr(last_state), None,
                                     batch, L, dim, N, _io_code(u), _stream(dev))
        if st != 0:
            raise SsmError(st, "ssm_scan_fwd_kernel")
        return y, last_state
    st = lib.ssm_scan_fwd_ex(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                             _ptr(delta_bias), int(bool(softplus)), _MODES[dt_mode], _ptr(h0),
                             _ptr(seq_lens), _ptr(reset), _ptr(y), _ptr(last_state), batch, L,
                             dim, N, _io_code(u), _stream(dev))
    if st != 0:
        raise SsmError(st, "ssm_scan_fwd_ex")
    return y, last_state


def step(state, u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True,
         dt_mode="zoh", y=None):
    """One decode step on the GPU; `state` (batch, dim, N) float32 is updated in place.

    u, delta, z: (batch, dim); B, C: (batch, N) -- float32 or bfloat16. Returns y like u.
    """
    import torch
    lib = load_library()
    if u.dim() != 2:
        raise ValueError("u must be (batch, dim)")
    batch, dim = u.shape
    N = A.shape[-1]
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on the GPU")
    io = u.dtype
    _io_code(u)
    _check(state, "state", (batch, dim, N), torch.float32, dev)
    _check(u, "u", (batch, dim), io, dev)
    _check(delta, "delta", (batch, dim), io, dev)
    _check(A, "A", (dim, N), torch.float32, dev)
    _check(B, "B", (batch, N), io, dev)
    _check(C, "C", (batch, N), io, dev)
    _check(D, "D", (dim,), torch.float32, dev)
    _check(z, "z", (batch, dim), io, dev)
    _check(delta_bias, "delta_bias", (dim,), torch.float32, dev)
    if y is None:
        y = torch.empty_like(u)
    _check(y, "y", (batch, dim), io, dev)
    st = lib.ssm_step(_ptr(state), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                      _ptr(z), _ptr(delta_bias), int(bool(softplus)), _MODES[dt_mode], _ptr(y),
                      batch, dim, N, _io_code(u), _stream(dev))
    if st != 0:
        raise SsmError(st, "ssm_step")
    return y


def conv1d_fwd(x, weight, bias=None, silu=True, window_in=None, seq_lens=None, reset=None,
               out=None, window_out=None, return_window=True):
    """The block's causal depthwise convolution (+ SiLU) over whole sequences on the GPU.

    x: (batch, L, dim) float32 or bfloat16; weight: (dim, k) float32, weight[c, i]
    multiplies the input i steps back (1 <= k <= 4); bias: (dim,) float32;
    window_in: optional (batch, k - 1, dim) earlier inputs, oldest first;
    seq_lens: optional (batch,) int32; reset: optional (batch, L) bool or uint8.
    Returns (out like x, window (batch, k - 1, dim) like x, or None if not requested).
    """
    import torch
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be (batch, L, dim)")
    batch, L, dim = x.shape
    k = weight.shape[-1]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on the GPU")
    io = x.dtype
    _io_code(x)
    _check(x, "x", (batch, L, dim), io, dev)
    _check(weight, "weight", (dim, k), torch.float32, dev)
    _check(bias, "bias", (dim,), torch.float32, dev)
    _check(window_in, "window_in", (batch, k - 1, dim), io, dev)
    _check(seq_lens, "seq_lens", (batch,), torch.int32, dev)
    if reset is not None and reset.dtype == torch.bool:
        reset = reset.view(torch.uint8)
    _check(reset, "reset", (batch, L), torch.uint8, dev)
    if out is None:
        out = torch.empty_like(x)
    _check(out, "out", (batch, L, dim), io, dev)
    if window_out is None and return_window:
        window_out = torch.empty((batch, k - 1, dim), dtype=io, device=dev)
    _check(window_out, "window_out", (batch, k - 1, dim), io, dev)
    st = lib.ssm_conv1d_fwd(_ptr(x), _ptr(weight), _ptr(bias), int(bool(silu)), _ptr(window_in),
                            _ptr(seq_lens), _ptr(reset), _ptr(out), _ptr(window_out), batch, L,
                            dim, k, _io_code(x), _stream(dev))
    if st != 0:
        raise SsmError(st, "ssm_conv1d_fwd")
    return out, window_out


def conv1d_step(window, x, weight, bias=None, silu=True, out=None):
    """One decoding step of the convolution on the GPU; `window` (batch, k - 1, dim),
    oldest first, is shifted in place.  x: (batch, dim). Returns out like x."""
    import torch
    lib = load_library()
    if x.dim() != 2:
        raise ValueError("x must be (batch, dim)")
    batch, dim = x.shape
    k = weight.shape[-1]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on the GPU")
    io = x.dtype
    _io_code(x)
    _check(window, "window", (batch, k - 1, dim), io, dev)
    _check(x, "x", (batch, dim), io, dev)
    _check(weight, "weight", (dim, k), torch.float32, dev)
    _check(bias, "bias", (dim,), torch.float32, dev)
    if out is None:
        out = torch.empty_like(x)
    _check(out, "out", (batch, dim), io, dev)
    st = lib.ssm_conv1d_step(_ptr(window), _ptr(x), _ptr(weight), _ptr(bias), int(bool(silu)),
                             _ptr(out), batch, dim, k, _io_code(x), _stream(dev))
    if st != 0:
        raise SsmError(st, "ssm_conv1d_step")
    return out


def conv1d_bwd_workspace_size(batch, L, dim, width):
    """Bytes of workspace ssm_conv1d_bwd needs for these sizes."""
    return int(load_library().ssm_conv1d_bwd_workspace_size(batch, L, dim, width))


def conv1d_bwd(x, weight, dout, bias=None, silu=True, window_in=None, seq_lens=None, reset=None,
               dwindow_out=None, workspace=None):
    """Gradients of conv1d_fwd on the GPU (same arguments): given dout like x
    and optionally dwindow_out (batch, k - 1, dim), the gradient of the window
    handed to decoding, returns a dict with dx (io dtype), dweight (dim, k)
    float32 and, where their inputs were given, dbias (float32) and dwindow_in
    (io dtype).  workspace: optional uint8 device tensor of at least
    conv1d_bwd_workspace_size() bytes."""
    import torch
    lib = load_library()
    batch, L, dim = x.shape
    k = weight.shape[1]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on the GPU")
    io = x.dtype
    _io_code(x)
    _check(x, "x", (batch, L, dim), io, dev)
    _check(dout, "dout", (batch, L, dim), io, dev)
    _check(weight, "weight", (dim, k), torch.float32, dev)
    _check(bias, "bias", (dim,), torch.float32, dev)
    _check(window_in, "window_in", (batch, k - 1, dim), io, dev)
    _check(dwindow_out, "dwindow_out", (batch, k - 1, dim), io, dev)
    _check(seq_lens, "seq_lens", (batch,), torch.int32, dev)
    if reset is not None:
        if reset.dtype == torch.bool:
            reset = reset.to(torch.uint8)
        _check(reset, "reset", (batch, L), torch.uint8, dev)
    need = conv1d_bwd_workspace_size(batch, L, dim, k)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if workspace.numel() < need:
        raise ValueError(f"workspace: need {need} bytes, got {workspace.numel()}")
    g = dict(dx=torch.empty_like(x), dweight=torch.empty((dim, k), dtype=torch.float32, device=dev),
             dbias=torch.empty((dim,), dtype=torch.float32, device=dev) if bias is not None else None,
             dwindow_in=torch.empty_like(window_in) if window_in is not None else None)
    st = lib.ssm_conv1d_bwd(_ptr(x), _ptr(weight), _ptr(bias), int(bool(silu)), _ptr(window_in),
                            _ptr(seq_lens), _ptr(reset), _ptr(dout), _ptr(dwindow_out),
                            _ptr(g["dx"]), _ptr(g["dweight"]), _ptr(g["dbias"]),
                            _ptr(g["dwindow_in"]), _ptr(workspace), workspace.numel(), batch, L,
                            dim, k, _io_code(x), _stream(dev))
    if st != 0:
        raise SsmError(st, "ssm_conv1d_bwd")
    return g


def scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None, softplus=True,
             dt_mode="zoh", h0=None, dlast=None, workspace=None, ckpt=None, noalloc=False,
             seq_lens=None, reset=None):
    """Gradients of scan_fwd / scan_fwd_ex on the GPU (states recomputed, not stored).

    dy: like u; dlast: optional (batch, dim, N) float32, the gradient of last_state.
    seq_lens (batch,) int32 and reset (batch, L) uint8 or bool: as for scan_fwd_ex
    (padding tokens get zero gradients; no gradient crosses a document start).
    Returns a dict: du, ddelta (of the raw delta), dB, dC (io dtype), dA (float32),
    and, where their inputs were given, dz (io dtype), dD, ddelta_bias, dh0 (float32).
    workspace: optional uint8 device tensor of at least scan_bwd_workspace_size() bytes.
    ckpt: optional checkpoints from scan_fwd_train (or scan_fwd with kernel and
    ckpt) on the same inputs, h0, lengths and resets; the states are then
    recomputed from them, without a forward sweep.
    noalloc: run ssm_scan_bwd_noalloc, whose workspace is the library's static
    device scratch (no workspace tensor; sizes within its limit only).
    """
    import torch
    lib = load_library()
    batch, L, dim = u.shape
    N = A.shape[-1]
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on the GPU")
    io = u.dtype
    _io_code(u)
    for t, name, shape in ((u, "u", (batch, L, dim)), (delta, "delta", (batch, L, dim)),
                           (B, "B", (batch, L, N)), (C, "C", (batch, L, N)),
                           (dy, "dy", (batch, L, dim)), (z, "z", (batch, L, dim))):
        _check(t, name, shape, io, dev)
    _check(A, "A", (dim, N), torch.float32, dev)
    _check(D, "D", (dim,), torch.float32, dev)
    _check(delta_bias, "delta_bias", (dim,), torch.float32, dev)
    _check(h0, "h0", (batch, dim, N), torch.float32, dev)
    _check(dlast, "dlast", (batch, dim, N), torch.float32, dev)
    _check(ckpt, "ckpt", (batch, (L + 15) // 16, dim, N), torch.float32, dev)
    _check(seq_lens, "seq_lens", (batch,), torch.int32, dev)
    if reset is not None:
        if reset.dtype == torch.bool:
            reset = reset.to(torch.uint8)
        _check(reset, "reset", (batch, L), torch.uint8, dev)
    need = scan_bwd_workspace_size(batch, L, dim, N)
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc takes no workspace")
    else:
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        if workspace.numel() < need:
            raise ValueError(f"workspace: need {need} bytes, got {workspace.numel()}")
    f32 = dict(dtype=torch.float32, device=dev)
    g = dict(du=torch.empty_like(u), ddelta=torch.empty_like(u),
             dB=torch.empty((batch, L, N), dtype=io, device=dev),
             dC=torch.empty((batch, L, N), dtype=io, device=dev),
             dA=torch.empty((dim, N), **f32),
             dz=torch.empty_like(u) if z is not None else None,
             dD=torch.empty((dim,), **f32) if D is not None else None,
             ddelta_bias=torch.empty((dim,), **f32) if delta_bias is not None else None,
             dh0=torch.empty((batch, dim, N), **f32) if h0 is not None else None)
    if noalloc:
        st = lib.ssm_scan_bwd_noalloc(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                      _ptr(z), _ptr(delta_bias), int(bool(softplus)),
                                      _MODES[dt_mode], _ptr(h0), _ptr(seq_lens), _ptr(reset),
                                      _ptr(dy), _ptr(dlast),
                                      _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]),
                                      _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]),
                                      _ptr(g["ddelta_bias"]), _ptr(g["dh0"]), _ptr(ckpt), batch,
                                      L, dim, N, _io_code(u), _stream(dev))
        if st != 0:
            raise SsmError(st, "ssm_scan_bwd_noalloc")
        return g
    st = lib.ssm_scan_bwd_ex(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                             _ptr(delta_bias), int(bool(softplus)), _MODES[dt_mode], _ptr(h0),
                             _ptr(seq_lens), _ptr(reset), _ptr(dy), _ptr(dlast), _ptr(g["du"]),
                             _ptr(g["ddelta"]),
                             _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]),
                             _ptr(g["dz"]), _ptr(g["ddelta_bias"]), _ptr(g["dh0"]), _ptr(ckpt),
                             _ptr(workspace), workspace.numel(), batch, L, dim, N, _io_code(u),
                             _stream(dev))
    if st != 0:
        raise SsmError(st, "ssm_scan_bwd_ex")
    return g


ALU_PROBES = {"fma": 0, "exp": 1, "mix": 2}


def alu_probe(op, sink, blocks, iters):
    """Launch the issue-rate probe `op` ("fma", "exp" or "mix") on the current
    stream: blocks x 256 lanes, iters iterations each; sink is a float32 device
    tensor of at least blocks * 256 elements.  Time it with events on the
    current stream."""
    import torch
    lib = load_library()
    if sink.dtype != torch.float32 or sink.device.type != "cuda" or sink.numel() < blocks * 256:
        raise ValueError("sink: float32 device tensor of at least blocks * 256 elements")
    st = lib.ssm_alu_probe(ALU_PROBES[op], _ptr(sink), int(blocks), int(iters),
                           _stream(sink.device))
    if st != 0:
        raise SsmError(st, "ssm_alu_probe")


def scan_kernel_name(batch, L, dim, N):
    """Name of the kernel ssm_scan_fwd runs for these sizes (host only)."""
    return load_library().ssm_scan_kernel_name(batch, L, dim, N).decode()


def scan_ckpt_size(batch, L, dim, N):
    """Bytes of the training forward's checkpoints for these sizes."""
    return int(load_library().ssm_scan_ckpt_size(batch, L, dim, N))


def scan_fwd_train(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True,
                   dt_mode="zoh", h0=None, y=None, last_state=None, ckpt=None, kernel=None,
                   seq_lens=None, reset=None):
    """The training forward: scan_fwd (with optional h0, seq_lens and reset, as
    there) that also keeps the state before every 16th token for scan_bwd.
    kernel as for scan_fwd.

    Returns (y, last_state, ckpt); ckpt is (batch, ceil(L/16), dim, N) float32.
    """
    import torch
    lib = load_library()
    if u.dim() != 3:
        raise ValueError("u must be (batch, L, dim)")
    batch, L, dim = u.shape
    N = A.shape[-1]
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on the GPU")
    io = u.dtype
    _io_code(u)
    for t, name, shape in ((u, "u", (batch, L, dim)), (delta, "delta", (batch, L, dim)),
                           (B, "B", (batch, L, N)), (C, "C", (batch, L, N)),
                           (z, "z", (batch, L, dim))):
        _check(t, name, shape, io, dev)
    _check(A, "A", (dim, N), torch.float32, dev)
    _check(D, "D", (dim,), torch.float32, dev)
    _check(delta_bias, "delta_bias", (dim,), torch.float32, dev)
    _check(h0, "h0", (batch, dim, N), torch.float32, dev)
    if y is None:
        y = torch.empty_like(u)
    _check(y, "y", (batch, L, dim), io, dev)
    if last_state is None:
        last_state = torch.empty((batch, dim, N), dtype=torch.float32, device=dev)
    _check(last_state, "last_state", (batch, dim, N), torch.float32, dev)
    if ckpt is None:
        ckpt = torch.empty((batch, (L + 15) // 16, dim, N), dtype=torch.float32, device=dev)
    _check(ckpt, "ckpt", (batch, (L + 15) // 16, dim, N), torch.float32, dev)
    _check(seq_lens, "seq_lens", (batch,), torch.int32, dev)
    if reset is not None:
        if reset.dtype == torch.bool:
            reset = reset.to(torch.uint8)
        _check(reset, "reset", (batch, L), torch.uint8, dev)
    if kernel is not None or seq_lens is not None or reset is not None:
        st = lib.ssm_scan_fwd_kernel(SCAN_KERNELS[kernel or "auto"], _ptr(u), _ptr(delta), _ptr(A),
                                     _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                                     int(bool(softplus)), _MODES[dt_mode], _ptr(h0),
                                     _ptr(seq_lens), _ptr(reset),
                                     _ptr(y), _ptr(last_state), _ptr(ckpt), batch, L, dim, N,
                                     _io_code(u), _stream(dev))
        if st != 0:
            raise SsmError(st, "ssm_scan_fwd_kernel")
        return y, last_state, ckpt
    st = lib.ssm_scan_fwd_ckpt(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                               _ptr(delta_bias), int(bool(softplus)), _MODES[dt_mode], _ptr(h0),
                               _ptr(y), _ptr(last_state), _ptr(ckpt), batch, L, dim, N,
                               _io_code(u), _stream(dev))
    if st != 0:
        raise SsmError(st, "ssm_scan_fwd_ckpt")
    return y, last_state, ckpt


def scan_bwd_workspace_size(batch, L, dim, N):
    """Bytes of workspace ssm_scan_bwd needs for these sizes."""
    return int(load_library().ssm_scan_bwd_workspace_size(batch, L, dim, N))


def ssd_fwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, softplus=True, dt_mode="euler",
            h0=None, y=None, last_state=None, return_last_state=True):
    """Mamba-2 / SSD layer on the GPU's matrix cores (one scalar decay per head).

    x, z: (batch, L, nheads, headdim) bfloat16; dt: (batch, L, nheads) float32;
    A, D, dt_bias: (nheads,) float32; B, C: (batch, L, N) bfloat16;
    h0: optional (batch, nheads, headdim, N) float32.  headdim a multiple of 16, N 64 or 128.
    Returns (y like x, last_state (batch, nheads, headdim, N) float32 or None).
    """
    import torch
    lib = load_library()
    if x.dim() != 4:
        raise ValueError("x must be (batch, L, nheads, headdim)")
    batch, L, H, P = x.shape
    N = B.shape[-1]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on the GPU")
    io = x.dtype
    _io_code(x)
    _check(x, "x", (batch, L, H, P), io, dev)
    _check(z, "z", (batch, L, H, P), io, dev)
    _check(dt, "dt", (batch, L, H), torch.float32, dev)
    _check(A, "A", (H,), torch.float32, dev)
    _check(D, "D", (H,), torch.float32, dev)
    _check(dt_bias, "dt_bias", (H,), torch.float32, dev)
    _check(B, "B", (batch, L, N), io, dev)
    _check(C, "C", (batch, L, N), io, dev)
    _check(h0, "h0", (batch, H, P, N), torch.float32, dev)
    if y is None:
        y = torch.empty_like(x)
    _check(y, "y", (batch, L, H, P), io, dev)
    if last_state is None and return_last_state:
        last_state = torch.empty((batch, H, P, N), dtype=torch.float32, device=dev)
    _check(last_state, "last_state", (batch, H, P, N), torch.float32, dev)
    st = lib.ssm_ssd_fwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                         _ptr(dt_bias), int(bool(softplus)), _MODES[dt_mode], _ptr(h0), _ptr(y),
                         _ptr(last_state), batch, L, H, P, N, _io_code(x), _stream(dev))
    if st != 0:
        raise SsmError(st, "ssm_ssd_fwd")
    return y, last_state
