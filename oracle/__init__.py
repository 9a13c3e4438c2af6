"""fp64 CPU oracle for the selective scan and its decode step.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``.  The HIP library never imports,
links or calls it, and it shares no code with the HIP path.

Every function follows the definitions in "Mamba and selective state spaces"
(zerotofrontier.app/ssm/mamba): the S6 definition box in "The selective
state-space model", the two rules of "The discretization the code actually
uses", the SiLU gate of "The Mamba block" and the step of "Decoding with a
constant-size cache".  The C source states each formula beside its code.

Inputs are converted to float64 here (bf16 and fp32 values convert exactly);
outputs stay float64.

Parity status: every function below is pinned by ``tests/test_oracle_pins.py``
against the pages' worked numbers, closed forms (LTI convolution, first-order
IIR filter), a brute-force mixing-matrix evaluation and invariants.  The
initial state, the sequence lengths and the document resets of ``scan_fwd`` are
pinned against independent routes to the same result: scanning the truncated
or split sequence, and the first page's remark that one very large step resets
the state.  The backward pass (``scan_bwd``) is pinned by central finite
differences of the forward; the convolution by numpy.convolve and the impulse
response.
"""
import ctypes
import os

import numpy as np

from . import build as _build

ZOH = 0
EULER = 1
_MODES = {"zoh": ZOH, "euler": EULER, ZOH: ZOH, EULER: EULER}

_lib = None
_dp = ctypes.POINTER(ctypes.c_double)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("SSM_ORACLE_LIB")  # a planted-mistake copy, in the mutation tests
    if path is None:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build()
    lib = ctypes.CDLL(path)
    lib.oracle_softplus.restype = ctypes.c_double
    lib.oracle_softplus.argtypes = [ctypes.c_double]
    lib.oracle_sigmoid.restype = ctypes.c_double
    lib.oracle_sigmoid.argtypes = [ctypes.c_double]
    lib.oracle_discretize.restype = None
    lib.oracle_discretize.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                      ctypes.c_int, _dp, _dp]
    lib.oracle_combine.restype = None
    lib.oracle_combine.argtypes = [ctypes.c_double] * 4 + [_dp, _dp]
    lib.oracle_scan_fwd.restype = None
    lib.oracle_scan_fwd.argtypes = [ctypes.c_void_p] * 9 + [ctypes.c_int, ctypes.c_int,
                                                            ctypes.c_void_p, ctypes.c_void_p] + \
        [ctypes.c_int64] * 4 + [ctypes.c_int]
    lib.oracle_scan_fwd_ex.restype = None
    lib.oracle_scan_fwd_ex.argtypes = [ctypes.c_void_p] * 11 + [ctypes.c_int, ctypes.c_int,
                                                               ctypes.c_void_p, ctypes.c_void_p] + \
        [ctypes.c_int64] * 4 + [ctypes.c_int]
    lib.oracle_step.restype = None
    lib.oracle_step.argtypes = [ctypes.c_void_p] * 9 + [ctypes.c_int, ctypes.c_int,
                                                        ctypes.c_void_p] + [ctypes.c_int64] * 3
    lib.oracle_step_mt.restype = None
    lib.oracle_step_mt.argtypes = [ctypes.c_void_p] * 9 + [ctypes.c_int, ctypes.c_int,
                                                           ctypes.c_void_p] + \
        [ctypes.c_int64] * 3 + [ctypes.c_int]
    lib.oracle_scan_bwd.restype = None
    lib.oracle_scan_bwd.argtypes = [ctypes.c_void_p] * 11 + [ctypes.c_int, ctypes.c_int] + \
        [ctypes.c_void_p] * 11 + [ctypes.c_int64] * 4
    lib.oracle_ssd_fwd.restype = None
    lib.oracle_ssd_fwd.argtypes = [ctypes.c_void_p] * 9 + [ctypes.c_int, ctypes.c_int,
                                                           ctypes.c_void_p, ctypes.c_void_p] + \
        [ctypes.c_int64] * 5
    lib.oracle_conv1d_fwd.restype = None
    lib.oracle_conv1d_fwd.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int, ctypes.c_void_p,
                                                              ctypes.c_void_p] + [ctypes.c_int64] * 4
    lib.oracle_conv1d_step.restype = None
    lib.oracle_conv1d_step.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int, ctypes.c_void_p] + \
        [ctypes.c_int64] * 3
    lib.oracle_conv1d_bwd.restype = None
    lib.oracle_conv1d_bwd.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int] + \
        [ctypes.c_void_p] * 6 + [ctypes.c_int64] * 4
    _lib = lib
    return lib


def host_threads() -> int:
    """Host threads the oracle uses by default: the CPUs this process may run
    on (its affinity mask), capped by a cgroup CPU quota and by OMP_NUM_THREADS
    where those are set (a machine that shares its cores between jobs grants
    each its share that way)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            quota, period = f.read().split()[:2]
        if quota != "max":
            n = min(n, max(1, -(-int(quota) // int(period))))
    except (OSError, ValueError):
        pass
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def softplus(v: float) -> float:
    """log(1 + e^v), overflow-safe."""
    return _load().oracle_softplus(float(v))


def sigmoid(v: float) -> float:
    return _load().oracle_sigmoid(float(v))


def discretize(delta: float, a: float, b: float, dt_mode="zoh"):
    """(abar, bbar) for one (channel, state) pair under ZOH or exponential-Euler."""
    ab = ctypes.c_double()
    bb = ctypes.c_double()
    _load().oracle_discretize(float(delta), float(a), float(b), _MODES[dt_mode],
                              ctypes.byref(ab), ctypes.byref(bb))
    return ab.value, bb.value


def combine(first, then):
    """Apply the affine step `first` = (a1, b1) and then `then` = (a2, b2)."""
    a = ctypes.c_double()
    b = ctypes.c_double()
    _load().oracle_combine(float(first[0]), float(first[1]), float(then[0]), float(then[1]),
                           ctypes.byref(a), ctypes.byref(b))
    return a.value, b.value


def scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True,
             dt_mode="zoh", h0=None, seq_lens=None, reset=None, nthreads=None):
    """Sequential fp64 selective scan.

    u, delta, z: (batch, L, dim); B, C: (batch, L, N); A: (dim, N); D, delta_bias: (dim,);
    h0: optional (batch, dim, N) initial state (zero when omitted);
    seq_lens: optional (batch,) real lengths (tokens past them are padding: y = 0,
    state kept); reset: optional (batch, L) flags, state zeroed before a flagged token.
    Returns (y (batch, L, dim), last_state (batch, dim, N)), both float64.
    """
    u = _f64(u)
    delta = _f64(delta)
    A = _f64(A)
    B = _f64(B)
    C = _f64(C)
    D = _f64(D)
    z = _f64(z)
    delta_bias = _f64(delta_bias)
    h0 = _f64(h0)
    batch, L, dim = u.shape
    N = A.shape[1]
    assert delta.shape == u.shape and A.shape == (dim, N)
    assert B.shape == (batch, L, N) and C.shape == (batch, L, N)
    assert D is None or D.shape == (dim,)
    assert z is None or z.shape == u.shape
    assert delta_bias is None or delta_bias.shape == (dim,)
    assert h0 is None or h0.shape == (batch, dim, N)
    if seq_lens is not None:
        seq_lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int64))
        assert seq_lens.shape == (batch,)
    if reset is not None:
        reset = np.ascontiguousarray(np.asarray(reset) != 0, dtype=np.uint8)
        assert reset.shape == (batch, L)
    y = np.empty((batch, L, dim), dtype=np.float64)
    last = np.empty((batch, dim, N), dtype=np.float64)
    if nthreads is None:
        nthreads = host_threads()
    lib = _load()
    if seq_lens is None and reset is None:
        lib.oracle_scan_fwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                            _ptr(delta_bias), _ptr(h0), int(bool(softplus)), _MODES[dt_mode],
                            _ptr(y), _ptr(last), batch, L, dim, N, int(nthreads))
    else:
        lib.oracle_scan_fwd_ex(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                               _ptr(delta_bias), _ptr(h0), _ptr(seq_lens), _ptr(reset),
                               int(bool(softplus)), _MODES[dt_mode], _ptr(y), _ptr(last),
                               batch, L, dim, N, int(nthreads))
    return y, last


def step(state, u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True,
         dt_mode="zoh", nthreads=None, inplace=False):
    """One fp64 decode step.

    state: (batch, dim, N) -- not modified (unless inplace: then it must be a
    C-contiguous float64 array, updated and returned); the updated state is returned.
    u, delta, z: (batch, dim); B, C: (batch, N).  Rows (b, c) are split over
    nthreads host threads (default: host_threads()).
    Returns (y (batch, dim), new_state (batch, dim, N)).
    """
    if inplace:
        assert isinstance(state, np.ndarray) and state.dtype == np.float64 \
            and state.flags.c_contiguous
        st = state
    else:
        st = np.array(state, dtype=np.float64, copy=True, order="C")
    u = _f64(u)
    delta = _f64(delta)
    A = _f64(A)
    B = _f64(B)
    C = _f64(C)
    D = _f64(D)
    z = _f64(z)
    delta_bias = _f64(delta_bias)
    batch, dim = u.shape
    N = A.shape[1]
    assert st.shape == (batch, dim, N) and B.shape == (batch, N) and C.shape == (batch, N)
    y = np.empty((batch, dim), dtype=np.float64)
    if nthreads is None:
        nthreads = host_threads()
    _load().oracle_step_mt(_ptr(st), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                           _ptr(z), _ptr(delta_bias), int(bool(softplus)), _MODES[dt_mode],
                           _ptr(y), batch, dim, N, int(nthreads))
    return y, st


def conv1d_fwd(x, weight, bias=None, silu=True, state_in=None, seq_lens=None, reset=None):
    """The block's causal depthwise convolution (+ SiLU) over whole sequences, fp64.

    x: (batch, L, dim); weight: (dim, k), weight[c, i] multiplies the input i
    steps back; bias: (dim,); state_in: optional (batch, k - 1, dim) window of
    earlier inputs, oldest first; seq_lens (batch,), reset (batch, L) as in
    scan_fwd.  Returns (out (batch, L, dim), state_out (batch, k - 1, dim)).
    """
    x = _f64(x)
    w = _f64(weight)
    bias = _f64(bias)
    state_in = _f64(state_in)
    batch, L, dim = x.shape
    k = w.shape[1]
    assert w.shape == (dim, k) and k >= 1
    assert bias is None or bias.shape == (dim,)
    assert state_in is None or state_in.shape == (batch, k - 1, dim)
    if seq_lens is not None:
        seq_lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int64))
        assert seq_lens.shape == (batch,)
    if reset is not None:
        reset = np.ascontiguousarray(np.asarray(reset) != 0, dtype=np.uint8)
        assert reset.shape == (batch, L)
    out = np.empty((batch, L, dim), dtype=np.float64)
    st = np.empty((batch, k - 1, dim), dtype=np.float64)
    _load().oracle_conv1d_fwd(_ptr(x), _ptr(w), _ptr(bias), _ptr(state_in), _ptr(seq_lens),
                              _ptr(reset), int(bool(silu)), _ptr(out), _ptr(st), batch, L, dim, k)
    return out, st


def conv1d_step(window, x, weight, bias=None, silu=True):
    """One decoding step of the convolution, fp64.

    window: (batch, k - 1, dim), oldest first -- not modified; x: (batch, dim).
    Returns (out (batch, dim), new_window).
    """
    win = np.array(window, dtype=np.float64, copy=True, order="C")
    x = _f64(x)
    w = _f64(weight)
    bias = _f64(bias)
    batch, dim = x.shape
    k = w.shape[1]
    assert win.shape == (batch, k - 1, dim) and w.shape == (dim, k)
    out = np.empty((batch, dim), dtype=np.float64)
    _load().oracle_conv1d_step(_ptr(win), _ptr(x), _ptr(w), _ptr(bias), int(bool(silu)),
                               _ptr(out), batch, dim, k)
    return out, win


def conv1d_bwd(x, weight, dout, bias=None, silu=True, state_in=None, seq_lens=None, reset=None,
               dstate_out=None):
    """Gradients of conv1d_fwd (same arguments), fp64: given dout (batch, L, dim)
    and optionally dstate_out (batch, k - 1, dim), the gradient of state_out,
    returns a dict with dx, dweight (dim, k) and, where their inputs are
    given, dbias and dstate_in."""
    x, w, dout = _f64(x), _f64(weight), _f64(dout)
    bias, state_in, dstate_out = _f64(bias), _f64(state_in), _f64(dstate_out)
    batch, L, dim = x.shape
    k = w.shape[1]
    assert w.shape == (dim, k) and dout.shape == x.shape
    assert state_in is None or state_in.shape == (batch, k - 1, dim)
    assert dstate_out is None or dstate_out.shape == (batch, k - 1, dim)
    if seq_lens is not None:
        seq_lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int64))
        assert seq_lens.shape == (batch,)
    if reset is not None:
        reset = np.ascontiguousarray(np.asarray(reset) != 0, dtype=np.uint8)
        assert reset.shape == (batch, L)
    out = dict(dx=np.empty_like(x), dweight=np.empty((dim, k)),
               dbias=np.empty(dim) if bias is not None else None,
               dstate_in=np.empty((batch, k - 1, dim)) if state_in is not None else None)
    _load().oracle_conv1d_bwd(_ptr(x), _ptr(w), _ptr(bias), _ptr(state_in), _ptr(seq_lens),
                              _ptr(reset), int(bool(silu)), _ptr(dout), _ptr(dstate_out),
                              _ptr(out["dx"]), _ptr(out["dweight"]), _ptr(out["dbias"]),
                              _ptr(out["dstate_in"]), batch, L, dim, k)
    return out


def scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None, softplus=True,
             dt_mode="zoh", h0=None, dlast=None, seq_lens=None, reset=None):
    """Gradients of the fp64 scan (scan_fwd, with h0, seq_lens and reset as
    there): given dy (batch, L, dim) and optionally dlast (batch, dim, N), the
    gradient of last_state, returns a dict with du, ddelta (of the raw delta),
    dA, dB, dC and, where their inputs are given, dD, dz, ddelta_bias and dh0
    -- all float64.  Padding tokens get zero gradients.  Every state is kept
    (small cases only).
    """
    u, delta, A, B, C = _f64(u), _f64(delta), _f64(A), _f64(B), _f64(C)
    dy, D, z, delta_bias, h0, dlast = _f64(dy), _f64(D), _f64(z), _f64(delta_bias), _f64(h0), \
        _f64(dlast)
    batch, L, dim = u.shape
    N = A.shape[1]
    assert dy.shape == u.shape and B.shape == (batch, L, N) and C.shape == (batch, L, N)
    assert dlast is None or dlast.shape == (batch, dim, N)
    assert h0 is None or h0.shape == (batch, dim, N)
    sl = None if seq_lens is None else np.ascontiguousarray(seq_lens, dtype=np.int64)
    rs = None if reset is None else np.ascontiguousarray(np.asarray(reset) != 0, dtype=np.uint8)
    assert sl is None or sl.shape == (batch,)
    assert rs is None or rs.shape == (batch, L)
    out = dict(du=np.empty_like(u), ddelta=np.empty_like(u), dA=np.empty((dim, N)),
               dB=np.empty((batch, L, N)), dC=np.empty((batch, L, N)))
    out["dD"] = np.empty(dim) if D is not None else None
    out["dz"] = np.empty_like(u) if z is not None else None
    out["ddelta_bias"] = np.empty(dim) if delta_bias is not None else None
    out["dh0"] = np.empty((batch, dim, N)) if h0 is not None else None
    _load().oracle_scan_bwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                            _ptr(delta_bias), _ptr(h0), _ptr(sl), _ptr(rs), int(bool(softplus)),
                            _MODES[dt_mode], _ptr(dy), _ptr(dlast), _ptr(out["du"]),
                            _ptr(out["ddelta"]),
                            _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]),
                            _ptr(out["dz"]), _ptr(out["ddelta_bias"]), _ptr(out["dh0"]),
                            batch, L, dim, N)
    return out


def ssd_fwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, softplus=True, dt_mode="euler",
            h0=None):
    """Mamba-2 / SSD layer, fp64: one scalar decay A[h] and one step size per
    (token, head); B, C shared by all heads.

    x, z: (batch, L, nheads, P); dt: (batch, L, nheads); A, D, dt_bias: (nheads,);
    B, C: (batch, L, N); h0: optional (batch, nheads, P, N).
    Returns (y (batch, L, nheads, P), last_state (batch, nheads, P, N)).
    """
    x, dt, A, B, C = _f64(x), _f64(dt), _f64(A), _f64(B), _f64(C)
    D, z, dt_bias, h0 = _f64(D), _f64(z), _f64(dt_bias), _f64(h0)
    batch, L, nheads, P = x.shape
    N = B.shape[2]
    assert dt.shape == (batch, L, nheads) and A.shape == (nheads,)
    assert B.shape == (batch, L, N) and C.shape == (batch, L, N)
    assert z is None or z.shape == x.shape
    assert h0 is None or h0.shape == (batch, nheads, P, N)
    y = np.empty_like(x)
    last = np.empty((batch, nheads, P, N))
    _load().oracle_ssd_fwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                           _ptr(dt_bias), _ptr(h0), int(bool(softplus)), _MODES[dt_mode],
                           _ptr(y), _ptr(last), batch, L, nheads, P, N)
    return y, last
