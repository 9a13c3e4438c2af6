"""Seeded synthetic inputs for the selective scan and the decode step.

Serves both the HIP path and the oracle; holds none of the scan's arithmetic.

Values are counter-based: element i of stream s under seed k is a pure function
of (k, s, i) (SplitMix64 of the stream position, then Box-Muller in float32), so any
subset of channels of a full-size workload can be regenerated without drawing
the rest.  That is what lets the oracle check sampled channels of the largest
shapes.

Shapes and distributions follow the Mamba layers the pages discuss:
  - A[c, n] = -(n + 1): the S4D-Real initialisation ("What each parameter does"
    and the ZOH note on the first page; "Additional model details" (3.6) on the
    second);
  - delta_bias = softplus^-1(dt), dt log-uniform in [1e-3, 1e-1] (same 3.6
    section, "where Delta starts");
  - u, raw delta, B, C, z, D ~ N(0, 1);
  - the long-sequence case mimics the selective-copying task of the first page's
    introduction: one fixed filler vector everywhere except 16 positions per
    sequence that hold fresh vectors.
bf16 values are round-to-nearest-even of the fp32 draw; both sides receive the
same bits.
"""
from dataclasses import dataclass, field
from typing import Dict, Optional, Sequence

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# stream ids
S_DT, S_D, S_STATE0, S_U, S_DELTA, S_B, S_C, S_Z, S_FILLER, S_DATA = range(1, 11)


def _mix(x: np.ndarray) -> np.ndarray:
    """SplitMix64 finaliser on a uint64 array (wrapping arithmetic)."""
    with np.errstate(over="ignore"):
        x = (x ^ (x >> np.uint64(30))) * _M1
        x = (x ^ (x >> np.uint64(27))) * _M2
        return x ^ (x >> np.uint64(31))


def _key(seed: int, stream: int) -> np.uint64:
    k = _mix(np.array([(seed * 1_000_003 + stream) & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64))
    return k[0]


def _hash(seed: int, stream: int, idx: np.ndarray) -> np.ndarray:
    """SplitMix64 of stream position idx: a uint64 per element."""
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(_key(seed, stream) + (idx + np.uint64(1)) * _GOLDEN)


def uniform(seed: int, stream: int, idx: np.ndarray) -> np.ndarray:
    """U(0,1) (open interval) in float64 at integer positions idx (53-bit)."""
    h = _hash(seed, stream, idx)
    return ((h >> np.uint64(11)).astype(np.float64) + 0.5) * (1.0 / 9007199254740992.0)


def _normal_block(seed, stream, idx, std):
    # one hash per value: 24 bits for the radius, 24 for the angle (Box-Muller,
    # cosine branch) -- tails reach about 5.9 standard deviations
    h = _hash(seed, stream, idx)
    u1 = ((h >> np.uint64(40)).astype(np.float32) + np.float32(0.5)) * np.float32(2.0 ** -24)
    u2 = ((h & np.uint64(0xFFFFFF)).astype(np.float32) + np.float32(0.5)) * np.float32(2.0 ** -24)
    z = np.sqrt(np.float32(-2.0) * np.log(u1)) * np.cos(np.float32(2.0 * np.pi) * u2)
    if std != 1.0:
        z = z * np.float32(std)
    return z.astype(np.float32, copy=False)


_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        import concurrent.futures
        import os
        try:
            n = len(os.sched_getaffinity(0))
        except (AttributeError, OSError):
            n = os.cpu_count() or 1
        omp = os.environ.get("OMP_NUM_THREADS", "")
        if omp.isdigit() and int(omp) > 0:
            n = min(n, int(omp))
        _POOL = concurrent.futures.ThreadPoolExecutor(max_workers=max(1, min(16, n)))
    return _POOL


def normal(seed: int, stream: int, idx: np.ndarray, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) as float32 at integer positions idx."""
    idx = np.asarray(idx)
    flat = idx.reshape(-1)
    n = flat.size
    blk = 1 << 21
    if n <= blk:
        return _normal_block(seed, stream, flat, std).reshape(idx.shape)
    out = np.empty(n, dtype=np.float32)

    def work(s0):
        out[s0:s0 + blk] = _normal_block(seed, stream, flat[s0:s0 + blk], std)

    list(_pool().map(work, range(0, n, blk)))
    return out.reshape(idx.shape)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even.  Finite inputs."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class ScanConfig:
    name: str
    batch: int
    L: int
    dim: int
    N: int
    io: str            # "f32" or "bf16"
    gate: bool
    seed: int
    filler: bool = False  # the long-sequence selective-copying-like u


@dataclass(frozen=True)
class StepConfig:
    name: str
    batch: int
    dim: int
    N: int
    io: str
    gate: bool
    seed: int
    steps: int
    state_std: float = 0.1


SCAN_CONFIGS: Dict[str, ScanConfig] = {
    "tiny": ScanConfig("tiny", 1, 256, 64, 16, "f32", False, 0),
    "mamba130m": ScanConfig("mamba130m", 8, 2048, 1536, 16, "bf16", True, 1),
    "mamba1p4b": ScanConfig("mamba1p4b", 8, 2048, 4096, 16, "bf16", True, 2),
    "longseq": ScanConfig("longseq", 4, 65536, 2048, 16, "bf16", False, 3, filler=True),
}
STEP_CONFIGS: Dict[str, StepConfig] = {
    "decode": StepConfig("decode", 256, 5120, 16, "bf16", True, 4, 1000),
}


def channel_params(seed: int, dim: int, N: int, channels: Optional[Sequence[int]] = None):
    """A (k, N), D (k,), delta_bias (k,) for the selected channels (all if None)."""
    ch = np.arange(dim) if channels is None else np.asarray(channels, dtype=np.int64)
    lo, hi = np.log(1e-3), np.log(1e-1)
    dt = np.exp(lo + (hi - lo) * uniform(seed, S_DT, ch))
    bias = np.log(np.expm1(dt)).astype(np.float32)  # softplus^-1(dt)
    D = normal(seed, S_D, ch)
    A = np.tile(-(np.arange(N, dtype=np.float32) + 1.0), (len(ch), 1))
    return A, D, bias


def _io(x: np.ndarray, io: str) -> np.ndarray:
    return to_bf16_bits(x) if io == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def filler_positions(seed: int, batch: int, L: int, count: int = 16) -> np.ndarray:
    """(batch, count) distinct positions per sequence, sorted."""
    out = np.empty((batch, count), dtype=np.int64)
    for b in range(batch):
        picked = []
        j = 0
        while len(picked) < count:
            p = int(uniform(seed, S_FILLER, np.array([1_000_000 + b * 4096 + j]))[0] * L)
            if p not in picked:
                picked.append(p)
            j += 1
        out[b] = sorted(picked)
    return out


def scan_inputs(cfg: ScanConfig, channels: Optional[Sequence[int]] = None) -> dict:
    """Inputs of one scan workload.

    With ``channels`` given, u / delta / z and the per-channel parameters are
    generated for those channels only (in that order); B and C are always whole.
    Tensors in the io dtype are returned as float32 arrays ("f32") or uint16
    bf16 bit patterns ("bf16"); A, D and delta_bias are always float32.
    """
    b, L, dim, N = cfg.batch, cfg.L, cfg.dim, cfg.N
    ch = np.arange(dim) if channels is None else np.asarray(channels, dtype=np.int64)
    k = len(ch)
    A, D, bias = channel_params(cfg.seed, dim, N, ch)

    def big(stream):
        out = np.empty((b, L, k), dtype=np.uint16 if cfg.io == "bf16" else np.float32)
        rows_per = max(1, (1 << 24) // max(k, 1))
        for bi in range(b):
            for t0 in range(0, L, rows_per):
                t1 = min(L, t0 + rows_per)
                idx = ((bi * L + np.arange(t0, t1, dtype=np.int64))[:, None] * dim + ch[None, :])
                out[bi, t0:t1] = _io(normal(cfg.seed, stream, idx), cfg.io)
        return out

    if cfg.filler:
        filler = normal(cfg.seed, S_U, ch)
        u = np.empty((b, L, k), dtype=np.uint16 if cfg.io == "bf16" else np.float32)
        u[...] = _io(filler, cfg.io)[None, None, :]
        pos = filler_positions(cfg.seed, b, L)
        for bi in range(b):
            for j, p in enumerate(pos[bi]):
                idx = (bi * 16 + j) * dim + ch
                u[bi, p] = _io(normal(cfg.seed, S_DATA, idx), cfg.io)
    else:
        u = big(S_U)
    delta = big(S_DELTA)
    bc_idx = np.arange(b * L * N, dtype=np.int64).reshape(b, L, N)
    Bm = _io(normal(cfg.seed, S_B, bc_idx), cfg.io)
    Cm = _io(normal(cfg.seed, S_C, bc_idx), cfg.io)
    z = big(S_Z) if cfg.gate else None
    return dict(u=u, delta=delta, A=A, B=Bm, C=Cm, D=D, z=z, delta_bias=bias,
                channels=ch, io=cfg.io)


def step_state0(cfg: StepConfig, channels: Optional[Sequence[int]] = None) -> np.ndarray:
    ch = np.arange(cfg.dim) if channels is None else np.asarray(channels, dtype=np.int64)
    idx = (np.arange(cfg.batch, dtype=np.int64)[:, None, None] * cfg.dim + ch[None, :, None]) * cfg.N \
        + np.arange(cfg.N, dtype=np.int64)[None, None, :]
    return normal(cfg.seed, S_STATE0, idx, std=cfg.state_std)


def step_inputs(cfg: StepConfig, step: int, channels: Optional[Sequence[int]] = None) -> dict:
    """Per-token inputs of decode step ``step`` (0-based); same conventions as scan_inputs."""
    ch = np.arange(cfg.dim) if channels is None else np.asarray(channels, dtype=np.int64)
    base = 16 + 8 * step
    idx = np.arange(cfg.batch, dtype=np.int64)[:, None] * cfg.dim + ch[None, :]
    bn = np.arange(cfg.batch * cfg.N, dtype=np.int64).reshape(cfg.batch, cfg.N)
    return dict(
        u=_io(normal(cfg.seed, base + S_U, idx), cfg.io),
        delta=_io(normal(cfg.seed, base + S_DELTA, idx), cfg.io),
        B=_io(normal(cfg.seed, base + S_B, bn), cfg.io),
        C=_io(normal(cfg.seed, base + S_C, bn), cfg.io),
        z=_io(normal(cfg.seed, base + S_Z, idx), cfg.io) if cfg.gate else None,
        channels=ch, io=cfg.io)


def step_inputs_range(cfg: StepConfig, s0: int, s1: int) -> list:
    """step_inputs for steps s0 .. s1 - 1 (all channels), generated in parallel
    on the host threads; the same values as one call per step."""
    return list(_pool().map(lambda s: step_inputs(cfg, s), range(s0, s1)))


def as_f64(x: Optional[np.ndarray], io: str) -> Optional[np.ndarray]:
    """The exact values a tensor in the io dtype holds, as float64."""
    if x is None:
        return None
    if io == "bf16" and x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


# ------------------------------------------------- the block's convolution

S_CONV_W, S_CONV_B, S_CONV_X, S_CONV_WIN = range(21, 25)


@dataclass(frozen=True)
class ConvConfig:
    name: str
    batch: int
    L: int          # 0 for the decoding workload (one token per step)
    dim: int
    k: int
    io: str
    seed: int
    steps: int = 0  # decoding steps


CONV_CONFIGS: Dict[str, ConvConfig] = {
    # the convolution in front of the Mamba-130M-shaped scan layer
    "conv130m": ConvConfig("conv130m", 8, 2048, 1536, 4, "bf16", 5),
    "conv_tiny": ConvConfig("conv_tiny", 2, 100, 70, 4, "f32", 6),
    # one decoding step of the convolution at the decode workload's width
    "conv_decode": ConvConfig("conv_decode", 256, 0, 5120, 4, "bf16", 7, steps=100),
}


def conv_params(seed: int, dim: int, k: int):
    """Depthwise weights (dim, k) and bias (dim,), U(-1/sqrt(k), 1/sqrt(k)) float32
    (the usual fan-in bound of a convolution with k taps per channel)."""
    bound = 1.0 / np.sqrt(k)
    w = (2.0 * uniform(seed, S_CONV_W, np.arange(dim * k)) - 1.0) * bound
    b = (2.0 * uniform(seed, S_CONV_B, np.arange(dim)) - 1.0) * bound
    return w.reshape(dim, k).astype(np.float32), b.astype(np.float32)


def conv_inputs(cfg: ConvConfig, channels: Optional[Sequence[int]] = None) -> dict:
    """x (batch, L, len(channels)) in the io dtype (bf16 bits or fp32) ~ N(0, 1),
    and the weights and bias of those channels."""
    ch = np.arange(cfg.dim) if channels is None else np.asarray(channels, dtype=np.int64)
    w, b = conv_params(cfg.seed, cfg.dim, cfg.k)
    idx = (np.arange(cfg.batch * cfg.L, dtype=np.int64)[:, None] * cfg.dim + ch[None, :])
    x = _io(normal(cfg.seed, S_CONV_X, idx), cfg.io).reshape(cfg.batch, cfg.L, len(ch))
    return dict(x=x, w=w[ch], bias=b[ch], io=cfg.io, channels=ch)


def conv_window0(cfg: ConvConfig) -> np.ndarray:
    """A decoding window (batch, k - 1, dim) of earlier inputs ~ N(0, 1), io dtype."""
    n = cfg.batch * (cfg.k - 1) * cfg.dim
    return _io(normal(cfg.seed, S_CONV_WIN, np.arange(n)), cfg.io).reshape(
        cfg.batch, cfg.k - 1, cfg.dim)


def conv_step_inputs(cfg: ConvConfig, step: int) -> np.ndarray:
    """The token (batch, dim) of decoding step `step`, io dtype."""
    idx = np.arange(cfg.batch * cfg.dim, dtype=np.int64) + (step + 1) * cfg.batch * cfg.dim
    return _io(normal(cfg.seed, S_CONV_X, idx), cfg.io).reshape(cfg.batch, cfg.dim)


# ----------------------------------------------- Mamba-2 / SSD (scalar decay)

S_SSD_A, S_SSD_DT, S_SSD_D, S_SSD_X, S_SSD_DTR, S_SSD_B, S_SSD_C, S_SSD_Z = range(31, 39)


@dataclass(frozen=True)
class SSDConfig:
    name: str
    batch: int
    L: int
    nheads: int
    P: int          # channels per head
    N: int          # state size
    io: str
    gate: bool
    seed: int


SSD_CONFIGS: Dict[str, SSDConfig] = {
    "ssd_tiny": SSDConfig("ssd_tiny", 2, 150, 3, 64, 64, "bf16", True, 8),
    # a Mamba-2-130M-shaped layer: d_model 768, expand 2 -> 1536 = 24 heads x 64, N 128
    "ssd130m": SSDConfig("ssd130m", 8, 2048, 24, 64, 128, "bf16", True, 9),
}


def ssd_head_params(seed: int, nheads: int):
    """A (nheads,) = -U[1, 16], D ~ N(0, 1), dt_bias = softplus^-1(dt) with dt
    log-uniform in [1e-3, 1e-1] (the step-size range of the scan's workloads)."""
    h = np.arange(nheads)
    A = -(1.0 + 15.0 * uniform(seed, S_SSD_A, h)).astype(np.float32)
    lo, hi = np.log(1e-3), np.log(1e-1)
    dt = np.exp(lo + (hi - lo) * uniform(seed, S_SSD_DT, h))
    dt_bias = np.log(np.expm1(dt)).astype(np.float32)
    D = normal(seed, S_SSD_D, h)
    return A, D, dt_bias


def ssd_inputs(cfg: SSDConfig, heads: Optional[Sequence[int]] = None) -> dict:
    """x, z (batch, L, len(heads), P) and dt (batch, L, len(heads)) in the io dtype
    (dt raw in fp32 always -- it is one value per token and head), B, C
    (batch, L, N) ~ N(0, 1) in the io dtype, head parameters in fp32.  With
    `heads`, only those heads are generated (B and C whole)."""
    b, L, H, P, N = cfg.batch, cfg.L, cfg.nheads, cfg.P, cfg.N
    hs = np.arange(H) if heads is None else np.asarray(heads, dtype=np.int64)
    A, D, dt_bias = ssd_head_params(cfg.seed, H)
    tok = np.arange(b * L, dtype=np.int64)
    xi = ((tok[:, None, None] * H + hs[None, :, None]) * P + np.arange(P)[None, None, :])
    x = _io(normal(cfg.seed, S_SSD_X, xi), cfg.io).reshape(b, L, len(hs), P)
    z = _io(normal(cfg.seed, S_SSD_Z, xi), cfg.io).reshape(b, L, len(hs), P) if cfg.gate else None
    dt = normal(cfg.seed, S_SSD_DTR, tok[:, None] * H + hs[None, :]).reshape(b, L, len(hs))
    bc = np.arange(b * L * N, dtype=np.int64).reshape(b, L, N)
    Bm = _io(normal(cfg.seed, S_SSD_B, bc), cfg.io)
    Cm = _io(normal(cfg.seed, S_SSD_C, bc), cfg.io)
    return dict(x=x, z=z, dt=dt.astype(np.float32), A=A[hs], D=D[hs], dt_bias=dt_bias[hs],
                B=Bm, C=Cm, io=cfg.io, heads=hs)
