"""The five workloads at full size on the GPU, compared with the fp64 oracle on
every channel.

The scan workloads (the Mamba-130M and Mamba-1.4B layers, the long-sequence
layer) run as the benchmark launches them: one full-size call with the
library's own kernel choice.  The oracle then recomputes every channel, a
block of channels at a time so that host memory stays bounded, from the same
input bits.  The decode workload runs its 1000 consecutive steps on the whole
256 x 5120 x 16 state, and the oracle steps the same state alongside; y is
compared at steps 1, 10, 100 and 1000, and the state after the last step.

The acceptance measure for bf16 I/O with an fp32 state is the relative RMS
error <= 1e-2, asserted over the whole tensor and for every channel on its
own (over its batch entries and tokens), so that a wrong channel tile cannot
hide inside a correct whole.
"""
import functools
import time

import numpy as np
import pytest
import torch

import oracle
import selective_state_space_66_amd as ssm
import workloads as W
from gpu_helpers import DEV, BF16_TOL, scan_gpu, to_dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


class _PerChannel:
    """Running sums for the relative RMS error, whole and per channel; the
    channel axis is given per tensor."""

    def __init__(self, nch):
        self.err = np.zeros(nch)
        self.ref = np.zeros(nch)

    def add(self, got, ref, ch_axis, ch0):
        axes = tuple(i for i in range(got.ndim) if i != ch_axis)
        d = got - ref
        k = got.shape[ch_axis]
        self.err[ch0:ch0 + k] += np.sum(d * d, axis=axes)
        self.ref[ch0:ch0 + k] += np.sum(ref * ref, axis=axes)

    def check(self, what):
        assert np.all(np.isfinite(self.err)), f"{what}: non-finite values"
        whole = float(np.sqrt(self.err.sum() / max(self.ref.sum(), 1e-300)))
        per = np.sqrt(self.err / np.maximum(self.ref, 1e-300))
        worst = int(np.argmax(per))
        assert whole <= BF16_TOL, f"{what}: relative RMS error {whole:.3e} > {BF16_TOL}"
        assert per[worst] <= BF16_TOL, \
            f"{what}: channel {worst} relative RMS error {per[worst]:.3e} > {BF16_TOL}"
        return whole, float(per[worst])


@functools.lru_cache(maxsize=1)
def _scan_workload(name):
    cfg = W.SCAN_CONFIGS[name]
    t = time.perf_counter()
    inp = W.scan_inputs(cfg)
    _say(f"[{name}] inputs generated in {time.perf_counter() - t:.1f} s")
    return cfg, inp


def _bf16_to_f64(bits):
    return W.bf16_bits_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("mode", ["zoh", "euler"])
@pytest.mark.parametrize("name", ["mamba130m", "mamba1p4b", "longseq"])
def test_scan_workload_every_channel(name, mode):
    cfg, inp = _scan_workload(name)
    b, L, dim, N = cfg.batch, cfg.L, cfg.dim, cfg.N
    _say(f"[{name}] {mode}: full-size launch ({ssm.scan_kernel_name(b, L, dim, N)})")
    y, last = scan_gpu(inp, mode)
    yb = y.view(torch.int16).cpu().numpy().view(np.uint16)  # the bf16 bits, (b, L, dim)
    lh = last.cpu().numpy().astype(np.float64)
    del y, last
    torch.cuda.empty_cache()
    assert yb.shape == (b, L, dim) and lh.shape == (b, dim, N)
    ys, ls = _PerChannel(dim), _PerChannel(dim)
    step = max(8, (1 << 25) // (b * L))  # about 32M elements of each (b, L, k) block
    t = time.perf_counter()
    for c0 in range(0, dim, step):
        c1 = min(dim, c0 + step)
        sl = slice(c0, c1)
        yr, lr = oracle.scan_fwd(
            _bf16_to_f64(inp["u"][:, :, sl]), _bf16_to_f64(inp["delta"][:, :, sl]),
            inp["A"][sl], _bf16_to_f64(inp["B"]), _bf16_to_f64(inp["C"]), D=inp["D"][sl],
            z=_bf16_to_f64(inp["z"][:, :, sl]) if inp["z"] is not None else None,
            delta_bias=inp["delta_bias"][sl], dt_mode=mode)
        ys.add(_bf16_to_f64(yb[:, :, sl]), yr, 2, c0)
        ls.add(lh[:, sl], lr, 1, c0)
    ey, eyc = ys.check(f"{name} y {mode}")
    el, elc = ls.check(f"{name} last_state {mode}")
    _say(f"[{name}] {mode}: oracle over all {dim} channels in {time.perf_counter() - t:.1f} s; "
         f"rel-rms y {ey:.2e} (worst channel {eyc:.2e}), last_state {el:.2e} (worst {elc:.2e})")


@pytest.mark.parametrize("shape", [(1, 2048, 1024), (1, 2048, 1536), (1, 65536, 128)])
def test_time_parallel_shapes_every_channel(shape):
    """The narrow shapes the benchmark times on the time-parallel kernels (the
    pages' speed-benchmark shape, the Mamba-130M layer at batch 1, a long
    narrow sequence), every channel against the oracle, both rules."""
    b, L, dim = shape
    cfg = W.ScanConfig(f"narrow{b}x{L}x{dim}", b, L, dim, 16, "bf16", True, 7)
    inp = W.scan_inputs(cfg)
    f = lambda k: _bf16_to_f64(inp[k])
    for mode in ("zoh", "euler"):
        _say(f"[{cfg.name}] {mode} ({ssm.scan_kernel_name(b, L, dim, 16)})")
        y, last = scan_gpu(inp, mode)
        yg = y.float().cpu().numpy().astype(np.float64)
        lg = last.cpu().numpy().astype(np.float64)
        yr, lr = oracle.scan_fwd(f("u"), f("delta"), inp["A"], f("B"), f("C"), D=inp["D"],
                                 z=f("z"), delta_bias=inp["delta_bias"], dt_mode=mode)
        ys, ls = _PerChannel(dim), _PerChannel(dim)
        ys.add(yg, yr, 2, 0)
        ls.add(lg, lr, 1, 0)
        ys.check(f"{cfg.name} y {mode}")
        ls.check(f"{cfg.name} last_state {mode}")


@pytest.mark.parametrize("mode", ["zoh", "euler"])
def test_decode_workload_thousand_steps(mode):
    """The decode workload: 1000 consecutive steps on the whole state (256 x
    5120 x 16, fp32), each with fresh bf16 tokens; the oracle steps an fp64
    copy of the same initial state with the same tokens."""
    cfg = W.STEP_CONFIGS["decode"]
    A, D, bias = W.channel_params(cfg.seed, cfg.dim, cfg.N)
    st0 = W.step_state0(cfg)
    st = to_dev(st0, "f32")
    ref_st = st0.astype(np.float64)
    Ad, Dd, bd = to_dev(A, "f32"), to_dev(D, "f32"), to_dev(bias, "f32")
    checks = {1, 10, 100, 1000}
    assert cfg.steps == 1000
    f = lambda x: W.as_f64(x, cfg.io)
    t0 = time.perf_counter()
    batch = 50
    for s0 in range(0, cfg.steps, batch):
        toks = W.step_inputs_range(cfg, s0, min(cfg.steps, s0 + batch))
        for i, inp in enumerate(toks):
            s = s0 + i
            y = ssm.step(st, to_dev(inp["u"], cfg.io), to_dev(inp["delta"], cfg.io), Ad,
                         to_dev(inp["B"], cfg.io), to_dev(inp["C"], cfg.io), D=Dd,
                         z=to_dev(inp["z"], cfg.io), delta_bias=bd, dt_mode=mode)
            yr, ref_st = oracle.step(ref_st, f(inp["u"]), f(inp["delta"]), A, f(inp["B"]),
                                     f(inp["C"]), D=D, z=f(inp["z"]), delta_bias=bias,
                                     dt_mode=mode, inplace=True)
            if s + 1 in checks:
                acc = _PerChannel(cfg.dim)
                acc.add(y.float().cpu().numpy().astype(np.float64), yr, 1, 0)
                e, ec = acc.check(f"decode y at step {s + 1} {mode}")
                _say(f"[decode] {mode} step {s + 1}: rel-rms y {e:.2e} (worst channel {ec:.2e}), "
                     f"{time.perf_counter() - t0:.1f} s")
    acc = _PerChannel(cfg.dim)
    acc.add(st.cpu().numpy().astype(np.float64), ref_st, 1, 0)
    e, ec = acc.check(f"decode state after 1000 steps {mode}")
    _say(f"[decode] {mode}: state after 1000 steps rel-rms {e:.2e} (worst channel {ec:.2e})")
