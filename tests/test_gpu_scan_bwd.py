"""GPU parity of ssm_scan_bwd against the oracle's backward pass (fp64, every
state kept), which is pinned by finite differences of the pinned forward.

Tolerances, per gradient tensor (each entry is a sum of many terms -- over
states, tokens, channels or batch entries -- so the error is measured against
the tensor's scale, not entry by entry):
  fp32 io: max |g - g_ref| <= 2e-5 * (1 + max |g_ref|).  An fp32 sum of n terms
           is off by up to about n eps times the largest term; the cases here
           sum at most a few thousand terms (dA over 3000 tokens), where the
           typical error, sqrt(n) eps, is ~3e-6 -- the bound leaves a factor of
           about 10 over the largest error measured (2.3e-6);
  bf16 io: relative RMS <= 1e-2 (the forward's bf16 bound; the inputs and dy
           are the same bf16 bits on both sides, and the gradients are
           rounded to bf16 once).
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import DEV, f64, rel_rms, to_dev, to_host64
import oracle
import selective_state_space_66_amd as ssm

pytestmark = pytest.mark.gpu

FP32_GRAD_TOL = 2e-5


def _cfg(batch, L, dim, N, io, gate, seed):
    return W.ScanConfig(f"g{batch}x{L}x{dim}x{N}", batch, L, dim, N, io, gate, seed)


def _dy(shape, io, seed):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=shape).astype(np.float32)
    return W.to_bf16_bits(x) if io == "bf16" else x


def _run(inp, mode, dy, softplus=True, h0=None, dlast=None, use_D=True, use_bias=True):
    io = inp["io"]
    g = ssm.scan_bwd(to_dev(inp["u"], io), to_dev(inp["delta"], io), to_dev(inp["A"], "f32"),
                     to_dev(inp["B"], io), to_dev(inp["C"], io), to_dev(dy, io),
                     D=to_dev(inp["D"], "f32") if use_D else None,
                     z=to_dev(inp["z"], io) if inp["z"] is not None else None,
                     delta_bias=to_dev(inp["delta_bias"], "f32") if use_bias else None,
                     softplus=softplus, dt_mode=mode,
                     h0=None if h0 is None else to_dev(h0, "f32"),
                     dlast=None if dlast is None else to_dev(dlast, "f32"))
    torch.cuda.synchronize()
    r = oracle.scan_bwd(f64(inp["u"], io), f64(inp["delta"], io), inp["A"], f64(inp["B"], io),
                        f64(inp["C"], io), f64(dy, io), D=inp["D"] if use_D else None,
                        z=f64(inp["z"], io) if inp["z"] is not None else None,
                        delta_bias=inp["delta_bias"] if use_bias else None, softplus=softplus,
                        dt_mode=mode, h0=None if h0 is None else h0.astype(np.float64),
                        dlast=None if dlast is None else dlast.astype(np.float64))
    return g, r


def _compare(g, r, io, what=""):
    errs = {}
    for k, ref in r.items():
        if ref is None:
            assert g[k] is None, k
            continue
        got = to_host64(g[k])
        assert got.shape == ref.shape, k
        assert np.all(np.isfinite(got)), f"{what} {k}: not finite"
        if io == "f32":
            errs[k] = float(np.abs(got - ref).max() / (1.0 + np.abs(ref).max()))
        else:
            errs[k] = rel_rms(got, ref)
    print(what, " ".join(f"{k}={v:.1e}" for k, v in errs.items()), flush=True)
    tol = FP32_GRAD_TOL if io == "f32" else 1e-2
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{what}: {bad}"
    return errs


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["zoh", "euler"])
@pytest.mark.parametrize("gate", [True, False])
def test_bwd_ragged(io, mode, gate):
    """3 channel tiles (the last 2 wide), 7 chunks (the last 3 long), h0 and
    the gradient of the final state."""
    inp = W.scan_inputs(_cfg(2, 99, 34, 16, io, gate, seed=90))
    dy = _dy((2, 99, 34), io, 91)
    rng = np.random.default_rng(92)
    h0 = rng.normal(size=(2, 34, 16)).astype(np.float32)
    dlast = rng.normal(size=(2, 34, 16)).astype(np.float32)
    g, r = _run(inp, mode, dy, h0=h0, dlast=dlast)
    _compare(g, r, io, f"{io} {mode} gate={gate}")


@pytest.mark.parametrize("N", [1, 3, 4, 8, 12, 16])
@pytest.mark.parametrize("mode", ["zoh", "euler"])
def test_bwd_state_sizes(N, mode):
    inp = W.scan_inputs(_cfg(2, 40, 20, N, "f32", True, seed=93 + N))
    dy = _dy((2, 40, 20), "f32", 94)
    g, r = _run(inp, mode, dy)
    _compare(g, r, "f32", f"N={N} {mode}")


@pytest.mark.parametrize("mode", ["zoh", "euler"])
def test_bwd_softplus_off_and_optional_inputs_absent(mode):
    inp = W.scan_inputs(_cfg(1, 50, 40, 16, "f32", False, seed=95))
    inp["delta"] = (np.abs(inp["delta"]) * 0.05).astype(np.float32)
    dy = _dy((1, 50, 40), "f32", 96)
    g, r = _run(inp, mode, dy, softplus=False, use_D=False, use_bias=False)
    _compare(g, r, "f32", f"softplus off {mode}")


def test_bwd_small_and_zero_A():
    """A = 0 (the limit Delta B) and slow channels (|Delta A| small: phi and
    phi' from their series)."""
    inp = W.scan_inputs(_cfg(2, 60, 48, 16, "f32", True, seed=97))
    A = inp["A"].copy()
    A[3, 5] = 0.0
    A[20, :] = -0.01
    A[40, 2] = 0.2
    inp["A"] = A
    dy = _dy((2, 60, 48), "f32", 98)
    for mode in ("zoh", "euler"):
        g, r = _run(inp, mode, dy)
        _compare(g, r, "f32", f"small A {mode}")


def test_bwd_long_sequence():
    inp = W.scan_inputs(_cfg(1, 3000, 32, 16, "f32", True, seed=99))
    dy = _dy((1, 3000, 32), "f32", 100)
    for mode in ("zoh", "euler"):
        g, r = _run(inp, mode, dy)
        _compare(g, r, "f32", f"long {mode}")


def test_bwd_deterministic_and_empty():
    inp = W.scan_inputs(_cfg(2, 70, 50, 16, "bf16", True, seed=101))
    dy = _dy((2, 70, 50), "bf16", 102)
    args = (to_dev(inp["u"], "bf16"), to_dev(inp["delta"], "bf16"), to_dev(inp["A"], "f32"),
            to_dev(inp["B"], "bf16"), to_dev(inp["C"], "bf16"), to_dev(dy, "bf16"))
    kw = dict(D=to_dev(inp["D"], "f32"), z=to_dev(inp["z"], "bf16"),
              delta_bias=to_dev(inp["delta_bias"], "f32"))
    g1 = ssm.scan_bwd(*args, **kw)
    g2 = ssm.scan_bwd(*args, **kw)
    torch.cuda.synchronize()
    for k in g1:
        if g1[k] is not None:
            assert torch.equal(g1[k], g2[k]), k
    # no tokens: dh0 = dlast, everything else zero
    A = torch.full((8, 16), -1.0, device=DEV)
    e = torch.zeros((2, 0, 8), device=DEV)
    eb = torch.zeros((2, 0, 16), device=DEV)
    dl = torch.randn((2, 8, 16), device=DEV)
    g = ssm.scan_bwd(e, e, A, eb, eb, e, D=torch.ones(8, device=DEV), h0=torch.zeros_like(dl),
                     dlast=dl)
    torch.cuda.synchronize()
    assert torch.equal(g["dh0"], dl) and torch.all(g["dA"] == 0) and torch.all(g["dD"] == 0)


def test_bwd_full_size_sampled():
    """The Mamba-130M layer at full size: dy for sampled channels only (zero
    elsewhere), so the oracle's backward on those channels is the exact
    reference for du, d delta, dz, dA, dD, d bias there, and dB, dC equal the
    sums over the sampled channels."""
    cfg = W.SCAN_CONFIGS["mamba130m"]
    inp = W.scan_inputs(cfg)
    ch = np.array([0, 1, 17, 600, 1535])
    dy = np.zeros((cfg.batch, cfg.L, cfg.dim), dtype=np.uint16)
    dsub = _dy((cfg.batch, cfg.L, len(ch)), "bf16", 103)
    dy[:, :, ch] = dsub
    sub = W.scan_inputs(cfg, channels=ch)
    chd = torch.from_numpy(ch).to(DEV)
    for mode in ("zoh", "euler"):
        g = ssm.scan_bwd(to_dev(inp["u"], "bf16"), to_dev(inp["delta"], "bf16"),
                         to_dev(inp["A"], "f32"), to_dev(inp["B"], "bf16"),
                         to_dev(inp["C"], "bf16"), to_dev(dy, "bf16"), D=to_dev(inp["D"], "f32"),
                         z=to_dev(inp["z"], "bf16"), delta_bias=to_dev(inp["delta_bias"], "f32"),
                         dt_mode=mode)
        torch.cuda.synchronize()
        r = oracle.scan_bwd(f64(sub["u"], "bf16"), f64(sub["delta"], "bf16"), sub["A"],
                            f64(sub["B"], "bf16"), f64(sub["C"], "bf16"), f64(dsub, "bf16"),
                            D=sub["D"], z=f64(sub["z"], "bf16"), delta_bias=sub["delta_bias"],
                            dt_mode=mode)
        got = {"du": g["du"].index_select(2, chd), "ddelta": g["ddelta"].index_select(2, chd),
               "dz": g["dz"].index_select(2, chd), "dA": g["dA"].index_select(0, chd),
               "dD": g["dD"].index_select(0, chd), "ddelta_bias": g["ddelta_bias"].index_select(0, chd),
               "dB": g["dB"], "dC": g["dC"], "dh0": None}
        _compare(got, r, "bf16", f"full {mode}")
        del g
        torch.cuda.empty_cache()


# ------------------------------------------------- the training forward's checkpoints

@pytest.mark.parametrize("kernel", ["seq1", "seq2", "seq4", "tpar", "wave", "wave4"])
@pytest.mark.parametrize("mode", ["zoh", "euler"])
def test_train_forward_checkpoints(kernel, mode):
    """scan_fwd_train gives scan_fwd's y and last_state bit for bit, and its
    checkpoint j is the state before token 16 j: the oracle's final state of
    the sequence cut there (j = 0: h0).  A ragged channel tile, a ragged last
    chunk, a zero and a slow channel (both ZOH forms)."""
    inp = W.scan_inputs(_cfg(2, 99, 34, 16, "f32", True, seed=110))
    A = inp["A"].copy()
    A[5, 2] = 0.0
    A[9, :] = -0.2
    inp["A"] = A
    h0 = np.random.default_rng(111).normal(size=(2, 34, 16)).astype(np.float32)
    args = (to_dev(inp["u"], "f32"), to_dev(inp["delta"], "f32"), to_dev(inp["A"], "f32"),
            to_dev(inp["B"], "f32"), to_dev(inp["C"], "f32"))
    kw = dict(D=to_dev(inp["D"], "f32"), z=to_dev(inp["z"], "f32"),
              delta_bias=to_dev(inp["delta_bias"], "f32"), dt_mode=mode, h0=to_dev(h0, "f32"))
    y, last, ck = ssm.scan_fwd_train(*args, kernel=kernel, **kw)
    y2, last2 = ssm.scan_fwd(*args, kernel=kernel, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(last, last2)
    ckh = to_host64(ck)
    assert ckh.shape == (2, 7, 34, 16)
    for j in range(7):
        t = 16 * j
        sub = dict(inp)
        for k in ("u", "delta", "z"):
            sub[k] = inp[k][:, :t]
        for k in ("B", "C"):
            sub[k] = inp[k][:, :t]
        _, lr = oracle.scan_fwd(sub["u"], sub["delta"], sub["A"], sub["B"], sub["C"], D=sub["D"],
                                z=sub["z"], delta_bias=sub["delta_bias"], dt_mode=mode,
                                h0=h0.astype(np.float64))
        err = np.abs(ckh[:, j] - lr) / (1.0 + np.abs(lr))
        assert err.max() <= 1e-4, f"checkpoint {j}: {err.max():.2e}"


@pytest.mark.parametrize("kernel", [None, "tpar", "wave", "wave4"])
@pytest.mark.parametrize("N", [3, 8])
def test_train_forward_checkpoints_small_state(kernel, N):
    """State sizes below 16 (padded state groups in the sequential kernel,
    element loads in the time-parallel one), ZOH: checkpoints against the
    oracle, and the backward from them against the oracle's backward."""
    inp = W.scan_inputs(_cfg(2, 70, 20, N, "f32", True, seed=116 + N))
    dy = _dy((2, 70, 20), "f32", 117)
    args = (to_dev(inp["u"], "f32"), to_dev(inp["delta"], "f32"), to_dev(inp["A"], "f32"),
            to_dev(inp["B"], "f32"), to_dev(inp["C"], "f32"))
    kw = dict(D=to_dev(inp["D"], "f32"), z=to_dev(inp["z"], "f32"),
              delta_bias=to_dev(inp["delta_bias"], "f32"))
    _, _, ck = ssm.scan_fwd_train(*args, kernel=kernel, **kw)
    g = ssm.scan_bwd(*args, to_dev(dy, "f32"), ckpt=ck, **kw)
    torch.cuda.synchronize()
    ckh = to_host64(ck)
    for j in range(5):
        t = 16 * j
        _, lr = oracle.scan_fwd(inp["u"][:, :t], inp["delta"][:, :t], inp["A"], inp["B"][:, :t],
                                inp["C"][:, :t], D=inp["D"], z=inp["z"][:, :t],
                                delta_bias=inp["delta_bias"])
        err = np.abs(ckh[:, j] - lr) / (1.0 + np.abs(lr))
        assert err.max() <= 1e-4, f"N={N} checkpoint {j}: {err.max():.2e}"
    r = oracle.scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], dy, D=inp["D"],
                        z=inp["z"], delta_bias=inp["delta_bias"])
    _compare(g, r, "f32", f"small state N={N} {kernel}")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["zoh", "euler"])
def test_bwd_from_forward_checkpoints(io, mode):
    """ssm_scan_bwd_ex with the training forward's checkpoints (no forward
    sweep in the backward) against the oracle's backward."""
    inp = W.scan_inputs(_cfg(2, 99, 34, 16, io, True, seed=112))
    dy = _dy((2, 99, 34), io, 113)
    rng = np.random.default_rng(114)
    h0 = rng.normal(size=(2, 34, 16)).astype(np.float32)
    dlast = rng.normal(size=(2, 34, 16)).astype(np.float32)
    args = (to_dev(inp["u"], io), to_dev(inp["delta"], io), to_dev(inp["A"], "f32"),
            to_dev(inp["B"], io), to_dev(inp["C"], io))
    kw = dict(D=to_dev(inp["D"], "f32"), z=to_dev(inp["z"], io),
              delta_bias=to_dev(inp["delta_bias"], "f32"), dt_mode=mode, h0=to_dev(h0, "f32"))
    _, _, ck = ssm.scan_fwd_train(*args, **kw)
    g = ssm.scan_bwd(*args, to_dev(dy, io), dlast=to_dev(dlast, "f32"), ckpt=ck, **kw)
    torch.cuda.synchronize()
    r = oracle.scan_bwd(f64(inp["u"], io), f64(inp["delta"], io), inp["A"], f64(inp["B"], io),
                        f64(inp["C"], io), f64(dy, io), D=inp["D"], z=f64(inp["z"], io),
                        delta_bias=inp["delta_bias"], dt_mode=mode, h0=h0.astype(np.float64),
                        dlast=dlast.astype(np.float64))
    _compare(g, r, io, f"from checkpoints {io} {mode}")


def test_bwd_from_forward_checkpoints_full_size_sampled():
    """The Mamba-130M layer, training forward then backward from its
    checkpoints (the launch configuration bench.py times): dy on sampled
    channels only, against the oracle's backward on those channels."""
    cfg = W.SCAN_CONFIGS["mamba130m"]
    inp = W.scan_inputs(cfg)
    ch = np.array([0, 1, 17, 600, 1535])
    dy = np.zeros((cfg.batch, cfg.L, cfg.dim), dtype=np.uint16)
    dsub = _dy((cfg.batch, cfg.L, len(ch)), "bf16", 115)
    dy[:, :, ch] = dsub
    sub = W.scan_inputs(cfg, channels=ch)
    chd = torch.from_numpy(ch).to(DEV)
    args = (to_dev(inp["u"], "bf16"), to_dev(inp["delta"], "bf16"), to_dev(inp["A"], "f32"),
            to_dev(inp["B"], "bf16"), to_dev(inp["C"], "bf16"))
    kw = dict(D=to_dev(inp["D"], "f32"), z=to_dev(inp["z"], "bf16"),
              delta_bias=to_dev(inp["delta_bias"], "f32"), dt_mode="zoh")
    _, _, ck = ssm.scan_fwd_train(*args, **kw)
    g = ssm.scan_bwd(*args, to_dev(dy, "bf16"), ckpt=ck, **kw)
    torch.cuda.synchronize()
    r = oracle.scan_bwd(f64(sub["u"], "bf16"), f64(sub["delta"], "bf16"), sub["A"],
                        f64(sub["B"], "bf16"), f64(sub["C"], "bf16"), f64(dsub, "bf16"),
                        D=sub["D"], z=f64(sub["z"], "bf16"), delta_bias=sub["delta_bias"],
                        dt_mode="zoh")
    got = {"du": g["du"].index_select(2, chd), "ddelta": g["ddelta"].index_select(2, chd),
           "dz": g["dz"].index_select(2, chd), "dA": g["dA"].index_select(0, chd),
           "dD": g["dD"].index_select(0, chd), "ddelta_bias": g["ddelta_bias"].index_select(0, chd),
           "dB": g["dB"], "dC": g["dC"], "dh0": None}
    _compare(got, r, "bf16", "full from checkpoints")


# ------------------------------------------------- lengths and document starts

def _varlen(batch, L, seed):
    """Lengths (one full, one short, one empty where batch > 2) and document
    starts (at token 0 of the first sequence, mid-chunk, on a chunk boundary,
    two in a row, one past a length, which is ignored)."""
    lens = np.array([L, L - 37, 0][:batch], dtype=np.int32)
    reset = np.zeros((batch, L), dtype=np.uint8)
    reset[0, [0, 21, 48, 49]] = 1
    if batch > 1:
        reset[1, [5, 32, L - 10]] = 1
    return lens, reset


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["zoh", "euler"])
@pytest.mark.parametrize("from_ckpt", [False, True])
def test_bwd_lengths_and_resets(io, mode, from_ckpt):
    """ssm_scan_bwd_ex with lengths and document starts, h0 and dlast, with
    its own forward sweep or from the training forward's checkpoints (taken
    with the same lengths and starts), against the oracle's backward."""
    inp = W.scan_inputs(_cfg(3, 99, 34, 16, io, True, seed=130))
    dy = _dy((3, 99, 34), io, 131)
    rng = np.random.default_rng(132)
    h0 = rng.normal(size=(3, 34, 16)).astype(np.float32)
    dlast = rng.normal(size=(3, 34, 16)).astype(np.float32)
    lens, reset = _varlen(3, 99, 133)
    args = (to_dev(inp["u"], io), to_dev(inp["delta"], io), to_dev(inp["A"], "f32"),
            to_dev(inp["B"], io), to_dev(inp["C"], io))
    kw = dict(D=to_dev(inp["D"], "f32"), z=to_dev(inp["z"], io),
              delta_bias=to_dev(inp["delta_bias"], "f32"), dt_mode=mode, h0=to_dev(h0, "f32"),
              seq_lens=torch.from_numpy(lens).to(DEV), reset=torch.from_numpy(reset).to(DEV))
    ck = ssm.scan_fwd_train(*args, **kw)[2] if from_ckpt else None
    g = ssm.scan_bwd(*args, to_dev(dy, io), dlast=to_dev(dlast, "f32"), ckpt=ck, **kw)
    torch.cuda.synchronize()
    r = oracle.scan_bwd(f64(inp["u"], io), f64(inp["delta"], io), inp["A"], f64(inp["B"], io),
                        f64(inp["C"], io), f64(dy, io), D=inp["D"], z=f64(inp["z"], io),
                        delta_bias=inp["delta_bias"], dt_mode=mode, h0=h0.astype(np.float64),
                        dlast=dlast.astype(np.float64), seq_lens=lens, reset=reset)
    _compare(g, r, io, f"varlen {io} {mode} ckpt={from_ckpt}")
    for b, n in enumerate(lens):  # padding rows are exactly zero
        for k in ("du", "ddelta", "dz", "dB", "dC"):
            assert torch.all(g[k][b, n:] == 0), f"{k} past length {n}"


@pytest.mark.parametrize("kernel", ["seq1", "seq2", "seq4", "tpar", "wave", "wave4"])
def test_bwd_lengths_and_resets_from_every_forward(kernel):
    """The checkpoints of every forward kernel, taken with lengths and
    document starts, give the backward the oracle's gradients."""
    inp = W.scan_inputs(_cfg(2, 80, 20, 16, "f32", True, seed=134))
    dy = _dy((2, 80, 20), "f32", 135)
    lens, reset = _varlen(2, 80, 136)
    args = (to_dev(inp["u"], "f32"), to_dev(inp["delta"], "f32"), to_dev(inp["A"], "f32"),
            to_dev(inp["B"], "f32"), to_dev(inp["C"], "f32"))
    kw = dict(D=to_dev(inp["D"], "f32"), z=to_dev(inp["z"], "f32"),
              delta_bias=to_dev(inp["delta_bias"], "f32"),
              seq_lens=torch.from_numpy(lens).to(DEV), reset=torch.from_numpy(reset).to(DEV))
    _, _, ck = ssm.scan_fwd_train(*args, kernel=kernel, **kw)
    g = ssm.scan_bwd(*args, to_dev(dy, "f32"), ckpt=ck, **kw)
    torch.cuda.synchronize()
    r = oracle.scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], dy, D=inp["D"],
                        z=inp["z"], delta_bias=inp["delta_bias"], seq_lens=lens, reset=reset)
    _compare(g, r, "f32", f"varlen from {kernel}")


def test_bwd_lengths_all_padding_and_state_sizes():
    """Every sequence empty (only dlast reaches dh0), and state sizes below 16
    with lengths and starts."""
    inp = W.scan_inputs(_cfg(2, 40, 12, 16, "f32", True, seed=137))
    dy = _dy((2, 40, 12), "f32", 138)
    dlast = np.random.default_rng(139).normal(size=(2, 12, 16)).astype(np.float32)
    h0 = np.zeros((2, 12, 16), dtype=np.float32)
    lens = np.zeros(2, dtype=np.int32)
    g = ssm.scan_bwd(to_dev(inp["u"], "f32"), to_dev(inp["delta"], "f32"), to_dev(inp["A"], "f32"),
                     to_dev(inp["B"], "f32"), to_dev(inp["C"], "f32"), to_dev(dy, "f32"),
                     D=to_dev(inp["D"], "f32"), z=to_dev(inp["z"], "f32"), h0=to_dev(h0, "f32"),
                     dlast=to_dev(dlast, "f32"), seq_lens=torch.from_numpy(lens).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(g["dh0"], to_dev(dlast, "f32"))
    for k in ("du", "ddelta", "dz", "dB", "dC", "dA", "dD"):
        assert torch.all(g[k] == 0), k
    for N in (3, 8):
        inp = W.scan_inputs(_cfg(2, 60, 20, N, "f32", True, seed=140 + N))
        dy = _dy((2, 60, 20), "f32", 141)
        lens, reset = _varlen(2, 60, 142)
        g = ssm.scan_bwd(to_dev(inp["u"], "f32"), to_dev(inp["delta"], "f32"),
                         to_dev(inp["A"], "f32"), to_dev(inp["B"], "f32"), to_dev(inp["C"], "f32"),
                         to_dev(dy, "f32"), D=to_dev(inp["D"], "f32"), z=to_dev(inp["z"], "f32"),
                         seq_lens=torch.from_numpy(lens).to(DEV),
                         reset=torch.from_numpy(reset).to(DEV))
        torch.cuda.synchronize()
        r = oracle.scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], dy, D=inp["D"],
                            z=inp["z"], seq_lens=lens, reset=reset)
        _compare(g, r, "f32", f"varlen N={N}")
