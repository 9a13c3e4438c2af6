"""GPU parity of ssm_conv1d_fwd / ssm_conv1d_step against the fp64 oracle.

Outputs: fp32 io within 1e-4 (1 + |ref|) elementwise, bf16 io within 1e-2
relative RMS (the scan's tolerances).  The decoding window is a copy of
inputs, so it must match bit for bit.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import DEV, assert_close, f64, to_dev, to_host64
import oracle
import selective_state_space_66_amd as ssm

pytestmark = pytest.mark.gpu


def _inputs(batch, L, dim, k, io, seed):
    return W.conv_inputs(W.ConvConfig(f"c{batch}x{L}x{dim}x{k}", batch, L, dim, k, io, seed))


def _window(batch, k, dim, io, seed):
    cfg = W.ConvConfig("w", batch, 0, dim, k, io, seed)
    return W.conv_window0(cfg)


def _gpu(inp, silu=True, window_in=None, seq_lens=None, reset=None):
    io = inp["io"]
    out, win = ssm.conv1d_fwd(to_dev(inp["x"], io), to_dev(inp["w"], "f32"),
                              bias=to_dev(inp["bias"], "f32"), silu=silu,
                              window_in=None if window_in is None else to_dev(window_in, io),
                              seq_lens=seq_lens, reset=reset)
    torch.cuda.synchronize()
    return out, win


def _ref(inp, silu=True, window_in=None, seq_lens=None, reset=None):
    io = inp["io"]
    return oracle.conv1d_fwd(f64(inp["x"], io), inp["w"], inp["bias"], silu=silu,
                             state_in=None if window_in is None else f64(window_in, io),
                             seq_lens=seq_lens, reset=reset)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("k", [1, 2, 3, 4])
@pytest.mark.parametrize("dim", [64, 70])  # 4-channel vectors, and the scalar path
@pytest.mark.parametrize("silu", [True, False])
def test_conv_fwd(io, k, dim, silu):
    inp = _inputs(3, 150, dim, k, io, seed=40 + k)
    win0 = _window(3, k, dim, io, seed=50 + k)
    out, win = _gpu(inp, silu=silu, window_in=win0)
    ro, rw = _ref(inp, silu=silu, window_in=win0)
    assert_close(to_host64(out), ro, io, "out")
    np.testing.assert_array_equal(to_host64(win), rw)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("dim", [64, 70])
def test_conv_lengths_and_resets(io, dim):
    """Lengths at 0, 1, 2, inside and at the edges of the 16-token runs and the
    64-token blocks; resets in the halo, at run starts and at t = 0; NaN in
    every padded input."""
    lens = [0, 1, 2, 15, 16, 17, 64, 65, 130, 130]
    L = 130
    inp = _inputs(len(lens), L, dim, 4, io, seed=60)
    x = inp["x"].copy()
    nan = np.uint16(0x7FC0) if io == "bf16" else np.float32(np.nan)
    for b, l in enumerate(lens):
        x[b, l:] = nan
    inp["x"] = x
    reset = np.zeros((len(lens), L), dtype=np.uint8)
    reset[4, [3, 14, 15]] = 1
    reset[5, [0, 16]] = 1
    reset[7, [62, 63, 64]] = 1
    reset[8, [17, 33, 127]] = 1
    reset[9, 129] = 1
    win0 = _window(len(lens), 4, dim, io, seed=61)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out, win = _gpu(inp, window_in=win0, seq_lens=sl, reset=torch.from_numpy(reset).to(DEV))
    ro, rw = _ref(inp, window_in=win0, seq_lens=lens, reset=reset)
    og = to_host64(out)
    for b, l in enumerate(lens):
        assert np.all(og[b, l:] == 0.0)
    assert_close(og, ro, io, "out")
    np.testing.assert_array_equal(to_host64(win), rw)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("k", [1, 2, 4])
def test_conv_steps_match_oracle(io, k):
    cfg = W.ConvConfig("s", 5, 0, 68, k, io, 70 + k)
    w, bias = W.conv_params(cfg.seed, cfg.dim, k)
    win = W.conv_window0(cfg)
    wd = to_dev(win, io) if k > 1 else torch.empty((5, 0, 68), device=DEV,
                                                    dtype=torch.float32 if io == "f32" else torch.bfloat16)
    rwin = f64(win, io)
    for s in range(12):
        x = W.conv_step_inputs(cfg, s)
        out = ssm.conv1d_step(wd, to_dev(x, io), to_dev(w, "f32"), bias=to_dev(bias, "f32"))
        torch.cuda.synchronize()
        ro, rwin = oracle.conv1d_step(rwin, f64(x, io), w, bias)
        assert_close(to_host64(out), ro, io, f"out step {s}")
        np.testing.assert_array_equal(to_host64(wd), rwin)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_prefill_then_decode(io):
    """The window a prefill returns continues, step by step, exactly where the
    whole-sequence convolution goes."""
    inp = _inputs(2, 60, 64, 4, io, seed=80)
    full, _ = _gpu(inp)
    head = dict(inp)
    head["x"] = np.ascontiguousarray(inp["x"][:, :41])
    _, win = _gpu(head)
    w, b = to_dev(inp["w"], "f32"), to_dev(inp["bias"], "f32")
    for t in range(41, 60):
        o = ssm.conv1d_step(win, to_dev(np.ascontiguousarray(inp["x"][:, t]), io), w, bias=b)
        torch.cuda.synchronize()
        assert torch.equal(o, full[:, t]), f"step {t}"


def test_empty_and_degenerate():
    w = torch.zeros((8, 4), device=DEV)
    x = torch.zeros((2, 0, 8), device=DEV)
    win_in = torch.randn((2, 3, 8), device=DEV)
    out, win = ssm.conv1d_fwd(x, w, window_in=win_in)
    torch.cuda.synchronize()
    assert out.shape == (2, 0, 8) and torch.equal(win, win_in)  # no tokens: the window carries over
    out0, _ = ssm.conv1d_fwd(torch.zeros((0, 5, 8), device=DEV), w)
    assert out0.shape == (0, 5, 8)


def test_conv_full_size_sampled():
    """The convolution in front of the Mamba-130M layer at full size; the oracle
    checks sampled channels."""
    cfg = W.CONV_CONFIGS["conv130m"]
    inp = W.conv_inputs(cfg)
    out, win = _gpu(inp)
    ch = np.array([0, 1, 2, 3, 255, 256, 700, 1531, 1535])
    sub = W.conv_inputs(cfg, channels=ch)
    ro, rw = _ref(sub)
    chd = torch.from_numpy(ch).to(DEV)
    assert_close(to_host64(out.index_select(2, chd)), ro, "bf16", "out")
    np.testing.assert_array_equal(to_host64(win.index_select(2, chd)), rw)


# ------------------------------------------------------------- backward pass

def _dout(shape, io, seed):
    x = np.random.default_rng(seed).normal(size=shape).astype(np.float32)
    return W.to_bf16_bits(x) if io == "bf16" else x


def _bwd_compare(g, r, io, what):
    """dx, dwindow_in: fp32 within 1e-4 (1 + |ref|) elementwise (a sum of at
    most k products); dweight, dbias (sums over every token of every sequence)
    within 2e-5 (1 + max |ref|) of the tensor's scale; bf16 io: relative RMS
    1e-2 for everything (inputs and dout are the same bf16 bits on both sides,
    dx is rounded to bf16 once)."""
    for k, ref in r.items():
        if ref is None:
            assert g[k] is None, k
            continue
        got = to_host64(g[k])
        assert got.shape == ref.shape, k
        assert np.all(np.isfinite(got)), f"{what} {k}"
        if io == "bf16":
            assert_close(got, ref, "bf16", f"{what} {k}")
        elif k in ("dweight", "dbias"):
            err = np.abs(got - ref).max() / (1.0 + np.abs(ref).max())
            assert err <= 2e-5, f"{what} {k}: {err:.2e}"
        else:
            assert_close(got, ref, "f32", f"{what} {k}")


def _bwd_run(inp, dout, silu=True, window_in=None, seq_lens=None, reset=None, dwo=None):
    io = inp["io"]
    g = ssm.conv1d_bwd(to_dev(inp["x"], io), to_dev(inp["w"], "f32"), to_dev(dout, io),
                       bias=to_dev(inp["bias"], "f32"), silu=silu,
                       window_in=None if window_in is None else to_dev(window_in, io),
                       seq_lens=None if seq_lens is None else torch.from_numpy(seq_lens).to(DEV),
                       reset=None if reset is None else torch.from_numpy(reset).to(DEV),
                       dwindow_out=None if dwo is None else to_dev(dwo, io))
    torch.cuda.synchronize()
    r = oracle.conv1d_bwd(f64(inp["x"], io), inp["w"], f64(dout, io), bias=inp["bias"], silu=silu,
                          state_in=None if window_in is None else f64(window_in, io),
                          seq_lens=seq_lens, reset=reset,
                          dstate_out=None if dwo is None else f64(dwo, io))
    r = dict(dx=r["dx"], dweight=r["dweight"], dbias=r["dbias"], dwindow_in=r["dstate_in"])
    return g, r


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("k", [1, 2, 3, 4])
@pytest.mark.parametrize("dim", [64, 70])
@pytest.mark.parametrize("silu", [True, False])
def test_conv_bwd(io, k, dim, silu):
    """Three sequences of 300 tokens (three 128-token spans, the last ragged),
    a carried-in window and the gradient of the window handed on."""
    inp = _inputs(3, 300, dim, k, io, seed=60 + k)
    win0 = _window(3, k, dim, io, seed=61 + k)
    dout = _dout((3, 300, dim), io, 62 + k)
    dwo = _dout((3, k - 1, dim), io, 63 + k)
    g, r = _bwd_run(inp, dout, silu=silu, window_in=win0, dwo=dwo)
    _bwd_compare(g, r, io, f"bwd k={k} dim={dim} silu={silu}")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("k", [2, 4])
@pytest.mark.parametrize("dim", [64, 70])
def test_conv_bwd_lengths_and_resets(io, k, dim):
    """Lengths (full, one inside a span, one shorter than the window, empty)
    and document starts (at token 0, mid-run, on a run edge, two in a row,
    one past a length), with and without a carried-in window."""
    batch, L = 4, 300
    inp = _inputs(batch, L, dim, k, io, seed=70 + k)
    dout = _dout((batch, L, dim), io, 71)
    dwo = _dout((batch, k - 1, dim), io, 72)
    lens = np.array([300, 133, 2, 0], dtype=np.int32)
    reset = np.zeros((batch, L), dtype=np.uint8)
    reset[0, [0, 5, 8, 9, 128, 250]] = 1
    reset[1, [7, 64, 200]] = 1
    reset[2, [1]] = 1
    for win0 in (None, _window(batch, k, dim, io, seed=73)):
        g, r = _bwd_run(inp, dout, window_in=win0, seq_lens=lens, reset=reset, dwo=dwo)
        _bwd_compare(g, r, io, f"varlen k={k} dim={dim} window={win0 is not None}")
        dx = to_host64(g["dx"])
        for b, n in enumerate(lens):
            assert np.all(dx[b, n:] == 0.0)


def test_conv_bwd_no_tokens_and_deterministic():
    """No tokens: the window's gradient passes through, dw and dbias are zero;
    two calls give the same bits."""
    k, dim = 4, 64
    x = torch.zeros((2, 0, dim), dtype=torch.float32, device=DEV)
    w = torch.randn((dim, k), device=DEV)
    win0 = torch.randn((2, k - 1, dim), device=DEV)
    dwo = torch.randn((2, k - 1, dim), device=DEV)
    g = ssm.conv1d_bwd(x, w, x, bias=torch.zeros(dim, device=DEV), window_in=win0,
                       dwindow_out=dwo)
    torch.cuda.synchronize()
    assert torch.equal(g["dwindow_in"], dwo)
    assert torch.all(g["dweight"] == 0) and torch.all(g["dbias"] == 0)
    inp = _inputs(2, 500, 96, 4, "bf16", seed=74)
    dout = _dout((2, 500, 96), "bf16", 75)
    args = (to_dev(inp["x"], "bf16"), to_dev(inp["w"], "f32"), to_dev(dout, "bf16"))
    g1 = ssm.conv1d_bwd(*args, bias=to_dev(inp["bias"], "f32"))
    g2 = ssm.conv1d_bwd(*args, bias=to_dev(inp["bias"], "f32"))
    torch.cuda.synchronize()
    for key in ("dx", "dweight", "dbias"):
        assert torch.equal(g1[key], g2[key]), key


def test_conv_bwd_full_size_sampled():
    """The Mamba-130M layer's convolution (batch 8, L 2048, D 1536, k 4, bf16)
    at full size: channels are independent, so the oracle on sampled channels
    is the exact reference for their dx, dweight and dbias."""
    cfg = W.CONV_CONFIGS["conv130m"]
    inp = W.conv_inputs(cfg)
    dout = _dout((cfg.batch, cfg.L, cfg.dim), "bf16", 76)
    g = ssm.conv1d_bwd(to_dev(inp["x"], "bf16"), to_dev(inp["w"], "f32"), to_dev(dout, "bf16"),
                       bias=to_dev(inp["bias"], "f32"))
    torch.cuda.synchronize()
    ch = np.array([0, 1, 5, 700, 1535])
    sub = W.conv_inputs(cfg, channels=ch)
    r = oracle.conv1d_bwd(f64(sub["x"], "bf16"), sub["w"], f64(dout[:, :, ch], "bf16"),
                          bias=sub["bias"])
    chd = torch.from_numpy(ch).to(DEV)
    got = dict(dx=g["dx"].index_select(2, chd), dweight=g["dweight"].index_select(0, chd),
               dbias=g["dbias"].index_select(0, chd), dwindow_in=None)
    _bwd_compare(got, dict(dx=r["dx"], dweight=r["dweight"], dbias=r["dbias"], dwindow_in=None),
                 "bf16", "full size")
