"""GPU parity of the time-parallel scan with eight tokens per lane
(scan_wave8.hip) against the oracle.

The library runs it for the 16-lane layout (the "wave4" kernel id, forced
here; the library's own choice for layers of 12288 rows or more) whenever the
call has bf16 io, N = 16, no lengths or document starts, a width that is a
multiple of 16 and 16-byte aligned rows; the cases below meet those
conditions.  They cover ragged last chunks (L not a multiple of its 128
tokens), sequences shorter than one chunk, h0, both rules, the gate on and
off, ZOH states in both of its forms (|A| >= 1/2 and below, in one wave), the
optional inputs absent, and the training forward's checkpoints.

Bounds: the final state is fp32, computed in fp32 from the same bf16 inputs as
the oracle's: max |s - s_ref| <= 1e-4 (1 + |s_ref|), the fp32 acceptance
bound.  y is rounded to bf16 once: relative RMS <= 1e-2 (the bf16 acceptance
bound), and elementwise |y - y_ref| <= 1e-2 (1 + |y_ref|), so that no single
token or channel can hide in the RMS.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import DEV, assert_close, f64, max_scaled_err, to_dev, to_host64
import oracle
import selective_state_space_66_amd as ssm
from test_gpu_scan_bwd import _compare, _dy

pytestmark = pytest.mark.gpu


def _cfg(batch, L, dim, gate, seed):
    return W.ScanConfig(f"w8_{batch}x{L}x{dim}", batch, L, dim, 16, "bf16", gate, seed)


def _run(inp, mode, h0=None, softplus=True, use_D=True, use_bias=True):
    y, last = ssm.scan_fwd(to_dev(inp["u"], "bf16"), to_dev(inp["delta"], "bf16"), to_dev(inp["A"], "f32"),
                           to_dev(inp["B"], "bf16"), to_dev(inp["C"], "bf16"),
                           D=to_dev(inp["D"], "f32") if use_D else None,
                           z=to_dev(inp["z"], "bf16") if inp["z"] is not None else None,
                           delta_bias=to_dev(inp["delta_bias"], "f32") if use_bias else None,
                           softplus=softplus, dt_mode=mode, kernel="wave4",
                           h0=None if h0 is None else to_dev(h0, "f32"))
    torch.cuda.synchronize()
    yr, lr = oracle.scan_fwd(f64(inp["u"], "bf16"), f64(inp["delta"], "bf16"), inp["A"], f64(inp["B"], "bf16"),
                             f64(inp["C"], "bf16"), D=inp["D"] if use_D else None,
                             z=f64(inp["z"], "bf16") if inp["z"] is not None else None,
                             delta_bias=inp["delta_bias"] if use_bias else None, softplus=softplus,
                             dt_mode=mode, h0=None if h0 is None else h0.astype(np.float64))
    yg, lg = to_host64(y), to_host64(last)
    assert_close(yg, yr, "bf16", "y")
    ey = max_scaled_err(yg, yr)
    assert ey <= 1e-2, f"y: max scaled error {ey:.3e}"
    el = max_scaled_err(lg, lr)
    assert el <= 1e-4, f"last_state: max scaled error {el:.3e}"
    return y, last


@pytest.mark.parametrize("L", [1, 100, 128, 129, 300])
@pytest.mark.parametrize("mode", ["zoh", "euler"])
@pytest.mark.parametrize("gate", [True, False])
def test_wave8_lengths_rules_gate(L, mode, gate):
    """3 channel tiles; one chunk or less, exactly one, one and a token, and
    three with a ragged tail."""
    inp = W.scan_inputs(_cfg(2, L, 48, gate, seed=400 + L))
    _run(inp, mode)


@pytest.mark.parametrize("mode", ["zoh", "euler"])
def test_wave8_initial_state(mode):
    inp = W.scan_inputs(_cfg(2, 200, 32, True, seed=410))
    h0 = np.random.default_rng(411).normal(size=(2, 32, 16)).astype(np.float32)
    _run(inp, mode, h0=h0)


def test_wave8_zoh_both_forms():
    """A state with |A| < 1/2 in channel 5, a channel of small A (20) and a zero
    A (channel 33, state 0): their waves take phi(Delta A), the others the g
    form."""
    inp = W.scan_inputs(_cfg(2, 260, 48, True, seed=420))
    A = inp["A"].copy()
    A[5, 3] = -0.3
    A[20, :] = -0.01
    A[33, 0] = 0.0
    inp["A"] = A
    h0 = np.random.default_rng(421).normal(size=(2, 48, 16)).astype(np.float32)
    _run(inp, "zoh", h0=h0)


@pytest.mark.parametrize("mode", ["zoh", "euler"])
def test_wave8_optional_inputs_absent(mode):
    """No D, no delta bias, softplus off (small positive steps)."""
    inp = W.scan_inputs(_cfg(1, 150, 16, False, seed=430))
    inp["delta"] = W.to_bf16_bits((np.abs(f64(inp["delta"], "bf16")) * 0.05).astype(np.float32))
    _run(inp, mode, softplus=False, use_D=False, use_bias=False)


def test_wave8_matches_the_four_token_kernel():
    """The same inputs through the four-tokens-per-lane kernel (taken when the
    width is not a multiple of 16: one more channel, sliced off) give the same
    y to bf16 rounding and the same final state to fp32 rounding."""
    inp = W.scan_inputs(_cfg(2, 300, 49, True, seed=440))
    full = [to_dev(inp[k], "bf16") for k in ("u", "delta")]
    A, B, C = to_dev(inp["A"], "f32"), to_dev(inp["B"], "bf16"), to_dev(inp["C"], "bf16")
    D, z, bias = to_dev(inp["D"], "f32"), to_dev(inp["z"], "bf16"), to_dev(inp["delta_bias"], "f32")
    y4, l4 = ssm.scan_fwd(full[0], full[1], A, B, C, D=D, z=z, delta_bias=bias, kernel="wave4")
    y8, l8 = ssm.scan_fwd(full[0][..., :48].contiguous(), full[1][..., :48].contiguous(), A[:48].contiguous(), B, C,
                          D=D[:48].contiguous(), z=z[..., :48].contiguous(), delta_bias=bias[:48].contiguous(),
                          kernel="wave4")
    torch.cuda.synchronize()
    dy = (y8.float() - y4[..., :48].float()).abs()
    assert float(dy.max()) <= 2.0 ** -7 * float(y4[..., :48].float().abs().max()), float(dy.max())
    assert torch.allclose(l8, l4[:, :48], rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("mode", ["zoh", "euler"])
@pytest.mark.parametrize("gate", [True, False])
def test_wave8_training_forward_checkpoints(mode, gate):
    """The training forward through this kernel: y and the final state equal
    the plain forward's bit for bit, and checkpoint j is the state before
    token 16 j (the oracle's final state of the sequence cut there; j = 0:
    h0), over a ragged last chunk (L 300: 19 checkpoints) with states in both
    ZOH forms.  Under ZOH the backward from those checkpoints matches the
    oracle's backward."""
    L, dim = 300, 48
    inp = W.scan_inputs(_cfg(2, L, dim, gate, seed=450 + gate))
    A = inp["A"].copy()
    A[5, 3] = -0.3
    A[20, :] = -0.01
    inp["A"] = A
    h0 = np.random.default_rng(451).normal(size=(2, dim, 16)).astype(np.float32)
    args = (to_dev(inp["u"], "bf16"), to_dev(inp["delta"], "bf16"), to_dev(inp["A"], "f32"),
            to_dev(inp["B"], "bf16"), to_dev(inp["C"], "bf16"))
    kw = dict(D=to_dev(inp["D"], "f32"), z=to_dev(inp["z"], "bf16") if gate else None,
              delta_bias=to_dev(inp["delta_bias"], "f32"), dt_mode=mode, h0=to_dev(h0, "f32"))
    y, last, ck = ssm.scan_fwd_train(*args, kernel="wave4", **kw)
    y2, last2 = ssm.scan_fwd(*args, kernel="wave4", **kw)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(last, last2)
    ckh = to_host64(ck)
    nck = (L + 15) // 16
    assert ckh.shape == (2, nck, dim, 16)
    u, dl, B, C = (f64(inp[k], "bf16") for k in ("u", "delta", "B", "C"))
    z = f64(inp["z"], "bf16") if gate else None
    for j in range(nck):
        t = 16 * j
        _, lr = oracle.scan_fwd(u[:, :t], dl[:, :t], inp["A"], B[:, :t], C[:, :t], D=inp["D"],
                                z=None if z is None else z[:, :t], delta_bias=inp["delta_bias"], dt_mode=mode,
                                h0=h0.astype(np.float64))
        err = max_scaled_err(ckh[:, j], lr)
        assert err <= 1e-4, f"checkpoint {j}: {err:.2e}"
    if mode == "zoh":
        dy = _dy((2, L, dim), "bf16", 452)
        g = ssm.scan_bwd(*args, to_dev(dy, "bf16"), ckpt=ck, **kw)
        torch.cuda.synchronize()
        r = oracle.scan_bwd(u, dl, inp["A"], B, C, f64(dy, "bf16"), D=inp["D"], z=z,
                            delta_bias=inp["delta_bias"], dt_mode=mode, h0=h0.astype(np.float64))
        _compare(g, r, "bf16", f"wave8 checkpoints gate={gate}")
