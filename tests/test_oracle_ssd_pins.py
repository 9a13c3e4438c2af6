"""Pins for the oracle's Mamba-2 / SSD layer (one scalar decay per head).

1. The SSD layer is the S6 layer whose A and step size are the same for every
   state and channel of a head; the already pinned scan oracle, given A and
   Delta repeated that way, must give the same outputs and final state.
2. The structured masked-matmul form the pages give for it ("The Mamba CUDA
   kernel" on the fourth page; the mixing matrix of "Selection breaks the
   convolution" on the first): Y = (M * (C B^T)) (w x) with
   M[t, s] = exp(A (cum_t - cum_s)) for t >= s, cum the running sum of Delta,
   evaluated with numpy matmuls -- a quadratic algorithm with no recurrence.
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle

RNG = np.random.default_rng(2024)


def _problem(batch=2, L=23, nheads=3, P=4, N=5, gate=True):
    return dict(
        x=RNG.normal(size=(batch, L, nheads, P)),
        dt=RNG.normal(size=(batch, L, nheads)),
        A=-RNG.uniform(0.3, 2.0, size=nheads),
        B=RNG.normal(size=(batch, L, N)),
        C=RNG.normal(size=(batch, L, N)),
        D=RNG.normal(size=nheads),
        z=RNG.normal(size=(batch, L, nheads, P)) if gate else None,
        dt_bias=RNG.normal(size=nheads) * 0.3,
    )


@pytest.mark.parametrize("mode", ["zoh", "euler"])
@pytest.mark.parametrize("gate", [True, False])
@pytest.mark.parametrize("softplus", [True, False])
def test_ssd_equals_scan_with_shared_decay(mode, gate, softplus):
    p = _problem(gate=gate)
    if not softplus:
        p["dt"] = np.abs(p["dt"]) + 0.01
        p["dt_bias"] = np.abs(p["dt_bias"])
    batch, L, H, P = p["x"].shape
    N = p["B"].shape[2]
    h0 = RNG.normal(size=(batch, H, P, N))
    y, last = oracle.ssd_fwd(**p, softplus=softplus, dt_mode=mode, h0=h0)
    dim = H * P
    ys, ls = oracle.scan_fwd(
        p["x"].reshape(batch, L, dim), np.repeat(p["dt"], P, axis=2),
        np.repeat(p["A"], P)[:, None].repeat(N, axis=1), p["B"], p["C"],
        D=np.repeat(p["D"], P), z=None if p["z"] is None else p["z"].reshape(batch, L, dim),
        delta_bias=np.repeat(p["dt_bias"], P), softplus=softplus, dt_mode=mode,
        h0=h0.reshape(batch, dim, N))
    np.testing.assert_allclose(y.reshape(batch, L, dim), ys, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(last.reshape(batch, dim, N), ls, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("mode", ["zoh", "euler"])
def test_ssd_equals_masked_matmul(mode):
    p = _problem(L=31, N=6)
    batch, L, H, P = p["x"].shape
    h0 = RNG.normal(size=(batch, H, P, 6))
    y, last = oracle.ssd_fwd(**p, dt_mode=mode, h0=h0)
    v = p["dt"] + p["dt_bias"]
    delta = np.logaddexp(0.0, v)  # softplus
    for b in range(batch):
        CB = p["C"][b] @ p["B"][b].T  # (L, L): C_t . B_s
        for h in range(H):
            a = p["A"][h]
            d = delta[b, :, h]
            cum = np.cumsum(d)
            w = d * (np.expm1(d * a) / (d * a)) if mode == "zoh" else d
            M = np.tril(np.exp(a * (cum[:, None] - cum[None, :])))
            xw = w[:, None] * p["x"][b, :, h, :]  # (L, P)
            ys = (M * CB) @ xw                    # the masked matmul
            ys += (p["C"][b] * np.exp(a * cum)[:, None]) @ h0[b, h].T  # from the initial state
            ys += p["D"][h] * p["x"][b, :, h, :]
            zz = p["z"][b, :, h, :]
            ys *= zz * expit(zz)
            np.testing.assert_allclose(y[b, :, h, :], ys, rtol=1e-11, atol=1e-11)
            lf = (np.exp(a * (cum[-1] - cum))[:, None] * p["B"][b]).T @ xw  # (N, P)
            lf += np.exp(a * cum[-1]) * h0[b, h].T
            np.testing.assert_allclose(last[b, h], lf.T, rtol=1e-11, atol=1e-11)
