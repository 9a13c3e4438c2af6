"""Pins for the oracle's backward pass of the causal depthwise convolution
("The Mamba block" on the first page: x_t = SiLU(sum_i w_i xt_{t-i} + b), with
the prefill extras of the scan -- a carried-in window, lengths, document
starts -- and the window it hands to decoding).  Two independent routes:
central finite differences of the oracle's own (already pinned) forward, and,
without the activation, the closed form of a linear filter's gradient from
numpy.correlate and plain sums."""
import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(5151)


def _problem(batch=2, L=11, dim=3, k=4):
    return dict(x=RNG.normal(size=(batch, L, dim)), weight=RNG.uniform(-0.8, 0.8, size=(dim, k)),
                bias=RNG.normal(size=dim) * 0.3)


def _loss(p, dout, dwin, **kw):
    out, win = oracle.conv1d_fwd(**p, **kw)
    s = float(np.sum(dout * out))
    if dwin is not None:
        s += float(np.sum(dwin * win))
    return s


def _fd(p, name, dout, dwin, eps=1e-6, **kw):
    base = p[name]
    g = np.zeros_like(base)
    for idx in np.ndindex(base.shape):
        q = dict(p)
        plus, minus = base.copy(), base.copy()
        plus[idx] += eps
        minus[idx] -= eps
        q[name] = plus
        lp = _loss(q, dout, dwin, **kw)
        q[name] = minus
        lm = _loss(q, dout, dwin, **kw)
        g[idx] = (lp - lm) / (2 * eps)
    return g


# (k, silu, lengths, document starts per sequence, carried-in window, window gradient)
CASES = [
    (4, True, None, None, False, False),
    (4, True, [11, 6], [[4], [0, 3]], True, True),
    (3, False, [2, 11], [[1], [7, 8]], True, True),   # a length shorter than the window
    (2, True, [11, 0], [[10], []], False, True),      # an empty sequence
    (1, True, [9, 11], [[2], [5]], True, True),       # no window at all
    (4, True, [11, 11], [[0], [2]], True, False),     # a start at token 0 drops the window
]


@pytest.mark.parametrize("k,silu,lens,starts,use_win,use_dwin", CASES)
def test_gradients_match_finite_differences(k, silu, lens, starts, use_win, use_dwin):
    p = _problem(k=k)
    batch, L, dim = p["x"].shape
    kw = dict(silu=silu)
    if lens is not None:
        kw["seq_lens"] = np.array(lens)
    if starts is not None:
        reset = np.zeros((batch, L), dtype=np.uint8)
        for b, ts in enumerate(starts):
            reset[b, ts] = 1
        kw["reset"] = reset
    if use_win:
        p["state_in"] = RNG.normal(size=(batch, k - 1, dim))
    dout = RNG.normal(size=(batch, L, dim))
    dwin = RNG.normal(size=(batch, k - 1, dim)) if use_dwin else None
    g = oracle.conv1d_bwd(p["x"], p["weight"], dout, bias=p["bias"], silu=silu,
                          state_in=p.get("state_in"), seq_lens=kw.get("seq_lens"),
                          reset=kw.get("reset"), dstate_out=dwin)
    names = [("x", "dx"), ("weight", "dweight"), ("bias", "dbias")]
    if use_win:
        names.append(("state_in", "dstate_in"))
    for inp, out in names:
        fd = _fd(p, inp, dout, dwin, **kw)
        assert g[out].shape == fd.shape
        if fd.size == 0:  # k = 1: no window
            continue
        err = np.abs(g[out] - fd).max() / (1.0 + np.abs(fd).max())
        assert err < 1e-7, f"{out}: {err:.2e}"
    if lens is not None:
        for b, n in enumerate(lens):  # inputs past a length feed nothing
            assert np.all(g["dx"][b, n:] == 0.0)


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_linear_filter_closed_form(k):
    """Without the activation, lengths or starts the layer is a linear causal
    filter: dx is dout correlated with the taps, dw_i the lag-i cross sum of
    dout and x, dbias the sum of dout."""
    p = _problem(k=k, L=17)
    batch, L, dim = p["x"].shape
    dout = RNG.normal(size=(batch, L, dim))
    g = oracle.conv1d_bwd(p["x"], p["weight"], dout, bias=p["bias"], silu=False)
    for b in range(batch):
        for c in range(dim):
            w = p["weight"][c]
            # dx_s = sum_i w_i dout_{s+i}: the valid part of correlating dout with w
            full = np.correlate(np.concatenate([dout[b, :, c], np.zeros(k - 1)]), w, mode="valid")
            np.testing.assert_allclose(g["dx"][b, :, c], full, rtol=1e-12, atol=1e-12)
    for c in range(dim):
        for i in range(k):
            expect = sum(float(np.dot(dout[b, i:, c], p["x"][b, :L - i, c])) for b in range(batch))
            assert g["dweight"][c, i] == pytest.approx(expect, rel=1e-12, abs=1e-12)
        assert g["dbias"][c] == pytest.approx(dout[:, :, c].sum(), rel=1e-12, abs=1e-12)
