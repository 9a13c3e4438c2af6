"""Pins for the oracle's backward pass: central finite differences of the
oracle's own (already pinned) forward pass.  The loss is a random linear
functional of the outputs, sum(dy * y) + sum(dlast * last_state), so its
gradient with respect to every input is exactly what scan_bwd returns.  The
finite differences know nothing of the reverse recurrence, the chain rule
through Delta A or the derivative of softplus."""
import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(777)


def _problem(batch=2, L=7, dim=3, N=4, gate=True, small_a=False):
    A = -RNG.uniform(0.5, 2.0, size=(dim, N))
    if small_a:
        A[0, 0] = 0.0      # the limit bbar = Delta B
        A[1, :] = -0.03    # |Delta A| < 0.1: phi' from its series
    return dict(
        u=RNG.normal(size=(batch, L, dim)),
        delta=RNG.normal(size=(batch, L, dim)) * 0.5,
        A=A,
        B=RNG.normal(size=(batch, L, N)),
        C=RNG.normal(size=(batch, L, N)),
        D=RNG.normal(size=dim),
        z=RNG.normal(size=(batch, L, dim)) if gate else None,
        delta_bias=RNG.normal(size=dim) * 0.3,
    )


def _loss(p, dy, dlast, **kw):
    y, last = oracle.scan_fwd(**p, **kw)
    return float(np.sum(dy * y) + np.sum(dlast * last))


def _fd(p, name, dy, dlast, eps=1e-6, **kw):
    base = p[name]
    g = np.zeros_like(base)
    for idx in np.ndindex(base.shape):
        q = dict(p)
        plus, minus = base.copy(), base.copy()
        plus[idx] += eps
        minus[idx] -= eps
        q[name] = plus
        lp = _loss(q, dy, dlast, **kw)
        q[name] = minus
        lm = _loss(q, dy, dlast, **kw)
        g[idx] = (lp - lm) / (2 * eps)
    return g


CASES = [
    ("zoh", True, True, False),
    ("zoh", False, True, True),
    ("zoh", True, False, False),
    ("euler", True, True, False),
    ("euler", False, False, True),
]


@pytest.mark.parametrize("mode,gate,softplus,small_a", CASES)
def test_gradients_match_finite_differences(mode, gate, softplus, small_a):
    p = _problem(gate=gate, small_a=small_a)
    if not softplus:
        p["delta"] = np.abs(p["delta"]) + 0.05  # keep Delta = raw + bias positive
        p["delta_bias"] = np.abs(p["delta_bias"])
    batch, L, dim = p["u"].shape
    N = p["A"].shape[1]
    h0 = RNG.normal(size=(batch, dim, N))
    dy = RNG.normal(size=(batch, L, dim))
    dlast = RNG.normal(size=(batch, dim, N))
    kw = dict(softplus=softplus, dt_mode=mode)
    g = oracle.scan_bwd(**p, dy=dy, h0=h0, dlast=dlast, **kw)
    q = dict(p, h0=h0)
    names = [("u", "du"), ("delta", "ddelta"), ("A", "dA"), ("B", "dB"), ("C", "dC"),
             ("D", "dD"), ("delta_bias", "ddelta_bias"), ("h0", "dh0")]
    if gate:
        names.append(("z", "dz"))
    for inp, out in names:
        fd = _fd(q, inp, dy, dlast, **kw)
        scale = 1.0 + np.abs(fd).max()
        err = np.abs(g[out] - fd).max() / scale
        assert err < 1e-7, f"{out}: {err:.2e}"


# lengths and document starts: (seq_lens, reset positions per sequence)
VARLEN = [
    ([7, 4], [[3], [2]]),        # a short sequence; one document start in each
    ([7, 7], [[0, 5], []]),      # a start at token 0 discards h0
    ([5, 0], [[1, 2], [0]]),     # two starts in a row; an empty sequence
]


@pytest.mark.parametrize("mode", ["zoh", "euler"])
@pytest.mark.parametrize("lens,starts", VARLEN)
def test_lengths_and_resets_match_finite_differences(mode, lens, starts):
    """The loss through the forward with lengths and document starts (padding
    outputs are the constant 0; a start forgets the state): every gradient,
    h0's included, against central differences of that forward."""
    p = _problem(gate=True)
    batch, L, dim = p["u"].shape
    N = p["A"].shape[1]
    reset = np.zeros((batch, L), dtype=np.uint8)
    for b, ts in enumerate(starts):
        reset[b, ts] = 1
    h0 = RNG.normal(size=(batch, dim, N))
    dy = RNG.normal(size=(batch, L, dim))
    dlast = RNG.normal(size=(batch, dim, N))
    kw = dict(dt_mode=mode, seq_lens=np.array(lens), reset=reset)
    g = oracle.scan_bwd(**p, dy=dy, h0=h0, dlast=dlast, **kw)
    q = dict(p, h0=h0)
    for inp, out in [("u", "du"), ("delta", "ddelta"), ("A", "dA"), ("B", "dB"), ("C", "dC"),
                     ("D", "dD"), ("delta_bias", "ddelta_bias"), ("h0", "dh0"), ("z", "dz")]:
        fd = _fd(q, inp, dy, dlast, **kw)
        scale = 1.0 + np.abs(fd).max()
        err = np.abs(g[out] - fd).max() / scale
        assert err < 1e-7, f"{out}: {err:.2e}"
    for b, n in enumerate(lens):  # padding tokens: exactly zero
        for name in ("du", "ddelta", "dz"):
            assert np.all(g[name][b, n:] == 0.0)
        assert np.all(g["dB"][b, n:] == 0.0) and np.all(g["dC"][b, n:] == 0.0)


def test_padding_equals_the_truncated_sequence():
    """A sequence of length n padded to L has the gradients of the same
    sequence cut to n tokens (the padding only passes dlast through)."""
    p = _problem(gate=True, batch=1, L=9)
    n = 5
    h0 = RNG.normal(size=(1, 3, 4))
    dy = RNG.normal(size=(1, 9, 3))
    dlast = RNG.normal(size=(1, 3, 4))
    g = oracle.scan_bwd(**p, dy=dy, h0=h0, dlast=dlast, seq_lens=np.array([n]))
    cut = {k: (v[:, :n] if k in ("u", "delta", "B", "C", "z") else v) for k, v in p.items()}
    gc = oracle.scan_bwd(**cut, dy=dy[:, :n], h0=h0, dlast=dlast)
    for k in ("du", "ddelta", "dB", "dC", "dz"):
        np.testing.assert_array_equal(g[k][:, :n], gc[k])
    for k in ("dA", "dD", "ddelta_bias", "dh0"):
        np.testing.assert_array_equal(g[k], gc[k])


def test_gradient_of_last_state_alone():
    """With dy = 0 only the final state carries gradient: dC = 0, and du at the
    last token is B-weighted through bbar only."""
    p = _problem(gate=False)
    batch, L, dim = p["u"].shape
    N = p["A"].shape[1]
    dlast = RNG.normal(size=(batch, dim, N))
    g = oracle.scan_bwd(**p, dy=np.zeros((batch, L, dim)), dlast=dlast)
    assert np.all(g["dC"] == 0.0) and np.all(g["dD"] == 0.0)
    fd = _fd(p, "u", np.zeros((batch, L, dim)), dlast)
    np.testing.assert_allclose(g["du"], fd, rtol=1e-6, atol=1e-8)


def test_phi_prime_branches_agree():
    """phi'(k) from the series (|k| < 0.1) and from the closed form meet at the
    switch point, and the derivative of phi by finite differences matches."""
    for k in (-0.5, -0.1000001, -0.0999999, -0.01, -1e-6, 0.05):
        h = 1e-5
        phi = lambda x: np.expm1(x) / x
        fd = (phi(k + h) - phi(k - h)) / (2 * h)
        A = np.array([[k]])  # Delta = 1 so kappa = A; dbbar/dA = B phi'(kappa)
        g = oracle.scan_bwd(np.ones((1, 1, 1)), np.ones((1, 1, 1)), A, np.ones((1, 1, 1)),
                            np.zeros((1, 1, 1)), dy=np.zeros((1, 1, 1)), softplus=False,
                            h0=np.zeros((1, 1, 1)), dlast=np.ones((1, 1, 1)))
        assert g["dA"][0, 0] == pytest.approx(fd, rel=1e-8, abs=1e-10)
