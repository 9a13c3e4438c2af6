"""Pins for the oracle's causal depthwise convolution ("The Mamba block" on the
first page) and its decoding window ("Decoding with a constant-size cache").
Expected values come from numpy.convolve and scipy's logistic function, from
the impulse response, and from independent routes to the same result (step by
step against the whole sequence, split sequences against one)."""
import numpy as np
import pytest
from scipy.special import expit

import oracle

RNG = np.random.default_rng(4242)


def _problem(batch=2, L=30, dim=5, k=4):
    return (RNG.normal(size=(batch, L, dim)), RNG.uniform(-0.5, 0.5, size=(dim, k)),
            RNG.uniform(-0.5, 0.5, size=dim))


def test_impulse_response_is_the_weights():
    """An input of 1 at t0 and 0 elsewhere gives, before the activation, the
    weight w_i at t0 + i (depthwise: each channel its own weights), plus the bias."""
    x = np.zeros((1, 12, 3))
    x[0, 4, :] = 1.0
    w = np.arange(12, dtype=np.float64).reshape(3, 4) + 1.0
    b = np.array([0.5, -1.0, 2.0])
    out, _ = oracle.conv1d_fwd(x, w, b, silu=False)
    for c in range(3):
        expect = np.full(12, b[c])
        expect[4:8] += w[c]
        np.testing.assert_array_equal(out[0, :, c], expect)


@pytest.mark.parametrize("k", [1, 2, 3, 4])
@pytest.mark.parametrize("silu", [True, False])
def test_matches_numpy_convolve(k, silu):
    """Per channel, the causal convolution is the first L terms of the full
    discrete convolution of the input with the channel's taps."""
    x, w, b = _problem(k=k)
    out, _ = oracle.conv1d_fwd(x, w, b, silu=silu)
    L = x.shape[1]
    for bi in range(x.shape[0]):
        for c in range(x.shape[2]):
            pre = np.convolve(x[bi, :, c], w[c])[:L] + b[c]
            ref = pre * expit(pre) if silu else pre
            np.testing.assert_allclose(out[bi, :, c], ref, rtol=1e-13, atol=1e-14)


def test_steps_reproduce_the_whole_sequence():
    """Decoding token by token with the window of inputs reproduces the forward
    pass at every step (the requirement stated for the decoding step)."""
    x, w, b = _problem()
    out, st_end = oracle.conv1d_fwd(x, w, b)
    win = np.zeros((2, 3, 5))
    for t in range(x.shape[1]):
        o, win = oracle.conv1d_step(win, x[:, t], w, b)
        np.testing.assert_allclose(o, out[:, t], rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(win, st_end)
    np.testing.assert_array_equal(st_end, x[:, -3:, :])  # the last three inputs, oldest first


def test_chunked_prefill_carries_the_window():
    x, w, b = _problem(L=40)
    out, st = oracle.conv1d_fwd(x, w, b)
    o1, s1 = oracle.conv1d_fwd(x[:, :17], w, b)
    o2, s2 = oracle.conv1d_fwd(x[:, 17:], w, b, state_in=s1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), out, rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(s2, st)
    # a chunk shorter than the window keeps the older inputs in it
    o3, s3 = oracle.conv1d_fwd(x[:, 17:19], w, b, state_in=s1)
    np.testing.assert_array_equal(s3, x[:, 16:19])


def test_reset_equals_separate_documents():
    x, w, b = _problem(L=30)
    reset = np.zeros((2, 30), dtype=bool)
    reset[0, 11] = True
    reset[1, 2] = True
    win0 = RNG.normal(size=(2, 3, 5))
    out, st = oracle.conv1d_fwd(x, w, b, state_in=win0, reset=reset)
    for bi, cut in ((0, 11), (1, 2)):
        oa, _ = oracle.conv1d_fwd(x[bi:bi + 1, :cut], w, b, state_in=win0[bi:bi + 1])
        ob, sb = oracle.conv1d_fwd(x[bi:bi + 1, cut:], w, b)
        np.testing.assert_array_equal(out[bi, :cut], oa[0])
        np.testing.assert_array_equal(out[bi, cut:], ob[0])
        np.testing.assert_array_equal(st[bi], sb[0])
    # a document of one token: its window is zeros except that token
    r2 = np.zeros((2, 30), dtype=bool)
    r2[:, 29] = True
    _, s = oracle.conv1d_fwd(x, w, b, reset=r2)
    assert np.all(s[:, :2] == 0.0)
    np.testing.assert_array_equal(s[:, 2], x[:, 29])


def test_seq_lens_equal_truncation():
    x, w, b = _problem(batch=4, L=20)
    win0 = RNG.normal(size=(4, 3, 5))
    lens = [20, 9, 2, 0]
    out, st = oracle.conv1d_fwd(x, w, b, state_in=win0, seq_lens=lens)
    for bi, l in enumerate(lens):
        ot, stt = oracle.conv1d_fwd(x[bi:bi + 1, :l], w, b, state_in=win0[bi:bi + 1])
        np.testing.assert_array_equal(out[bi, :l], ot[0])
        assert np.all(out[bi, l:] == 0.0)
        np.testing.assert_array_equal(st[bi], stt[0])
    # length 2 keeps the newest carried-in input; length 0 keeps the whole window
    np.testing.assert_array_equal(st[2], np.concatenate([win0[2, 2:], x[2, :2]]))
    np.testing.assert_array_equal(st[3], win0[3])


def test_pointwise_width_one():
    x, w, b = _problem(k=1)
    out, st = oracle.conv1d_fwd(x, w, b, silu=False)
    np.testing.assert_allclose(out, x * w[:, 0] + b, rtol=1e-15, atol=0)
    assert st.shape == (2, 0, 5)
