"""Pins for the fp64 oracle: the pages' worked numbers, closed forms, brute force
and invariants.  None of these re-calls the oracle's own routine to produce the
expected value; each checks it against something fixed independently of it.
"""
import math

import numpy as np
import pytest
from scipy import signal

import oracle

RNG = np.random.default_rng(12345)


def _scan1(x, delta_raw, A=-1.0, B=1.0, C=1.0, D=0.0, softplus=False, dt_mode="zoh", bias=0.0,
           z=None, h0=None):
    """Single batch, single channel, N = 1 scan with constant B, C."""
    x = np.asarray(x, dtype=np.float64)
    L = len(x)
    u = x.reshape(1, L, 1)
    d = np.asarray(delta_raw, dtype=np.float64).reshape(1, L, 1)
    Bm = np.full((1, L, 1), B)
    Cm = np.full((1, L, 1), C)
    zz = None if z is None else np.asarray(z, dtype=np.float64).reshape(1, L, 1)
    hh = None if h0 is None else np.array(h0, dtype=np.float64).reshape(1, 1, 1)
    y, last = oracle.scan_fwd(u, d, np.array([[A]]), Bm, Cm, D=np.array([D]), z=zz,
                              delta_bias=np.array([bias]), softplus=softplus, dt_mode=dt_mode,
                              h0=hh)
    return y.reshape(L), last.reshape(())


# ---------------------------------------------------------------- page numbers

def test_zoh_worked_numbers(pages):
    g = pages["zoh"]
    for case in g["cases"]:
        ab, bb = oracle.discretize(case["delta"], g["A"], g["B"], "zoh")
        assert abs(ab - case["abar"]) <= case["tol"]
        assert abs(bb - case["bbar"]) <= case["tol"]
        # with A = -1, B = 1 the two shares add up to one (same section)
        assert ab + bb == pytest.approx(1.0, abs=1e-15)


def test_selective_copy_by_hand(pages):
    g = pages["selective_copy_by_hand"]
    # softplus off: Delta is given directly; A = -1, B = C = 1, D = 0, ZOH
    y, last = _scan1(g["x"], g["delta"], softplus=False, dt_mode="zoh")
    assert np.max(np.abs(y - np.array(g["h"]))) <= g["tol"]
    assert abs(last - g["h"][-1]) <= g["tol"]


@pytest.mark.parametrize("mode", ["zoh", "euler"])
def test_tea_example(pages, mode):
    """Abar = 0.5, Bbar = 1 realised as A = -1, raw = 0, bias = 0, softplus on
    (Delta = ln 2, abar = 0.5) with B = 2 under ZOH ((0.5 - 1)/(-1) * 2 = 1) or
    B = 1/ln 2 under exponential-Euler (ln 2 * B = 1)."""
    g = pages["tea_recurrence"]
    Bv = 2.0 if mode == "zoh" else 1.0 / math.log(2.0)
    y, last = _scan1(g["x"], [0.0] * 4, B=Bv, softplus=True, dt_mode=mode)
    np.testing.assert_allclose(y, g["y"], rtol=0, atol=1e-12)
    # the convolution road of the same section: y_4 = sum_k K_k x_{4-k}
    K = np.array(g["kernel"])
    assert float(np.dot(K, np.array(g["x"])[::-1])) == pytest.approx(y[-1], abs=1e-12)


def test_merge_example(pages):
    g = pages["merge"]
    s = [tuple(p) for p in g["steps"]]
    p01 = oracle.combine(s[0], s[1])
    p23 = oracle.combine(s[2], s[3])
    assert p01 == pytest.approx(tuple(g["pair01"]), abs=g["tol"])
    assert p23 == pytest.approx(tuple(g["pair23"]), abs=g["tol"])
    assert oracle.combine(p01, p23) == pytest.approx(tuple(g["all"]), abs=g["tol"])
    # associativity on random triples
    for _ in range(20):
        a, b, c = (tuple(RNG.normal(size=2)) for _ in range(3))
        left = oracle.combine(oracle.combine(a, b), c)
        right = oracle.combine(a, oracle.combine(b, c))
        assert left == pytest.approx(right, rel=1e-12, abs=1e-12)


def test_theorem1_numbers(pages):
    g = pages["theorem1"]
    for case in g["cases"]:
        d = oracle.softplus(case["z"])
        ab, bb = oracle.discretize(d, -1.0, 1.0, "zoh")
        assert abs(d - case["delta"]) <= case["tol"]
        assert abs(ab - case["abar"]) <= case["tol"]
        assert abs(bb - case["gate"]) <= case["tol"]
        assert abs(oracle.sigmoid(case["z"]) - case["gate"]) <= case["tol"]


def test_theorem1_gate_identity(pages):
    """Selection is a gate: with N = 1, A = -1, B = 1, ZOH and Delta = softplus(z),
    h_t = (1 - sigma(z_t)) h_{t-1} + sigma(z_t) x_t; extreme z stay finite."""
    T = 200
    zs = RNG.normal(scale=4.0, size=T)
    zs[::37] = 1000.0
    zs[5::41] = -1000.0
    x = RNG.normal(size=T)
    y, _ = _scan1(x, zs, softplus=True, dt_mode="zoh")
    h = 0.0
    ref = []
    for zt, xt in zip(zs, x):
        g = 1.0 / (1.0 + math.exp(-zt)) if zt >= 0 else math.exp(zt) / (1.0 + math.exp(zt))
        h = (1.0 - g) * h + g * xt
        ref.append(h)
    assert np.all(np.isfinite(y))
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    # exponential-Euler: same decay, the write becomes softplus(z) itself
    y2, _ = _scan1(x, zs, softplus=True, dt_mode="euler")
    h = 0.0
    ref2 = []
    for zt, xt in zip(zs, x):
        sp = max(zt, 0.0) + math.log1p(math.exp(-abs(zt)))
        g = 1.0 / (1.0 + math.exp(-zt)) if zt >= 0 else math.exp(zt) / (1.0 + math.exp(zt))
        h = (1.0 - g) * h + sp * xt
        ref2.append(h)
    assert np.all(np.isfinite(y2))
    np.testing.assert_allclose(y2, ref2, rtol=1e-12, atol=1e-12)


def test_softplus_numbers(pages):
    g = pages["softplus"]
    for case in g["cases"]:
        assert abs(oracle.softplus(case["v"]) - case["out"]) <= g["tol"]
    for v in (1000.0, -1000.0, 0.0, 30.0, -30.0):
        assert math.isfinite(oracle.softplus(v))
    assert oracle.softplus(1000.0) == 1000.0
    assert oracle.softplus(0.0) == pytest.approx(math.log(2.0), abs=1e-16)


def test_softplus_inverse_numbers(pages):
    g = pages["softplus_inverse"]
    for case in g["cases"]:
        # the printed bias maps back to its step size through the oracle's softplus
        assert oracle.softplus(case["bias"]) == pytest.approx(case["u"], rel=5e-3)


def test_io_count(pages):
    g = pages["io_count"]
    B, L, D, N = 1, 2048, 1024, 16
    assert B * L * D * N == g["plain"]
    assert B * L * D + D * N == g["fused"]


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("mode", ["zoh", "euler"])
def test_lti_first_order_iir(mode):
    """N = 1 with constant Delta, B, C: the scan is the textbook first-order IIR
    filter y = C * lfilter([bbar], [1, -abar], x) + D x."""
    L = 300
    x = RNG.normal(size=L)
    A, Bv, Cv, Dv, dt = -0.7, 1.3, -0.4, 0.25, 0.37
    y, _ = _scan1(x, np.full(L, dt), A=A, B=Bv, C=Cv, D=Dv, softplus=False, dt_mode=mode)
    abar = math.exp(dt * A)
    bbar = (abar - 1.0) / A * Bv if mode == "zoh" else dt * Bv
    ref = Cv * signal.lfilter([bbar], [1.0, -abar], x) + Dv * x
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("mode", ["zoh", "euler"])
def test_lti_convolution_kernel(mode):
    """Delta, B, C held constant over t: y = Kbar * u + D u with
    Kbar_j = sum_n C_n abar_n^j bbar_n (the convolution form)."""
    batch, L, dim, N = 2, 96, 3, 5
    u = RNG.normal(size=(batch, L, dim))
    A = -np.exp(RNG.normal(size=(dim, N)))
    Bc = RNG.normal(size=(batch, N))
    Cc = RNG.normal(size=(batch, N))
    Dv = RNG.normal(size=dim)
    dts = np.exp(RNG.uniform(np.log(1e-2), np.log(1.0), size=dim))
    delta = np.broadcast_to(dts, (batch, L, dim)).copy()
    Bm = np.broadcast_to(Bc[:, None, :], (batch, L, N)).copy()
    Cm = np.broadcast_to(Cc[:, None, :], (batch, L, N)).copy()
    y, _ = oracle.scan_fwd(u, delta, A, Bm, Cm, D=Dv, softplus=False, dt_mode=mode)
    for b in range(batch):
        for c in range(dim):
            abar = np.exp(dts[c] * A[c])
            bbar = (abar - 1.0) / A[c] * Bc[b] if mode == "zoh" else dts[c] * Bc[b]
            j = np.arange(L)[:, None]
            K = np.sum(Cc[b][None, :] * abar[None, :] ** j * bbar[None, :], axis=1)
            ref = np.convolve(u[b, :, c], K)[:L] + Dv[c] * u[b, :, c]
            np.testing.assert_allclose(y[b, :, c], ref, rtol=1e-10, atol=1e-10)


def _mixing_matrix_ref(u, delta_raw, A, B, C, D, z, bias, softplus, mode):
    """Brute force from the mixing-matrix theorem ("Selection breaks the
    convolution"): M_ts = sum_n C_tn exp(A_n sum_{r=s+1..t} Delta_r) bbar_sn,
    y = M u + D u, then the SiLU gate.  O(L^2 N), no recurrence."""
    batch, L, dim = u.shape
    N = A.shape[1]
    y = np.empty_like(u)
    for b in range(batch):
        for c in range(dim):
            v = delta_raw[b, :, c] + bias[c]
            dlt = np.logaddexp(0.0, v) if softplus else v
            S = np.concatenate([[0.0], np.cumsum(dlt)])  # S[t+1] = sum_{r<=t} Delta_r
            M = np.zeros((L, L))
            for n in range(N):
                a = A[c, n]
                if mode == "zoh":
                    bbar = (np.expm1(dlt * a) / a if a != 0 else dlt) * B[b, :, n]
                else:
                    bbar = dlt * B[b, :, n]
                seg = S[1:, None] - S[None, 1:]           # sum_{r=s+1..t} Delta_r
                tri = np.tri(L, dtype=bool)
                decay = np.where(tri, np.exp(a * np.where(tri, seg, 0.0)), 0.0)
                M += C[b, :, n][:, None] * decay * bbar[None, :]
            out = M @ u[b, :, c] + D[c] * u[b, :, c]
            if z is not None:
                zz = z[b, :, c]
                out = out * zz / (1.0 + np.exp(-zz))
            y[b, :, c] = out
    return y


@pytest.mark.parametrize("mode", ["zoh", "euler"])
@pytest.mark.parametrize("gate", [False, True])
@pytest.mark.parametrize("softplus", [True, False])
def test_brute_force_mixing_matrix(mode, gate, softplus):
    batch, L, dim, N = 2, 48, 3, 4
    u = RNG.normal(size=(batch, L, dim))
    raw = RNG.normal(size=(batch, L, dim))
    if not softplus:
        raw = np.abs(raw) * 0.3  # a positive step size when given directly
    A = -np.exp(RNG.normal(size=(dim, N)))
    A[1, 2] = 0.0  # the ZOH limit bbar = Delta B
    B = RNG.normal(size=(batch, L, N))
    C = RNG.normal(size=(batch, L, N))
    D = RNG.normal(size=dim)
    bias = RNG.normal(size=dim) * 0.5 - 1.0
    z = RNG.normal(size=(batch, L, dim)) if gate else None
    y, _ = oracle.scan_fwd(u, raw, A, B, C, D=D, z=z, delta_bias=bias, softplus=softplus,
                           dt_mode=mode)
    ref = _mixing_matrix_ref(u, raw, A, B, C, D, z, bias, softplus, mode)
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- invariants

def _cut(p, s0, s1):
    """The tokens [s0, s1) of a problem dict (per-channel parameters kept)."""
    return {k: (v[:, s0:s1] if (k in ("u", "delta", "z", "B", "C") and v is not None) else v)
            for k, v in p.items()}


def _rand_problem(batch=2, L=40, dim=5, N=16, gate=True):
    return dict(
        u=RNG.normal(size=(batch, L, dim)),
        delta=RNG.normal(size=(batch, L, dim)),
        A=-(np.arange(N) + 1.0)[None, :].repeat(dim, 0) * np.exp(RNG.normal(size=(dim, 1)) * 0.3),
        B=RNG.normal(size=(batch, L, N)),
        C=RNG.normal(size=(batch, L, N)),
        D=RNG.normal(size=dim),
        z=RNG.normal(size=(batch, L, dim)) if gate else None,
        delta_bias=np.log(np.expm1(np.exp(RNG.uniform(np.log(1e-3), np.log(1e-1), size=dim)))),
    )


@pytest.mark.parametrize("mode", ["zoh", "euler"])
def test_causality(mode):
    p = _rand_problem()
    y0, _ = oracle.scan_fwd(**p, dt_mode=mode)
    t = 17
    p2 = dict(p)
    p2["u"] = p["u"].copy()
    p2["u"][:, t, :] += 3.0
    y1, _ = oracle.scan_fwd(**p2, dt_mode=mode)
    assert np.array_equal(y0[:, :t], y1[:, :t])
    assert not np.allclose(y0[:, t], y1[:, t])


@pytest.mark.parametrize("mode", ["zoh", "euler"])
def test_linearity_in_u(mode):
    p = _rand_problem(gate=False)
    u2 = RNG.normal(size=p["u"].shape)
    ya, _ = oracle.scan_fwd(**p, dt_mode=mode)
    yb, _ = oracle.scan_fwd(**{**p, "u": u2}, dt_mode=mode)
    yc, _ = oracle.scan_fwd(**{**p, "u": 2.0 * p["u"] - 0.5 * u2}, dt_mode=mode)
    np.testing.assert_allclose(yc, 2.0 * ya - 0.5 * yb, rtol=1e-10, atol=1e-11)


def test_zero_input_gives_zero():
    p = _rand_problem()
    p["u"] = np.zeros_like(p["u"])
    y, last = oracle.scan_fwd(**p)
    assert np.all(y == 0.0) and np.all(last == 0.0)


@pytest.mark.parametrize("mode", ["zoh", "euler"])
def test_zero_step_passes_state_through(mode):
    """Delta = 0 (softplus off, raw = bias = 0): the token is ignored, the state
    is untouched, and y = D u (gated)."""
    p = _rand_problem()
    h0 = RNG.normal(size=(2, 5, 16))
    p["delta"] = np.zeros_like(p["delta"])
    p["delta_bias"] = np.zeros(5)
    y, last = oracle.scan_fwd(**p, softplus=False, dt_mode=mode, h0=h0)
    np.testing.assert_array_equal(last, h0)
    z = p["z"]
    read = np.einsum("bln,bcn->blc", p["C"], h0)
    ref = (read + p["D"] * p["u"]) * z / (1.0 + np.exp(-z))
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_zoh_saturation():
    """Under ZOH the write saturates at B/|A| as Delta grows; under
    exponential-Euler it keeps growing like Delta B."""
    for a in (-0.5, -1.0, -7.0):
        _, bb = oracle.discretize(1e4, a, 1.7, "zoh")
        assert bb == pytest.approx(1.7 / abs(a), rel=1e-12)
        _, be = oracle.discretize(1e4, a, 1.7, "euler")
        assert be == pytest.approx(1.7e4, rel=1e-12)


def test_channel_and_batch_permutation_equivariance():
    p = _rand_problem(batch=3, dim=6)
    y, last = oracle.scan_fwd(**p)
    perm = RNG.permutation(6)
    q = dict(p)
    for k in ("u", "delta", "z"):
        q[k] = p[k][:, :, perm]
    q["A"] = p["A"][perm]
    q["D"] = p["D"][perm]
    q["delta_bias"] = p["delta_bias"][perm]
    y2, last2 = oracle.scan_fwd(**q)
    np.testing.assert_array_equal(y2, y[:, :, perm])
    np.testing.assert_array_equal(last2, last[:, perm])
    bp = np.array([2, 0, 1])
    r = {k: (v[bp] if k in ("u", "delta", "z", "B", "C") else v) for k, v in p.items()}
    y3, last3 = oracle.scan_fwd(**r)
    np.testing.assert_array_equal(y3, y[bp])
    np.testing.assert_array_equal(last3, last[bp])


@pytest.mark.parametrize("mode", ["zoh", "euler"])
def test_scan_equals_repeated_steps(mode):
    """Decoding token by token reproduces the full forward at every step
    ("Decoding with a constant-size cache")."""
    p = _rand_problem()
    y, last = oracle.scan_fwd(**p, dt_mode=mode)
    st = np.zeros((2, 5, 16))
    for t in range(p["u"].shape[1]):
        yt, st = oracle.step(st, p["u"][:, t], p["delta"][:, t], p["A"], p["B"][:, t],
                             p["C"][:, t], D=p["D"], z=p["z"][:, t], delta_bias=p["delta_bias"],
                             dt_mode=mode)
        np.testing.assert_allclose(yt, y[:, t], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(st, last, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("mode", ["zoh", "euler"])
def test_prefill_then_decode(mode):
    """Prefill keeps only the final state; scanning u[:L1] and then stepping
    through u[L1:] reproduces scan(u)."""
    p = _rand_problem()
    y, last = oracle.scan_fwd(**p, dt_mode=mode)
    L1 = 23
    head = _cut(p, 0, L1)
    yh, st = oracle.scan_fwd(**head, dt_mode=mode)
    np.testing.assert_allclose(yh, y[:, :L1], rtol=1e-13, atol=1e-14)
    for t in range(L1, p["u"].shape[1]):
        yt, st = oracle.step(st, p["u"][:, t], p["delta"][:, t], p["A"], p["B"][:, t],
                             p["C"][:, t], D=p["D"], z=p["z"][:, t], delta_bias=p["delta_bias"],
                             dt_mode=mode)
        np.testing.assert_allclose(yt, y[:, t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(st, last, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("mode", ["zoh", "euler"])
def test_segment_composition_with_combine(mode):
    """Splitting L into segments and composing each segment's (decay, end-state)
    pair with the associative combine gives the same final state as the
    sequential recurrence; the scan from a non-zero h0 agrees with it."""
    p = _rand_problem(batch=1, dim=2, N=3, gate=False)
    _, last = oracle.scan_fwd(**p, dt_mode=mode)
    L = p["u"].shape[1]
    cuts = [0, 7, 19, 31, L]
    pairs = []
    for s0, s1 in zip(cuts[:-1], cuts[1:]):
        seg = _cut(p, s0, s1)
        _, end = oracle.scan_fwd(**seg, dt_mode=mode)  # zero initial state
        dsum = np.logaddexp(0.0, seg["delta"][0] + p["delta_bias"]).sum(axis=0)  # (dim,)
        decay = np.exp(dsum[:, None] * p["A"])  # product of abar over the segment
        pairs.append((decay, end[0]))
    for c in range(2):
        for n in range(3):
            acc = (1.0, 0.0)
            for dec, end in pairs:
                acc = oracle.combine(acc, (dec[c, n], end[c, n]))
            assert acc[1] == pytest.approx(last[0, c, n], rel=1e-11, abs=1e-13)
    # h0 route: scan the tail from the state after the first cut
    head = _cut(p, 0, 19)
    tail = _cut(p, 19, L)
    _, mid = oracle.scan_fwd(**head, dt_mode=mode)
    _, end2 = oracle.scan_fwd(**tail, dt_mode=mode, h0=mid)
    np.testing.assert_allclose(end2, last, rtol=1e-12, atol=1e-13)


def test_threads_do_not_change_results():
    p = _rand_problem(batch=3, dim=7)
    y1, l1 = oracle.scan_fwd(**p, nthreads=1)
    y8, l8 = oracle.scan_fwd(**p, nthreads=8)
    assert np.array_equal(y1, y8) and np.array_equal(l1, l8)


def test_empty_sequence():
    p = _rand_problem(L=0)
    y, last = oracle.scan_fwd(**p)
    assert y.shape == (2, 0, 5) and np.all(last == 0.0)


# ------------------------------------------- initial state, lengths, resets


def _one(p, b):
    """Batch entry b of a problem dict, as a batch of one."""
    return {k: (v[b:b + 1] if (k in ("u", "delta", "z", "B", "C") and v is not None) else v)
            for k, v in p.items()}


@pytest.mark.parametrize("mode", ["zoh", "euler"])
def test_seq_lens_equal_truncation(mode):
    """A sequence of length l followed by padding gives, on its l real tokens,
    exactly the scan of those tokens alone; padded positions output 0 and the
    final state is the state after token l - 1."""
    p = _rand_problem(batch=4, L=30)
    h0 = RNG.normal(size=(4, 5, 16))
    lens = [30, 17, 1, 0]
    y, last = oracle.scan_fwd(**p, dt_mode=mode, h0=h0, seq_lens=lens)
    for b, l in enumerate(lens):
        yb, lb = oracle.scan_fwd(**_cut(_one(p, b), 0, l), dt_mode=mode, h0=h0[b:b + 1])
        np.testing.assert_array_equal(y[b, :l], yb[0])
        assert np.all(y[b, l:] == 0.0)
        np.testing.assert_array_equal(last[b], lb[0])
    # lengths outside [0, L] are clamped
    y2, last2 = oracle.scan_fwd(**p, dt_mode=mode, h0=h0, seq_lens=[99, 17, 1, -5])
    np.testing.assert_array_equal(y2, y)
    np.testing.assert_array_equal(last2, last)


@pytest.mark.parametrize("mode", ["zoh", "euler"])
def test_reset_equals_separate_documents(mode):
    """Two documents packed into one sequence with a reset at the break give
    exactly the two documents scanned separately, the second from zero."""
    p = _rand_problem(batch=2, L=40)
    h0 = RNG.normal(size=(2, 5, 16))
    reset = np.zeros((2, 40), dtype=bool)
    reset[0, 13] = True
    reset[1, 29] = True
    y, last = oracle.scan_fwd(**p, dt_mode=mode, h0=h0, reset=reset)
    for b, cut in ((0, 13), (1, 29)):
        one = _one(p, b)
        ya, _ = oracle.scan_fwd(**_cut(one, 0, cut), dt_mode=mode, h0=h0[b:b + 1])
        yb, lb = oracle.scan_fwd(**_cut(one, cut, 40), dt_mode=mode)
        np.testing.assert_array_equal(y[b, :cut], ya[0])
        np.testing.assert_array_equal(y[b, cut:], yb[0])
        np.testing.assert_array_equal(last[b], lb[0])


def test_reset_at_start_discards_h0():
    p = _rand_problem(batch=2, L=12)
    reset = np.zeros((2, 12), dtype=bool)
    reset[:, 0] = True
    y, last = oracle.scan_fwd(**p, h0=RNG.normal(size=(2, 5, 16)), reset=reset)
    y0, last0 = oracle.scan_fwd(**p)
    np.testing.assert_array_equal(y, y0)
    np.testing.assert_array_equal(last, last0)


def test_left_padding_with_reset():
    """Left padding (garbage before the real tokens) with a reset at the first
    real token gives the unpadded scan on the real tokens."""
    p = _rand_problem(batch=1, L=25)
    pad = 9
    reset = np.zeros((1, 25), dtype=bool)
    reset[0, pad] = True
    y, last = oracle.scan_fwd(**p, reset=reset)
    yr, lr = oracle.scan_fwd(**_cut(p, pad, 25))
    np.testing.assert_array_equal(y[:, pad:], yr)
    np.testing.assert_array_equal(last, lr)


def test_large_step_resets_like_the_flag():
    """"One token with a large Delta" resets the state ("What each parameter
    does" on the first page): under ZOH a step of 1e4 makes abar = exp(Delta A)
    underflow to 0, so the scan equals the scan with a reset flag at that token
    (same Delta), and nothing before it reaches the outputs after it."""
    p = _rand_problem(batch=1, L=30)
    p["delta_bias"] = np.zeros(5)
    p["delta"] = np.abs(p["delta"]) * 0.1
    p["delta"][0, 11, :] = 1e4
    y, last = oracle.scan_fwd(**p, softplus=False)
    reset = np.zeros((1, 30), dtype=bool)
    reset[0, 11] = True
    yf, lf = oracle.scan_fwd(**p, softplus=False, reset=reset)
    np.testing.assert_array_equal(y, yf)
    np.testing.assert_array_equal(last, lf)
    q = dict(p)
    q["u"] = p["u"].copy()
    q["u"][0, :11] += RNG.normal(size=(11, 5))
    y2, _ = oracle.scan_fwd(**q, softplus=False)
    np.testing.assert_array_equal(y2[:, 11:], y[:, 11:])
