"""GPU parity of ssm_ssd_fwd (Mamba-2 / SSD on the matrix cores) against the
oracle's plain recurrence, on the same bf16 bits: relative RMS <= 1e-2 on y
and on the final state (the bf16 bound of the scan; the kernel's operands are
bf16 and its sums fp32, which a numpy model of the same rounding puts at
about 2.5e-3)."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import DEV, assert_close, f64, to_dev, to_host64
import oracle
import selective_state_space_66_amd as ssm

pytestmark = pytest.mark.gpu


def _cfg(batch, L, H, N, gate, seed, P=64):
    return W.SSDConfig(f"s{batch}x{L}x{H}x{P}x{N}", batch, L, H, P, N, "bf16", gate, seed)


def _gpu(inp, mode, softplus=True, h0=None, use_D=True):
    y, last = ssm.ssd_fwd(to_dev(inp["x"], "bf16"), to_dev(inp["dt"], "f32"),
                          to_dev(inp["A"], "f32"), to_dev(inp["B"], "bf16"),
                          to_dev(inp["C"], "bf16"), D=to_dev(inp["D"], "f32") if use_D else None,
                          z=to_dev(inp["z"], "bf16") if inp["z"] is not None else None,
                          dt_bias=to_dev(inp["dt_bias"], "f32"), softplus=softplus,
                          dt_mode=mode, h0=None if h0 is None else to_dev(h0, "f32"))
    torch.cuda.synchronize()
    return y, last


def _ref(inp, mode, softplus=True, h0=None, use_D=True):
    return oracle.ssd_fwd(f64(inp["x"], "bf16"), inp["dt"].astype(np.float64), inp["A"],
                          f64(inp["B"], "bf16"), f64(inp["C"], "bf16"),
                          D=inp["D"] if use_D else None,
                          z=f64(inp["z"], "bf16") if inp["z"] is not None else None,
                          dt_bias=inp["dt_bias"], softplus=softplus, dt_mode=mode,
                          h0=None if h0 is None else h0.astype(np.float64))


@pytest.mark.parametrize("N", [64, 128])
@pytest.mark.parametrize("mode", ["euler", "zoh"])
@pytest.mark.parametrize("gate", [True, False])
def test_ssd_ragged(N, mode, gate):
    """3 chunks, the last 22 tokens long; an initial state."""
    inp = W.ssd_inputs(_cfg(2, 150, 3, N, gate, seed=110))
    h0 = np.random.default_rng(111).normal(size=(2, 3, 64, N)).astype(np.float32)
    y, last = _gpu(inp, mode, h0=h0)
    yr, lr = _ref(inp, mode, h0=h0)
    e1 = assert_close(to_host64(y), yr, "bf16", "y")
    e2 = assert_close(to_host64(last), lr, "bf16", "last_state")
    print(f"N={N} {mode} gate={gate}: y {e1:.2e} last {e2:.2e}", flush=True)


@pytest.mark.parametrize("P", [16, 32, 48, 128])
@pytest.mark.parametrize("N", [64, 128])
@pytest.mark.parametrize("mode", ["euler", "zoh"])
def test_ssd_head_sizes(P, N, mode):
    """Heads of 16, 32, 48 and 128 channels (one to eight 16-channel blocks per
    head), three chunks with a ragged last one, an initial state, the gate."""
    inp = W.ssd_inputs(_cfg(2, 150, 3, N, True, seed=120 + P, P=P))
    h0 = np.random.default_rng(121 + P).normal(size=(2, 3, P, N)).astype(np.float32)
    y, last = _gpu(inp, mode, h0=h0)
    yr, lr = _ref(inp, mode, h0=h0)
    assert y.shape == (2, 150, 3, P) and last.shape == (2, 3, P, N)
    assert_close(to_host64(y), yr, "bf16", f"y P={P}")
    assert_close(to_host64(last), lr, "bf16", f"last_state P={P}")


@pytest.mark.parametrize("L", [1, 17, 64, 65, 200])
def test_ssd_lengths(L):
    inp = W.ssd_inputs(_cfg(1, L, 2, 64, True, seed=112 + L))
    y, last = _gpu(inp, "euler")
    yr, lr = _ref(inp, "euler")
    assert_close(to_host64(y), yr, "bf16", "y")
    assert_close(to_host64(last), lr, "bf16", "last_state")


def test_ssd_softplus_off_no_skip():
    inp = W.ssd_inputs(_cfg(2, 100, 2, 128, False, seed=113))
    inp["dt"] = (np.abs(inp["dt"]) * 0.05).astype(np.float32)
    inp["dt_bias"] = np.abs(inp["dt_bias"]) * 0.01
    y, last = _gpu(inp, "zoh", softplus=False, use_D=False)
    yr, lr = _ref(inp, "zoh", softplus=False, use_D=False)
    assert_close(to_host64(y), yr, "bf16", "y")
    assert_close(to_host64(last), lr, "bf16", "last_state")


def test_ssd_chunked_prefill_and_empty():
    """Two calls, the second from the first's final state, equal one call; no
    tokens returns h0."""
    inp = W.ssd_inputs(_cfg(1, 200, 2, 64, True, seed=114))
    yr, lr = _ref(inp, "euler")
    a = {k: (v[:, :90] if k in ("x", "z", "dt", "B", "C") else v) for k, v in inp.items()}
    b = {k: (np.ascontiguousarray(v[:, 90:]) if k in ("x", "z", "dt", "B", "C") else v)
         for k, v in inp.items()}
    y1, l1 = _gpu({k: (np.ascontiguousarray(v) if isinstance(v, np.ndarray) else v)
                   for k, v in a.items()}, "euler")
    y2, l2 = _gpu(b, "euler", h0=to_host64(l1).astype(np.float32))
    y = torch.cat([y1, y2], dim=1)
    assert_close(to_host64(y), yr, "bf16", "y")
    assert_close(to_host64(l2), lr, "bf16", "last_state")
    h0 = torch.randn((2, 3, 64, 64), device=DEV)
    e = torch.zeros((2, 0, 3, 64), dtype=torch.bfloat16, device=DEV)
    eb = torch.zeros((2, 0, 64), dtype=torch.bfloat16, device=DEV)
    _, last = ssm.ssd_fwd(e, torch.zeros((2, 0, 3), device=DEV), torch.full((3,), -1.0, device=DEV),
                          eb, eb, h0=h0)
    torch.cuda.synchronize()
    assert torch.equal(last, h0)


def test_ssd_full_size_sampled():
    """The Mamba-2-130M-shaped layer at full size; the oracle checks two heads."""
    cfg = W.SSD_CONFIGS["ssd130m"]
    inp = W.ssd_inputs(cfg)
    heads = [0, 17]
    sub = W.ssd_inputs(cfg, heads=heads)
    hd = torch.tensor(heads, device=DEV)
    for mode in ("euler", "zoh"):
        y, last = _gpu(inp, mode)
        yr, lr = _ref(sub, mode)
        e1 = assert_close(to_host64(y.index_select(2, hd)), yr, "bf16", f"y {mode}")
        e2 = assert_close(to_host64(last.index_select(1, hd)), lr, "bf16", f"last {mode}")
        print(f"full {mode}: y {e1:.2e} last {e2:.2e}", flush=True)


# -------------------------------------------- the grouped kernel (three slices per block)

@pytest.mark.parametrize("N", [64, 128])
@pytest.mark.parametrize("mode", ["euler", "zoh"])
def test_ssd_grouped_ragged(N, mode):
    """128 sequences of 2 heads x 32 channels: 4 slices per batch entry, so
    256 blocks of three slices take the grouped kernel, and the second block
    of each entry has two spare groups.  Two chunks (the last ragged), h0."""
    inp = W.ssd_inputs(_cfg(128, 100, 2, N, True, seed=140 + N, P=32))
    h0 = np.random.default_rng(141).normal(size=(128, 2, 32, N)).astype(np.float32)
    y, last = _gpu(inp, mode, h0=h0)
    yr, lr = _ref(inp, mode, h0=h0)
    assert_close(to_host64(y), yr, "bf16", f"grouped y N={N} {mode}")
    assert_close(to_host64(last), lr, "bf16", f"grouped last N={N} {mode}")


def test_ssd_grouped_equals_one_slice():
    """Every batch entry is independent, and the grouped kernel runs each
    slice's arithmetic exactly as the one-slice kernel: entry 5 of a 96-entry
    run (grouped: 96 x 4 blocks) equals the same entry run alone (one-slice:
    12 blocks), bit for bit."""
    inp = W.ssd_inputs(_cfg(96, 150, 3, 128, True, seed=142, P=64))
    h0 = np.random.default_rng(143).normal(size=(96, 3, 64, 128)).astype(np.float32)
    y, last = _gpu(inp, "zoh", h0=h0)
    one = {k: (v[5:6] if isinstance(v, np.ndarray) and v.ndim >= 2 and v.shape[0] == 96 else v)
           for k, v in inp.items()}
    y1, last1 = _gpu(one, "zoh", h0=h0[5:6])
    assert torch.equal(y[5:6], y1) and torch.equal(last[5:6], last1)
