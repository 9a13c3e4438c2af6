"""The seeded input generator: determinism, subset consistency, distributions,
the bf16 rounding rule and the long-sequence filler structure."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W


def test_bf16_rounding_matches_torch():
    x = np.concatenate([W.normal(7, 1, np.arange(200_000)),
                        np.array([1.0, -1.0, 0.0, 3.0e38, 1e-40, 1.00390625, 1.01171875],
                                 dtype=np.float32)])
    ours = W.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = W.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_counter_based_subsets_agree():
    cfg = W.ScanConfig("t", 2, 33, 70, 16, "bf16", True, 11)
    full = W.scan_inputs(cfg)
    ch = [69, 0, 13, 13, 40]
    sub = W.scan_inputs(cfg, channels=ch)
    for k in ("u", "delta", "z"):
        assert np.array_equal(sub[k], full[k][:, :, ch])
    for k in ("A", "D", "delta_bias"):
        assert np.array_equal(sub[k], full[k][ch])
    assert np.array_equal(sub["B"], full["B"]) and np.array_equal(sub["C"], full["C"])
    again = W.scan_inputs(cfg)
    for k in ("u", "delta", "z", "B", "C"):
        assert np.array_equal(again[k], full[k])


def test_distributions():
    x = W.normal(3, 5, np.arange(400_000))
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01
    u = W.uniform(3, 6, np.arange(400_000))
    assert u.min() > 0.0 and u.max() < 1.0 and abs(u.mean() - 0.5) < 0.01
    A, D, bias = W.channel_params(5, 4096, 16)
    assert np.array_equal(A[17], -(np.arange(16) + 1.0).astype(np.float32))
    dt = np.array([oracle.softplus(float(b)) for b in bias[:512]])
    assert dt.min() >= 1e-3 * (1 - 1e-5) and dt.max() <= 1e-1 * (1 + 1e-5)
    # log-uniform: the mean of log(dt) sits mid-range
    assert abs(np.log(dt).mean() - 0.5 * (np.log(1e-3) + np.log(1e-1))) < 0.2


def test_streams_differ():
    a = W.normal(1, W.S_U, np.arange(1000))
    b = W.normal(1, W.S_DELTA, np.arange(1000))
    c = W.normal(2, W.S_U, np.arange(1000))
    assert not np.array_equal(a, b) and not np.array_equal(a, c)
    s0 = W.step_inputs(W.STEP_CONFIGS["decode"], 0, channels=[0, 1])
    s1 = W.step_inputs(W.STEP_CONFIGS["decode"], 1, channels=[0, 1])
    assert not np.array_equal(s0["u"], s1["u"])


def test_filler_structure():
    cfg = W.ScanConfig("f", 3, 512, 40, 16, "bf16", False, 3, filler=True)
    inp = W.scan_inputs(cfg)
    u = inp["u"]
    filler = W.to_bf16_bits(W.normal(3, W.S_U, np.arange(40)))
    for b in range(3):
        odd = [t for t in range(512) if not np.array_equal(u[b, t], filler)]
        assert len(odd) == 16
    assert inp["z"] is None


@pytest.mark.parametrize("name", sorted(W.SCAN_CONFIGS))
def test_scan_config_shapes(name):
    cfg = W.SCAN_CONFIGS[name]
    inp = W.scan_inputs(cfg, channels=[0, cfg.dim - 1]) if cfg.L * cfg.batch > 100_000 \
        else W.scan_inputs(cfg)
    k = len(inp["channels"])
    assert inp["u"].shape == (cfg.batch, cfg.L, k)
    assert inp["B"].shape == (cfg.batch, cfg.L, cfg.N)
    assert inp["A"].shape == (k, cfg.N)
    assert (inp["z"] is not None) == cfg.gate
