"""Seeded input generators: determinism, bf16 rounding, shapes (CPU only)."""
import numpy as np
import torch

import workloads as W


def test_bf16_rounding_matches_torch():
    a = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 3
    # include exact ties between two bf16 neighbours
    ties = (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    a = np.concatenate([a, ties, -ties])
    ours = W.round_bf16(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours, ref)


def test_deterministic_and_distinct_seeds():
    w = W.custom(T=33, d=16, f=24, E=4, k=2, bias_std=1.0)
    a, b = W.make_inputs(w), W.make_inputs(w)
    for key in a:
        if a[key] is None:
            continue
        assert np.array_equal(a[key], b[key]), key
    c = W.make_inputs(W.with_seed(w, (42, 99)))
    assert not np.array_equal(a["x"], c["x"])


def test_workload_shapes_and_bf16_exact():
    for w in (W.TINY_FP32, W.MID_BF16, W.FINE_GRAINED, W.EXPERT_CHOICE):
        inp = W.make_inputs(W.Workload(**{**w.__dict__, "T": 64}), experts=False)
        assert inp["x"].shape == (64, w.d)
        assert inp["Wg"].shape == (w.d, w.E)
        if w.dtype == "bf16":
            assert np.array_equal(W.round_bf16(inp["x"]), inp["x"])
    assert W.EXPERT_CHOICE.capacity == 512
    assert W.MIXTRAL_LAYER.rows == 32768
    assert sorted(W.WORKLOADS) == sorted(w.name for w in (W.TINY_FP32, W.MID_BF16, W.MIXTRAL_LAYER,
                                                          W.FINE_GRAINED, W.EXPERT_CHOICE))


def test_stds_roughly_right():
    w = W.custom(T=4096, d=64, f=64, E=4, x_std=0.5, wg_std=0.1, w_std=0.02, dtype="fp32")
    inp = W.make_inputs(w)
    assert abs(inp["x"].std() - 0.5) < 0.01
    assert abs(inp["Wgate"].std() - 0.02) < 0.001
