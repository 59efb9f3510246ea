"""GPU parity of the router z-loss (the Korean page's router_z_loss: mean over tokens
of the squared log-partition of the router logits) against the fp64 oracle, through
the C ABI, in every routing mode.

The device computes each token's log-partition in fp32 from fp32 logits; the oracle
in fp64 from exact logits. Tolerance: relative 1e-5 (fp32 logits over d <= 4096 bf16
products carry a relative error of order 1e-6).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle import moe_oracle as O
from tests import parity as PR

pytestmark = pytest.mark.gpu

RTOL = 1e-5


@pytest.fixture(scope="module")
def moe():
    import sparse_mixture_experts_sum_amd as M
    M.load_library()
    return M


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _z_ref(inp):
    return O.router_z_loss(O.router_logits(inp["x"], inp["Wg"], inp["b"]))


def _mode_kw(w):
    return dict(k=w.k, mode=w.mode, capacity_factor=w.cf, renormalize=w.renormalize)


def run_z_case(M, w, route_only=False):
    _say(w)
    inp = W.make_inputs(w, experts=not route_only)
    dev = PR.device_inputs(inp, w)
    if route_only:
        out = M.moe_route(dev["x"], dev["Wg"], dev["b"], want_z_loss=True, **_mode_kw(w))
    else:
        out = M.moe_forward(dev["x"], dev["Wg"], dev["b"], dev["Wgate"], dev["Wup"], dev["Wdown"],
                            want_z_loss=True, want_stats=w.mode != "ec", **_mode_kw(w))
    torch.cuda.synchronize()
    z = float(out["z_loss"].cpu()[0])
    ref = _z_ref(inp)
    assert abs(z - ref) <= RTOL * abs(ref), f"z-loss {z} vs oracle {ref}"
    _say(f"  ok: z {z:.7g} oracle {ref:.7g}")
    return out, dev


def test_zloss_token_choice_mid(moe):
    run_z_case(moe, W.MID_BF16)


def test_zloss_mixtral_skewed_full_size(moe):
    # all 16384 tokens of the Mixtral-shaped layer, router bias N(0, 1)
    run_z_case(moe, W.MIXTRAL_LAYER, route_only=True)


def test_zloss_fine_grained_e64(moe):
    run_z_case(moe, W.FINE_GRAINED, route_only=True)


def test_zloss_expert_choice(moe):
    run_z_case(moe, W.EXPERT_CHOICE)


def test_zloss_with_capacity(moe):
    run_z_case(moe, W.custom("z_capacity", T=1000, d=256, f=128, E=8, k=2, mode="tc_capacity",
                             cf=0.5, bias_std=1.0, seed=(42, 201)))


@pytest.mark.parametrize("T", [1, 63, 65, 1000])
def test_zloss_ragged_fp32(moe, T):
    run_z_case(moe, W.custom(f"z_fp32_{T}", dtype="fp32", T=T, d=128, f=64, E=6, k=2,
                             x_std=0.5, wg_std=0.3, seed=(42, 210 + T)), route_only=True)


def test_zloss_large_logits(moe):
    # biases of tens: exp of an unshifted logit would overflow fp32
    run_z_case(moe, W.custom("z_large", dtype="fp32", T=300, d=64, f=64, E=16, k=2,
                             bias_std=60.0, seed=(42, 220)), route_only=True)


def test_zloss_40_experts_statistics_rounds(moe):
    # 40 experts: the dispatch's 1024-thread statistics block takes the 41 items (40 experts
    # and the z-loss) in two rounds of 32, the z-loss item in the second
    run_z_case(moe, W.custom("z_e40", T=1500, d=256, f=128, E=40, k=3, bias_std=0.5,
                             seed=(42, 231)))


def test_zloss_changes_nothing_else(moe):
    # the same call with and without the z-loss: every other output bitwise equal,
    # and the router-only z-loss equals the layer's
    w = W.custom("z_bitwise", T=777, d=256, f=128, E=8, k=2, bias_std=0.5, seed=(42, 230))
    out, dev = run_z_case(moe, w)
    plain = moe.moe_forward(dev["x"], dev["Wg"], dev["b"], dev["Wgate"], dev["Wup"], dev["Wdown"],
                            k=w.k)
    r = moe.moe_route(dev["x"], dev["Wg"], dev["b"], k=w.k, want_z_loss=True)
    torch.cuda.synchronize()
    for n in ("y", "idx", "w", "probs", "counts", "f", "p", "loss"):
        assert torch.equal(out[n], plain[n]), n
    assert torch.equal(r["z_loss"], out["z_loss"])


def test_zloss_empty_batch(moe):
    x = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    Wg = torch.zeros(64, 8, dtype=torch.bfloat16, device="cuda")
    r = moe.moe_route(x, Wg, None, k=2, want_z_loss=True)
    torch.cuda.synchronize()
    assert float(r["z_loss"].cpu()[0]) == 0.0
