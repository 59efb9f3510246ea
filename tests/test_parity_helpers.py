"""The test-side helper that evaluates the layer with its hidden activation rounded once to
bf16 (parity.mix_hidden_bf16), against the oracle's exact mix."""
import numpy as np

import workloads as W
from oracle import moe_oracle as O
from tests import parity as PR


def test_hidden_bf16_mix_is_the_exact_mix_within_one_bf16_rounding_of_h():
    w = W.custom("hid", dtype="bf16", T=300, d=64, f=128, E=5, k=2, seed=(42, 5))
    inp = W.make_inputs(w)
    idx, wts, _, _ = O.route_tc(inp["x"], inp["Wg"], inp["b"], w.k, True)
    y = O.mix(inp["x"], idx, wts, inp["Wgate"], inp["Wup"], inp["Wdown"])
    yh = PR.mix_hidden_bf16(inp["x"], idx, wts, inp["Wgate"], inp["Wup"], inp["Wdown"])
    # elementwise bound: round to nearest moves each h by at most 2^-9 of its magnitude
    x = inp["x"].astype(np.float64)
    bound = np.zeros_like(y)
    for t in range(w.T):
        for j in range(w.k):
            e = idx[t, j]
            h = O.silu(x[t] @ inp["Wgate"][e]) * (x[t] @ inp["Wup"][e])
            bound[t] += abs(wts[t, j]) * (np.abs(h) @ np.abs(inp["Wdown"][e].astype(np.float64)))
    assert np.all(np.abs(yh - y) <= 2.0 ** -9 * bound + 1e-15)
    assert np.max(np.abs(yh - y)) > 0  # the rounding is there


def test_hidden_bf16_mix_rounds_to_nearest_even():
    # one token, one expert, d_model = d_ff = 1: silu(64) is 64 in fp64 and 64 * (2^-6 + 2^-14)
    # = 1 + 2^-8, exactly halfway between the bf16 neighbours 1 and 1 + 2^-7, so round to
    # nearest even gives 1: y = W_down * 1
    Wgate = np.full((1, 1, 1), 64.0, np.float32)
    Wup = np.full((1, 1, 1), 2.0 ** -6 + 2.0 ** -14, np.float32)
    Wdown = np.full((1, 1, 3), 2.0, np.float32)
    x = np.ones((1, 1), np.float32)
    assert O.silu(64.0) * float(Wup[0, 0, 0]) == 1 + 2.0 ** -8
    yh = PR.mix_hidden_bf16(x, np.zeros((1, 1), int), np.ones((1, 1)), Wgate, Wup, Wdown)
    assert np.array_equal(yh, np.full((1, 3), 2.0))
    # one ulp of h above halfway rounds up
    Wup[0, 0, 0] = np.float32(2.0 ** -6 + 2.0 ** -14 + 2.0 ** -20)
    yh = PR.mix_hidden_bf16(x, np.zeros((1, 1), int), np.ones((1, 1)), Wgate, Wup, Wdown)
    assert np.array_equal(yh, np.full((1, 3), 2.0 * (1 + 2.0 ** -7)))
