"""GPU parity over a seeded sweep of small random layer shapes (every routing mode and both
dtypes), against the fp64 oracle: the fixed cases elsewhere pin the five workloads and chosen
edge cases, this sweep covers combinations nobody picked (odd token counts, expert counts that
are not powers of two, d_model / d_ff at every multiple of 64 up to 512 / 1024, bias on or off).

The case list is drawn once from a fixed seed, so every run checks the same cases.
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from tests.test_gpu_capacity import run_capacity_case
from tests.test_gpu_parity import moe, run_ec_case, run_tc_case  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu


def _cases(n: int = 24, seed: int = 2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        mode = ("tc", "tc", "capacity", "ec")[i % 4]
        dtype = "fp32" if rng.random() < 0.3 else "bf16"
        T = int(rng.integers(1, 2500))
        d = 64 * int(rng.integers(1, 9))
        f = 64 * int(rng.integers(1, 17))
        E = int(rng.integers(1, 65))
        k = int(rng.integers(1, min(E, 8) + 1))
        bias = 0.5 if rng.random() < 0.5 else None
        cf = float(np.round(rng.uniform(0.3, 2.0), 3))
        if mode == "ec":
            k = 1
            cf = max(cf, float(np.ceil(E / T * 1000) / 1000))  # at least one token per expert
            if np.floor(T * cf / E) > T:
                cf = float(E)
        out.append(dict(i=i, mode=mode, dtype=dtype, T=T, d=d, f=f, E=E, k=k, bias=bias, cf=cf))
    return out


CASES = _cases()


@pytest.mark.parametrize("c", CASES, ids=lambda c: f"{c['i']:02d}-{c['mode']}-{c['dtype']}")
def test_random_shape(moe, c):
    w = W.custom(f"sweep{c['i']}", dtype=c["dtype"], T=c["T"], d=c["d"], f=c["f"], E=c["E"],
                 k=c["k"], mode="ec" if c["mode"] == "ec" else "tc", cf=c["cf"],
                 bias_std=c["bias"], seed=(42, 900 + c["i"]))
    if c["mode"] == "tc":
        run_tc_case(moe, w)
    elif c["mode"] == "capacity":
        run_capacity_case(moe, w, c["cf"])
    else:
        run_ec_case(moe, w)
