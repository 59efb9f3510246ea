"""GPU parity over a seeded sweep of small random layer shapes (every routing mode and both
dtypes), against the fp64 oracle: the fixed cases elsewhere pin the five workloads and chosen
edge cases, this sweep covers combinations nobody picked (odd token counts, expert counts that
are not powers of two, d_model / d_ff at every multiple of 64 up to 512 / 1024, bias on or off).

The case list is drawn once from a fixed seed, so every run checks the same cases. Token-choice
outputs in bf16 are held to the 2e-2 bar, or, where a single bf16 rounding of the hidden
activation alone misses it (long-tailed outputs at small d_model), to within 10% of that
rounding's own error (parity.check_y).
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
        run_tc_case(moe, w, hidden_fallback=True)
    elif c["mode"] == "capacity":
        run_capacity_case(moe, w, c["cf"], hidden_fallback=True)
    else:
        run_ec_case(moe, w)


# ---- a second sweep: training noise, routing-only calls and larger layers ------------------

def _cases2(n: int = 24, seed: int = 2027):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = ("noisy", "route", "big")[i % 3]
        dtype = "fp32" if rng.random() < 0.3 else "bf16"
        E = int(rng.integers(2, 65))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.integers(64, 3000))
        d = 64 * int(rng.integers(1, 17))
        f = 64 * int(rng.integers(1, 33))
        mode = ("tc", "tc", "capacity", "ec")[int(rng.integers(0, 4))]
        while T * k * d * f > 2e9:  # keep the fp64 oracle to about a second
            T = max(64, T // 2)
            f = max(64, f // 128 * 64)  # halved, still a multiple of 64
        c = dict(i=100 + i, kind=kind, mode=mode, dtype=dtype, T=T, d=d, f=f, E=E, k=k,
                 bias=0.5 if rng.random() < 0.5 else None, cf=float(np.round(rng.uniform(0.5, 2.0), 3)),
                 wn=bool(rng.random() < 0.5), draw=bool(rng.random() < 0.5))
        if kind == "noisy" and mode == "ec":
            c["mode"] = "tc"  # noise is a token-choice feature
        if c["mode"] == "ec":
            c["k"] = 1
            c["cf"] = max(c["cf"], float(np.ceil(E / T * 1000) / 1000))
        out.append(c)
    return out


CASES2 = _cases2()


def _route_case(M, w, c):
    """moe_route alone: routing, probabilities, statistics and z-loss against the oracle."""
    from tests.test_gpu_parity import _np, _say
    import torch
    from oracle import moe_oracle as O
    from tests import parity as PR
    _say(w, "route only", c["mode"])
    inp = W.make_inputs(w, experts=False)
    dev = PR.device_inputs(inp, w)
    mode = {"tc": "tc", "capacity": "tc_capacity", "ec": "ec"}[c["mode"]]
    out = M.moe_route(dev["x"], dev["Wg"], dev["b"], k=w.k, mode=mode, capacity_factor=c["cf"],
                      renormalize=w.renormalize, want_z_loss=True)
    torch.cuda.synchronize()
    z_ref = O.router_z_loss(O.router_logits(inp["x"], inp["Wg"], inp["b"]))
    assert abs(float(_np(out["z_loss"])[0]) - z_ref) <= 1e-5 * abs(z_ref)
    if mode == "ec":
        idx_r, score_r, S_r, s_r = O.route_ec(inp["x"], inp["Wg"], inp["b"], c["cf"])
        ref = {"idx": idx_r, "w": score_r, "probs": S_r, "logits": s_r}
        PR.check_ec_routing(_np(out["idx"]), _np(out["w"]), ref, w.capacity)
        assert np.all(_np(out["counts"]) == w.capacity)
        _say("  ok")
        return
    idx, probs = _np(out["idx"]), _np(out["probs"])
    _, _, p_ref, _ = O.route_tc(inp["x"], inp["Wg"], inp["b"], w.k, w.renormalize)
    np.testing.assert_allclose(probs, p_ref, rtol=0, atol=1e-5 if w.dtype == "bf16" else 1e-6)
    exempt = PR.check_tc_routing(idx, None if mode == "tc_capacity" else _np(out["w"]), p_ref,
                                 w.k, w.renormalize)
    # the statistics from the standalone entry point, on the device's own routing
    f_ref, pm_ref, loss_ref, c_ref = O.aux_stats(p_ref, idx.astype(np.int64), w.E, w.k)
    np.testing.assert_array_equal(_np(out["counts"]), c_ref)
    st = M.moe_aux_loss(out["probs"], out["idx"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(st["counts"]), c_ref)
    np.testing.assert_allclose(_np(st["f"]), f_ref, rtol=1e-6, atol=0)
    np.testing.assert_allclose(_np(st["p"]), pm_ref, rtol=1e-5, atol=1e-7)
    np.testing.assert_allclose(_np(st["loss"])[0], loss_ref, rtol=1e-5)
    _say(f"  ok: exempt tokens {int(exempt.sum())}")


@pytest.mark.parametrize("c", CASES2, ids=lambda c: f"{c['i']}-{c['kind']}-{c['mode']}-{c['dtype']}")
def test_random_shape_noise_route_big(moe, c):
    w = W.custom(f"sweep{c['i']}", dtype=c["dtype"], T=c["T"], d=c["d"], f=c["f"], E=c["E"],
                 k=c["k"], mode="ec" if c["mode"] == "ec" else "tc", cf=c["cf"],
                 bias_std=c["bias"], seed=(42, 900 + c["i"]))
    if c["kind"] == "noisy":
        from tests.test_gpu_noise import run_noisy_case
        nz = W.make_noise(w, wn_std=0.02 if c["wn"] else None, eps_scale=1.0)
        draw = (1000 + c["i"], 7 * c["i"], 1.0) if c["draw"] else None
        mode = "tc_capacity" if c["mode"] == "capacity" else "tc"
        run_noisy_case(moe, w, nz, mode=mode, cf=c["cf"], draw=draw, hidden_fallback=True)
    elif c["kind"] == "route":
        _route_case(moe, w, c)
    elif c["mode"] == "tc":
        run_tc_case(moe, w, hidden_fallback=True)
    elif c["mode"] == "capacity":
        run_capacity_case(moe, w, c["cf"], hidden_fallback=True)
    else:
        run_ec_case(moe, w)


# ---- a third sweep: token counts at the edges (a handful of tokens, block boundaries, and
# batches past the one-launch dispatch and the register-held expert-choice columns) ---------

def _cases3(n: int = 16, seed: int = 2028):
    rng = np.random.default_rng(seed)
    Ts = [1, 2, 3, 63, 64, 65, 127, 129, 16385, 20000, 32767, 32769, 40000, 47000, 5, 1000]
    out = []
    for i in range(n):
        T = Ts[i]
        mode = ("tc", "capacity", "ec", "tc")[i % 4]
        dtype = "fp32" if rng.random() < 0.25 else "bf16"
        E = int(rng.integers(1, 65))
        k = int(rng.integers(1, min(E, 8) + 1))
        cf = float(np.round(rng.uniform(0.3, 2.0), 3))
        if mode == "ec":
            k = 1
            cf = max(cf, float(np.ceil(E / T * 1000) / 1000))
            if np.floor(T * cf / E) > T:
                cf = float(E)
        out.append(dict(i=200 + i, mode=mode, dtype=dtype, T=T, d=64 * int(rng.integers(1, 3)),
                        f=64 * int(rng.integers(1, 3)), E=E, k=k, cf=cf,
                        bias=0.5 if rng.random() < 0.5 else None))
    return out


CASES3 = _cases3()


@pytest.mark.parametrize("c", CASES3, ids=lambda c: f"{c['i']}-T{c['T']}-{c['mode']}-{c['dtype']}")
def test_random_token_counts(moe, c):
    w = W.custom(f"sweep{c['i']}", dtype=c["dtype"], T=c["T"], d=c["d"], f=c["f"], E=c["E"],
                 k=c["k"], mode="ec" if c["mode"] == "ec" else "tc", cf=c["cf"],
                 bias_std=c["bias"], seed=(42, 900 + c["i"]))
    if c["mode"] == "tc":
        run_tc_case(moe, w, hidden_fallback=True)
    elif c["mode"] == "capacity":
        run_capacity_case(moe, w, c["cf"], hidden_fallback=True)
    else:
        run_ec_case(moe, w)


# ---- a fourth sweep: d_ff of 8192 and more, where the down projection splits the K range of
# its last partial round of tiles across workgroups (stream-K, partial sums in a fixed order)

def _cases4(n: int = 8, seed: int = 2029):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        f = 64 * int(rng.integers(128, 257))  # 8192 .. 16384
        d = 64 * int(rng.integers(1, 9))
        E = int(rng.integers(1, 17))
        k = int(rng.integers(1, min(E, 2) + 1))
        T = int(rng.integers(50, 4000))
        while T * k * d * f > 2e9:  # keep the fp64 oracle to about a second
            T = max(50, T // 2)
        out.append(dict(i=300 + i, T=T, d=d, f=f, E=E, k=k, cap=bool(rng.random() < 0.3),
                        cf=float(np.round(rng.uniform(0.5, 1.5), 3)),
                        bias=0.5 if rng.random() < 0.5 else None))
    return out


CASES4 = _cases4()


@pytest.mark.parametrize("c", CASES4, ids=lambda c: f"{c['i']}-f{c['f']}-{'cap' if c['cap'] else 'tc'}")
def test_random_stream_k_shapes(moe, c):
    w = W.custom(f"sweep{c['i']}", dtype="bf16", T=c["T"], d=c["d"], f=c["f"], E=c["E"], k=c["k"],
                 bias_std=c["bias"], seed=(42, 900 + c["i"]))
    if c["cap"]:
        run_capacity_case(moe, w, c["cf"], hidden_fallback=True)
    else:
        run_tc_case(moe, w, hidden_fallback=True)


# ---- the down projection's tile height ------------------------------------------------------
# The host runs the down projection in 192-row tiles when at most (R / 192 + E) row tiles times
# d_model / 256 column tiles fit one round of the 256 workgroups, and in 256-row tiles
# otherwise. The cases below sit on both sides of that rule, with groups skewed by a router
# bias so that some are empty or shorter than one tile and most end in a partial tile.

TILE_CASES = [
    # (T, d_model, d_ff, E, k, bias std): rows R = T k
    (3000, 256, 512, 8, 2, 2.0),    # 6000 rows: 39 + 8 row tiles of 192, one column tile
    (2500, 512, 384, 5, 2, 1.0),    # 5000 rows: (26 + 5) x 2 column tiles of 192 rows
    (4096, 768, 256, 8, 2, None),   # 8192 rows: (42 + 8) x 3 = 150 tiles of 192 rows
    (24000, 256, 512, 8, 2, 1.0),   # 48000 rows: 250 + 8 > 256: 256-row tiles
    (9000, 1024, 256, 8, 2, 0.5),   # 18000 rows: (93 + 8) x 4 > 256: 256-row tiles
]


@pytest.mark.parametrize("c", TILE_CASES, ids=lambda c: f"T{c[0]}-d{c[1]}-E{c[3]}")
def test_down_projection_tile_height(moe, c):
    T, d, f, E, k, bias = c
    w = W.custom(f"tiles-T{T}-d{d}", dtype="bf16", T=T, d=d, f=f, E=E, k=k, bias_std=bias,
                 seed=(42, 700 + T % 97))
    run_tc_case(moe, w, hidden_fallback=True)


# ---- the expert-choice combine by token blocks ----------------------------------------------
# From d_model 512 on, the expert-choice combine takes 16 consecutive tokens per workgroup and
# finds each expert's run of them in its token list; the cases cover a partial last block, a
# single block, experts whose lists skip a block entirely, many experts, and (d_model 256) the
# per-token kernel below that width.

EC_BLOCK_CASES = [
    # (T, d_model, d_ff, E, capacity factor, bias std)
    (1000, 768, 256, 12, 1.3, None),   # 63 blocks, the last one of 8 tokens
    (17, 512, 128, 3, 2.0, None),      # one full block and one of a single token
    (2048, 512, 192, 64, 0.5, 1.0),    # 64 experts of 16 tokens: most blocks absent from a list
    (777, 1024, 128, 5, 4.0, 0.5),     # C = 621 of 777 tokens: most tokens in several lists
    (300, 256, 128, 6, 1.0, None),     # d_model 256: one wave per token
]


@pytest.mark.parametrize("c", EC_BLOCK_CASES, ids=lambda c: f"T{c[0]}-d{c[1]}-E{c[3]}")
def test_expert_choice_combine_blocks(moe, c):
    T, d, f, E, cf, bias = c
    w = W.custom(f"ecblk-T{T}-d{d}", dtype="bf16", T=T, d=d, f=f, E=E, k=1, mode="ec", cf=cf,
                 bias_std=bias, seed=(42, 800 + T % 89))
    run_ec_case(moe, w)


# ---- repeated calls and a reused workspace on the two paths above ---------------------------
# A second call gives the same bits, and a call that reuses the workspace of a larger call
# (whose run table, rows and tiles are still there) gives the bits of a call with a fresh one.

def _layer(moe, dev, w, **kw):
    return moe.moe_forward(dev["x"], dev["Wg"], dev["b"], dev["Wgate"], dev["Wup"], dev["Wdown"],
                           **kw)


@pytest.mark.parametrize("mode", ["ec", "tc"])
def test_block_combine_and_192_tiles_repeat_and_reuse_workspace(moe, mode):
    import torch
    from tests import parity as PR
    kw = dict(mode="ec", capacity_factor=1.3, want_stats=False) if mode == "ec" else dict(k=2)
    big = W.custom(f"reuse-big-{mode}", dtype="bf16", T=1000, d=768, f=256, E=12,
                   k=1 if mode == "ec" else 2, mode=mode, cf=1.3, seed=(42, 611))
    small = W.custom(f"reuse-small-{mode}", dtype="bf16", T=333, d=768, f=256, E=12,
                     k=1 if mode == "ec" else 2, mode=mode, cf=1.3, bias_std=0.7, seed=(42, 612))
    dev_b = PR.device_inputs(W.make_inputs(big), big)
    dev_s = PR.device_inputs(W.make_inputs(small), small)
    first = _layer(moe, dev_b, big, **kw)
    again = _layer(moe, dev_b, big, workspace=first["workspace"], **kw)
    fresh = _layer(moe, dev_s, small, **kw)
    reused = _layer(moe, dev_s, small, workspace=first["workspace"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(first["y"], again["y"])
    assert torch.equal(fresh["y"], reused["y"])
    assert torch.equal(fresh["idx"], reused["idx"])


# ---- two row groups in the down projection's columns order ---------------------------------
# With 16 or more output column tiles (d_model >= 4096) and weights smaller than four times
# the rows (E * d_model < 4 * rows), the down projection's XCDs split a group's row tiles in
# two and its columns in four. Cases: 256-row tiles, 192-row tiles (one round), and 256-row
# tiles whose last round is split along K (d_ff 8192: stream-K).

ROW_GROUP_CASES = [
    # (T, d_model, d_ff, E, k, bias std)
    (1500, 4096, 256, 2, 2, 0.5),    # 3000 rows: 17 x 16 tiles of 256 rows
    (2400, 4096, 256, 2, 1, None),   # 2400 rows: 14 x 16 tiles of 192 rows, one round
    (1500, 4096, 8192, 2, 2, 0.5),   # stream-K in the last round
]


@pytest.mark.parametrize("c", ROW_GROUP_CASES, ids=lambda c: f"T{c[0]}-f{c[2]}-k{c[4]}")
def test_down_projection_two_row_groups(moe, c):
    T, d, f, E, k, bias = c
    w = W.custom(f"rowgroups-T{T}-f{f}", dtype="bf16", T=T, d=d, f=f, E=E, k=k, bias_std=bias,
                 seed=(42, 650 + T % 83))
    run_tc_case(moe, w, hidden_fallback=True)


# Groups whose rows run just past a whole number of 256-row tiles (the last row tile holds 1,
# 64 or 65 rows). With E = 2 and k = 2 every token goes to both experts, so each group has
# exactly T rows. Cases: gate/up and the 192-row down projection of small layers, the down
# projection in 256-row tiles (d_model 4096) with and without stream-K, and a skewed
# 16-expert mix.
BOUNDARY_CASES = [
    # (T, d_model, d_ff, E, k, bias std)
    (257, 256, 512, 2, 2, None),
    (320, 1024, 512, 2, 2, None),
    (321, 1024, 512, 2, 2, None),
    (576, 512, 1024, 2, 2, None),
    (1537, 4096, 256, 2, 2, None),
    (1600, 4096, 256, 2, 2, None),
    (1600, 4096, 8192, 2, 2, None),
    (3000, 1024, 1408, 16, 2, 0.3),
]


@pytest.mark.parametrize("c", BOUNDARY_CASES, ids=lambda c: f"T{c[0]}-d{c[1]}-f{c[2]}-E{c[3]}")
def test_groups_just_past_a_tile_boundary(moe, c):
    T, d, f, E, k, bias = c
    w = W.custom(f"boundary-T{T}-d{d}-f{f}-E{E}", dtype="bf16", T=T, d=d, f=f, E=E, k=k,
                 bias_std=bias, seed=(42, 700 + T % 97))
    run_tc_case(moe, w, hidden_fallback=True)
