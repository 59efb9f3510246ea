"""GPU parity of token choice with an expert capacity (机器学习基础系列——混合专家模型,
expert_capacity_routing) against the fp64 oracle, through the C ABI.

Routing rules are those of the plain token-choice tests (near-tie tokens may take the
device's experts); given the device's top-k, which assignments survive the capacity
is integer work and must match the oracle bit for bit, as must the dispatch tables.
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


@pytest.fixture(scope="module")
def moe():
    import sparse_mixture_experts_sum_amd as M
    M.load_library()
    return M


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _np(t):
    return None if t is None else t.detach().cpu().numpy()


def _ws_i32(M, out, which, n):
    off = M.workspace_offset(out["shape"], which)
    return _np(out["workspace"][off:off + 4 * n].view(torch.int32))


def run_capacity_case(M, w: W.Workload, cf: float, inp=None, sample=None, hidden_fallback=False):
    """Returns (device outputs, kept mask the oracle derives from the device's top-k).
    hidden_fallback: see parity.check_y."""
    _say(w, "cf", cf)
    if inp is None:
        inp = W.make_inputs(w)
    dev = PR.device_inputs(inp, w)
    out = M.moe_forward(dev["x"], dev["Wg"], dev["b"], dev["Wgate"], dev["Wup"], dev["Wdown"],
                        k=w.k, mode="tc_capacity", capacity_factor=cf,
                        renormalize=w.renormalize)
    torch.cuda.synchronize()
    T, E, k = w.T, w.E, w.k
    cap = O.tc_capacity(T, E, k, cf)
    assert M.capacity(out["shape"]) == cap
    idx, wd, probs, counts = (_np(out[n]) for n in ("idx", "w", "probs", "counts"))
    idx_ref, w_ref, kept_ref, p_ref, s_ref, load_ref = O.route_tc_capacity(
        inp["x"], inp["Wg"], inp["b"], k, cf, w.renormalize)
    np.testing.assert_allclose(probs, p_ref, rtol=0, atol=1e-5 if w.dtype == "bf16" else 1e-6)
    exempt = PR.check_tc_routing(idx, None, p_ref, k, w.renormalize)
    PR.check_counts(counts, idx, idx_ref, exempt, E)  # counts are taken before any drop
    idx64 = idx.astype(np.int64)

    # which assignments stay: exact, given the device's experts
    kept, load = O.capacity_keep(idx64, E, cap)
    pos = _ws_i32(M, out, M.WS_POS, T * k).reshape(T, k)
    assert np.array_equal(pos >= 0, kept), f"kept slots differ on {np.sum((pos >= 0) != kept)}"
    if not exempt.any():
        assert np.array_equal(load, load_ref)

    # dispatch tables: groups sized min(count, cap), rows a bijection onto kept slots
    offsets = _ws_i32(M, out, M.WS_OFFSETS, E + 1)
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), load)
    R = int(offsets[E])
    assert R == int(np.minimum(O.expert_counts(idx64, E), cap).sum())
    src = _ws_i32(M, out, M.WS_SRC, max(R, 1))[:R]
    rows = pos[kept]
    assert np.array_equal(np.sort(rows), np.arange(R)), "kept rows are not a bijection onto [0, R)"
    tt = np.nonzero(kept)[0]
    assert np.array_equal(src[rows], tt)
    ee = idx64[kept]
    assert np.all((rows >= offsets[ee]) & (rows < offsets[ee + 1])), "row outside its expert group"
    # stable: inside a group rows follow token order
    for e in range(E):
        ts = src[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(ts) > 0)

    # weights after the capacity
    w_use = O.capacity_weights(p_ref, idx64, kept, w.renormalize)
    werr = float(np.max(np.abs(wd.astype(np.float64) - w_use))) if T else 0.0
    assert werr <= 1e-5, f"weights differ by {werr}"
    assert np.all(wd[~kept] == 0.0)

    # output: the oracle layer evaluated on the same routing
    toks = np.arange(T)
    if sample is not None and sample < T:
        toks = np.sort(np.random.default_rng(7).choice(T, size=sample, replace=False))
    y_ref = O.mix(inp["x"][toks], idx64[toks], w_use[toks], inp["Wgate"], inp["Wup"], inp["Wdown"])
    y = _np(out["y"])
    hid = (lambda: PR.mix_hidden_bf16(inp["x"][toks], idx64[toks], w_use[toks], inp["Wgate"],
                                      inp["Wup"], inp["Wdown"])) if hidden_fallback else None
    err = PR.check_y(y[toks], y_ref, w.dtype, hidden_ref=hid) if T else 0.0
    if not exempt.any() and sample is None and 0 < T <= 4096:
        ref = O.forward_tc_capacity(inp["x"], inp["Wg"], inp["b"], inp["Wgate"], inp["Wup"],
                                    inp["Wdown"], k, cf, w.renormalize)
        PR.check_y(y, ref["y"], w.dtype, hidden_ref=hid)
    # statistics before any drop
    f_ref, pm_ref, loss_ref, _ = O.aux_stats(p_ref, idx64, E, k)
    np.testing.assert_allclose(_np(out["f"]), f_ref, rtol=1e-6, atol=0)
    np.testing.assert_allclose(_np(out["p"]), pm_ref, rtol=1e-5, atol=1e-7)
    np.testing.assert_allclose(_np(out["loss"])[0], loss_ref, rtol=1e-5)
    _say(f"  ok: cap {cap}, dropped {int((~kept).sum())} of {T * k}, y err {err:.3e}, "
         f"exempt {int(exempt.sum())}")
    return out, kept


def test_capacity_mid_bf16_heavy_drops(moe):
    # skewed router bias: most tokens want the same two experts
    w = W.custom("cap_mid_skewed", T=2048, d=512, f=1024, E=8, k=2, bias_std=1.0, seed=(42, 101))
    out, kept = run_capacity_case(moe, w, 1.0)
    assert (~kept).sum() > 0.1 * w.T * w.k


def test_capacity_fp32_ragged_no_renormalisation(moe):
    w = W.custom("cap_fp32_ragged", dtype="fp32", T=1000, d=128, f=256, E=8, k=2,
                 renormalize=False, x_std=0.5, wg_std=0.1, bias_std=0.5, seed=(42, 102))
    run_capacity_case(moe, w, 0.75)


@pytest.mark.parametrize("T", [1, 63, 257])
def test_capacity_small_and_ragged(moe, T):
    w = W.custom(f"cap_ragged_{T}", T=T, d=128, f=192, E=4, k=2, bias_std=0.5, seed=(42, 110 + T))
    run_capacity_case(moe, w, 1.25)


def test_capacity_factor_not_exact_in_binary(moe):
    # cf = 0.9: the capacity int((T / E) * cf * k) is taken in double on both sides (180
    # here); the groups and drops follow it exactly
    w = W.custom("cap_cf09", T=1000, d=128, f=128, E=10, k=2, bias_std=0.7, seed=(42, 610))
    assert O.tc_capacity(1000, 10, 2, 0.9) == 180
    run_capacity_case(moe, w, 0.9)


def test_capacity_two_kernel_dispatch(moe):
    # 625 router blocks: the capacity is applied by the dispatch scan and the permute kernel
    # (the path past the fused dispatch's 512 blocks). 50025 of 80000 slots dropped, 15951
    # tokens lose both; h rounded to bf16 alone puts this case at 0.0162 of the output RMS
    # (the zeros of fully dropped tokens lower the RMS: with cf 0.8, d = d_ff = 64 that
    # rounding alone exceeds the 2e-2 bar)
    w = W.custom("cap_T40000", T=40000, d=128, f=256, E=16, k=2, bias_std=0.5, seed=(42, 611))
    run_capacity_case(moe, w, 1.0)


def test_capacity_fine_grained_top4(moe):
    w = W.custom("cap_e64_top4", T=1024, d=256, f=192, E=64, k=4, bias_std=0.3, seed=(42, 103))
    run_capacity_case(moe, w, 1.0)


def test_capacity_max_k_64_experts(moe):
    # k = 8 of 64 experts with a tight capacity: every token loses some slots
    w = W.custom("cap_k8_e64", T=600, d=128, f=128, E=64, k=8, bias_std=1.0, seed=(42, 107))
    out, kept = run_capacity_case(moe, w, 0.5)
    assert (~kept).any(axis=1).mean() > 0.2


def test_capacity_that_drops_nothing_is_plain_token_choice(moe):
    # cf = E / k gives C = T: no expert can overflow, so the layer is plain token choice
    w = W.custom("cap_none_dropped", T=512, d=256, f=256, E=8, k=2, bias_std=1.0, seed=(42, 104))
    out, kept = run_capacity_case(moe, w, w.E / w.k)
    assert kept.all()
    dev = PR.device_inputs(W.make_inputs(w), w)
    plain = moe.moe_forward(dev["x"], dev["Wg"], dev["b"], dev["Wgate"], dev["Wup"], dev["Wdown"],
                            k=w.k)
    torch.cuda.synchronize()
    for n in ("y", "idx", "w", "counts", "f", "p", "loss"):
        assert torch.equal(out[n], plain[n]), n


def test_zero_capacity_drops_everything(moe):
    # T / E * cf * k < 1: C = 0, every assignment dropped, y = 0, statistics unchanged
    w = W.custom("cap_zero", T=7, d=64, f=64, E=8, k=1, seed=(42, 105))
    out, kept = run_capacity_case(moe, w, 1.0)
    assert not kept.any()
    assert torch.count_nonzero(out["y"]).item() == 0
    assert torch.count_nonzero(out["w"]).item() == 0


def test_route_only_matches_forward(moe):
    w = W.custom("cap_route", T=777, d=256, f=128, E=8, k=2, bias_std=1.0, seed=(42, 106))
    dev = PR.device_inputs(W.make_inputs(w), w)
    _say(w)
    r = moe.moe_route(dev["x"], dev["Wg"], dev["b"], k=w.k, mode="tc_capacity",
                      capacity_factor=0.5)
    f = moe.moe_forward(dev["x"], dev["Wg"], dev["b"], dev["Wgate"], dev["Wup"], dev["Wdown"],
                        k=w.k, mode="tc_capacity", capacity_factor=0.5)
    torch.cuda.synchronize()
    for n in ("idx", "w", "probs", "counts"):
        assert torch.equal(r[n], f[n]), n
    assert torch.count_nonzero(r["w"] == 0).item() > 0


def test_capacity_mixtral_layer_full(moe):
    # the full Mixtral-shaped layer with a skewed router, capacity factor 1: every output
    # against the oracle evaluated on the same routing
    w = W.MIXTRAL_LAYER
    run_capacity_case(moe, w, 1.0)
