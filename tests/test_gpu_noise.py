"""GPU parity of noisy top-k gating (the Korean page's TopKGating, training branch:
logits + softplus(x W_noise) * eps; additive eps for the fixed-scale form) against
the fp64 oracle, through the C ABI. The normal draw eps is either an input that both
sides read, or drawn by the router kernel from (seed, offset) while the oracle
evaluates the same counter-based definition (Philox4x32-10 and Box-Muller) in fp64;
routing follows the near-tie rules of the plain token-choice tests.
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


def _dev_noise(nz, w):
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return (PR.to_dev(nz["Wn"], dt) if nz["Wn"] is not None else None,
            PR.to_dev(nz["eps"], torch.float32))


def run_noisy_case(M, w, nz, sample=None, mode="tc", cf=1.0, draw=None, hidden_fallback=False):
    """nz: the noise inputs (W_noise, eps). draw = (seed, offset, scale): the router
    kernel draws eps instead, and the oracle takes its fp64 evaluation of the same
    definition (nz["eps"] is replaced). hidden_fallback: see parity.check_y."""
    _say(w, "noise", "softplus" if nz["Wn"] is not None else "additive", mode,
         "drawn in the kernel %r" % (draw,) if draw else "eps passed")
    inp = W.make_inputs(w)
    dev = PR.device_inputs(inp, w)
    Wn, eps = _dev_noise(nz, w)
    if draw is not None:
        seed, offset, scale = draw
        eps = M.NoiseDraw(seed, offset, scale)
        nz = dict(nz, eps=O.noise_draw(w.T, w.E, seed, offset, scale))
    out = M.moe_forward(dev["x"], dev["Wg"], dev["b"], dev["Wgate"], dev["Wup"], dev["Wdown"],
                        k=w.k, mode=mode, capacity_factor=cf, renormalize=w.renormalize,
                        want_z_loss=True, W_noise=Wn, eps=eps)
    torch.cuda.synchronize()
    idx, wd, probs, counts = (_np(out[n]) for n in ("idx", "w", "probs", "counts"))
    idx_ref, w_ref, p_ref, s_ref = O.route_tc_noisy(inp["x"], inp["Wg"], inp["b"], nz["Wn"],
                                                    nz["eps"], w.k, w.renormalize)
    np.testing.assert_allclose(probs, p_ref, rtol=0, atol=1e-5 if w.dtype == "bf16" else 1e-6)
    capacity = mode == "tc_capacity"
    exempt = PR.check_tc_routing(idx, None if capacity else wd, p_ref, w.k, w.renormalize)
    PR.check_counts(counts, idx, idx_ref, exempt, w.E)
    idx64 = idx.astype(np.int64)
    if capacity:
        kept, _ = O.capacity_keep(idx64, w.E, O.tc_capacity(w.T, w.E, w.k, cf))
        w_use = O.capacity_weights(p_ref, idx64, kept, w.renormalize)
        assert np.max(np.abs(wd - w_use)) <= 1e-5
    else:
        w_use = O.gate_weights(p_ref, idx64, w.renormalize)
    toks = np.arange(w.T)
    if sample is not None and sample < w.T:
        toks = np.sort(np.random.default_rng(7).choice(w.T, size=sample, replace=False))
    y_ref = O.mix(inp["x"][toks], idx64[toks], w_use[toks], inp["Wgate"], inp["Wup"], inp["Wdown"])
    hid = (lambda: PR.mix_hidden_bf16(inp["x"][toks], idx64[toks], w_use[toks], inp["Wgate"],
                                      inp["Wup"], inp["Wdown"])) if hidden_fallback else None
    err = PR.check_y(_np(out["y"])[toks], y_ref, w.dtype, hidden_ref=hid)
    f_ref, pm_ref, loss_ref, _ = O.aux_stats(p_ref, idx64, w.E, w.k)
    np.testing.assert_allclose(_np(out["f"]), f_ref, rtol=1e-6, atol=0)
    np.testing.assert_allclose(_np(out["p"]), pm_ref, rtol=1e-5, atol=1e-7)
    np.testing.assert_allclose(_np(out["loss"])[0], loss_ref, rtol=1e-5)
    z_ref = O.router_z_loss(s_ref)
    assert abs(float(_np(out["z_loss"])[0]) - z_ref) <= 1e-5 * abs(z_ref)
    # the noise must have moved some routing, or the case tests nothing
    plain = O.topk_experts(O.softmax_rows(O.router_logits(inp["x"], inp["Wg"], inp["b"])), w.k)
    moved = int(np.sum(np.any(np.sort(plain, 1) != np.sort(idx_ref, 1), axis=1)))
    assert moved > 0
    _say(f"  ok: y err {err:.3e}, tokens rerouted by the noise {moved}, exempt {int(exempt.sum())}")
    return out, inp, dev


def test_noisy_mid_bf16(moe):
    w = W.MID_BF16
    run_noisy_case(moe, w, W.make_noise(w, wn_std=0.05))


def test_noisy_fine_grained_e64_top4(moe):
    w = W.custom("noisy_e64_top4", T=2048, d=512, f=256, E=64, k=4, seed=(42, 301))
    run_noisy_case(moe, w, W.make_noise(w, wn_std=0.05))


def test_noisy_24_experts_two_slices(moe):
    # bf16, E = 24: W_g and W_noise staged as they lie, two LDS slices (d = 2048)
    w = W.custom("noisy_e24", T=333, d=2048, f=128, E=24, k=3, wg_std=0.05, seed=(42, 310))
    run_noisy_case(moe, w, W.make_noise(w, wn_std=0.05))


def test_additive_noise_fp32_ragged(moe):
    # the fixed-scale form: logits + noise_std * eps, noise_std = 0.1
    w = W.custom("additive_fp32", dtype="fp32", T=1000, d=128, f=64, E=8, k=2, x_std=0.5,
                 wg_std=0.1, renormalize=False, seed=(42, 302))
    run_noisy_case(moe, w, W.make_noise(w, wn_std=None, eps_scale=0.1))


@pytest.mark.parametrize("T", [1, 65])
def test_noisy_small_fp32(moe, T):
    w = W.custom(f"noisy_fp32_{T}", dtype="fp32", T=T, d=64, f=64, E=16, k=2, x_std=1.0,
                 wg_std=0.3, seed=(42, 303 + T))
    nz = W.make_noise(w, wn_std=0.3, eps_scale=3.0)
    if T == 1:  # one token: a large draw on an unselected expert with a large noise
        # scale softplus(x W_noise) moves it
        inp = W.make_inputs(w, experts=False)
        top = O.topk_experts(O.softmax_rows(O.router_logits(inp["x"], inp["Wg"], inp["b"])), 2)
        scale = (inp["x"].astype(np.float64) @ nz["Wn"].astype(np.float64))[0]
        scale[top[0]] = -np.inf
        nz["eps"][0, :] = 0.0
        nz["eps"][0, int(np.argmax(scale))] = 40.0
    run_noisy_case(moe, w, nz)


def test_noisy_with_capacity(moe):
    w = W.custom("noisy_capacity", T=1024, d=256, f=128, E=8, k=2, bias_std=0.5, seed=(42, 305))
    run_noisy_case(moe, w, W.make_noise(w, wn_std=0.05), mode="tc_capacity", cf=0.75)


def test_noisy_capacity_fp32_raw_gates(moe):
    # fp32, softplus noise, an expert capacity, and no renormalisation
    w = W.custom("noisy_cap_fp32", dtype="fp32", T=500, d=128, f=64, E=8, k=2, x_std=0.5,
                 wg_std=0.2, bias_std=0.5, renormalize=False, seed=(42, 309))
    run_noisy_case(moe, w, W.make_noise(w, wn_std=0.2), mode="tc_capacity", cf=0.6)


def test_noisy_mixtral_layer_full(moe):
    # every output of the full Mixtral-shaped layer with training noise
    w = W.MIXTRAL_LAYER
    run_noisy_case(moe, w, W.make_noise(w, wn_std=0.02))


def test_zero_draw_is_bitwise_plain_routing(moe):
    # eps = 0: softplus(x W_noise) * 0 adds exactly 0, so every output equals the
    # noiseless call bit for bit (the noise variant also stages its LDS slices
    # differently; the MFMA accumulation order over k is the same)
    w = W.custom("zero_draw", T=777, d=512, f=128, E=16, k=2, bias_std=0.5, seed=(42, 306))
    inp = W.make_inputs(w)
    dev = PR.device_inputs(inp, w)
    nz = W.make_noise(w, wn_std=0.05)
    nz["eps"][:] = 0.0
    Wn, eps = _dev_noise(nz, w)
    _say(w, "zero draw")
    a = moe.moe_forward(dev["x"], dev["Wg"], dev["b"], dev["Wgate"], dev["Wup"], dev["Wdown"],
                        k=2, want_z_loss=True, W_noise=Wn, eps=eps)
    b = moe.moe_forward(dev["x"], dev["Wg"], dev["b"], dev["Wgate"], dev["Wup"], dev["Wdown"],
                        k=2, want_z_loss=True)
    torch.cuda.synchronize()
    for n in ("y", "idx", "w", "probs", "counts", "f", "p", "loss", "z_loss"):
        assert torch.equal(a[n], b[n]), n


def test_route_only_matches_forward(moe):
    w = W.custom("noisy_route", T=500, d=256, f=128, E=8, k=2, seed=(42, 307))
    inp = W.make_inputs(w)
    dev = PR.device_inputs(inp, w)
    Wn, eps = _dev_noise(W.make_noise(w, wn_std=0.05), w)
    _say(w, "route vs forward")
    r = moe.moe_route(dev["x"], dev["Wg"], dev["b"], k=2, want_z_loss=True, W_noise=Wn, eps=eps)
    f = moe.moe_forward(dev["x"], dev["Wg"], dev["b"], dev["Wgate"], dev["Wup"], dev["Wdown"],
                        k=2, want_z_loss=True, W_noise=Wn, eps=eps)
    torch.cuda.synchronize()
    for n in ("idx", "w", "probs", "counts", "z_loss"):
        assert torch.equal(r[n], f[n]), n


def test_expert_choice_refuses_noise(moe):
    w = W.custom("noisy_ec", T=256, d=64, f=64, E=4, k=1, mode="ec", seed=(42, 308))
    inp = W.make_inputs(w, experts=False)
    dev = PR.device_inputs(inp, w)
    _, eps = _dev_noise(W.make_noise(w, wn_std=None), w)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_route(dev["x"], dev["Wg"], None, mode="ec", eps=eps)
    assert ei.value.status == 3


# ---------------------------------------------------------------------------------
# the training noise drawn in the router kernel (moe_noise with eps = NULL)
# ---------------------------------------------------------------------------------

@pytest.mark.parametrize("E", [6, 64])
def test_drawn_noise_seen_through_probs(moe, E):
    # W_g = 0, no bias, additive noise of scale 1: the logits are the draw itself, so the
    # probabilities show every element of the kernel's draw against the oracle's fp64
    # evaluation of the same (seed, offset; t, e) definition. T ragged, seed and offset
    # with high words set, E = 6 ends inside a group of four experts.
    T, d = 4097, 64
    seed, offset = (0xA5A5 << 32) | 0x1234, (7 << 32) | 99
    _say("drawn noise through probs", T, E, hex(seed), hex(offset))
    g = torch.Generator(device="cuda").manual_seed(11)
    x = torch.randn(T, d, device="cuda", generator=g).to(torch.bfloat16)
    Wg = torch.zeros(d, E, device="cuda", dtype=torch.bfloat16)
    r = moe.moe_route(x, Wg, None, k=2, eps=moe.NoiseDraw(seed, offset, 1.0))
    torch.cuda.synchronize()
    eps_ref = O.noise_draw(T, E, seed, offset)
    p_ref = O.softmax_rows(eps_ref)
    np.testing.assert_allclose(_np(r["probs"]), p_ref, rtol=0, atol=2e-6)
    exempt = PR.check_tc_routing(_np(r["idx"]), _np(r["w"]), p_ref, 2, True)
    assert exempt.sum() < T // 100
    # the logits' spread is that of N(0, 1) draws: the largest probability of a token
    # reaches well above uniform for most tokens
    assert np.median(p_ref.max(axis=1)) > 2.0 / E


def test_drawn_noise_matches_its_definition_to_fp32_rounding(moe):
    # The same setting as above, read back sharper: with W_g = 0 the logits are the draw, so
    # ln p_e differs from eps_e by one constant per token; what is left after removing it is
    # the draw's own error (plus about 2.4e-7 from the fp32 probabilities). Half of the u
    # values need 25 significant bits ((j + 1/2) / 2^24 with j >= 2^23) and are not fp32
    # numbers; computing ln u or the angle from such a rounded u is off by up to 7e-6 near
    # u = 1 on this draw, far outside the bound, which allows a few fp32 roundings of |eps|.
    T, d, E = 4097, 64, 64
    seed, offset = (0xA5A5 << 32) | 0x1234, (7 << 32) | 99
    _say("drawn noise against its definition", T, E)
    g = torch.Generator(device="cuda").manual_seed(11)
    x = torch.randn(T, d, device="cuda", generator=g).to(torch.bfloat16)
    Wg = torch.zeros(d, E, device="cuda", dtype=torch.bfloat16)
    r = moe.moe_route(x, Wg, None, k=2, eps=moe.NoiseDraw(seed, offset, 1.0))
    torch.cuda.synchronize()
    eps_ref = O.noise_draw(T, E, seed, offset)
    D = np.log(_np(r["probs"]).astype(np.float64)) - eps_ref
    D -= np.median(D, axis=1, keepdims=True)
    tol = 5e-7 + 2.0 ** -21 * np.abs(eps_ref)
    bad = np.abs(D) > tol
    assert not bad.any(), (f"{int(bad.sum())} draws off by up to {np.abs(D).max():.3g}; "
                           f"worst at {np.unravel_index(np.argmax(np.abs(D) / tol), D.shape)}")


def test_drawn_noise_mid_bf16(moe):
    w = W.MID_BF16
    run_noisy_case(moe, w, W.make_noise(w, wn_std=0.05), draw=(2024, 1, 1.0))


def test_drawn_noise_fine_grained_e64_top4(moe):
    w = W.custom("drawn_e64_top4", T=2048, d=512, f=256, E=64, k=4, seed=(42, 311))
    run_noisy_case(moe, w, W.make_noise(w, wn_std=0.05), draw=(99, 12345, 1.0))


def test_drawn_additive_noise_fp32_ragged(moe):
    # the fixed-scale form drawn in the kernel: logits + 0.1 * n(t, e)
    w = W.custom("drawn_additive_fp32", dtype="fp32", T=1000, d=128, f=64, E=8, k=2, x_std=0.5,
                 wg_std=0.1, renormalize=False, seed=(42, 312))
    run_noisy_case(moe, w, W.make_noise(w, wn_std=None), draw=(7, 0, 0.1))


def test_drawn_noise_with_capacity(moe):
    w = W.custom("drawn_capacity", T=1024, d=256, f=128, E=8, k=2, bias_std=0.5, seed=(42, 313))
    run_noisy_case(moe, w, W.make_noise(w, wn_std=0.05), mode="tc_capacity", cf=0.75,
                   draw=(5, 3, 1.0))


def test_drawn_noise_mixtral_layer_full(moe):
    # every output of the full Mixtral-shaped layer with the draw made in the router
    w = W.MIXTRAL_LAYER
    run_noisy_case(moe, w, W.make_noise(w, wn_std=0.02), draw=(0xC0FFEE, 42, 1.0))


def test_drawn_noise_is_deterministic_and_moves_with_offset(moe):
    w = W.custom("drawn_offsets", T=1500, d=256, f=128, E=16, k=2, seed=(42, 314))
    inp = W.make_inputs(w)
    dev = PR.device_inputs(inp, w)
    Wn, _ = _dev_noise(W.make_noise(w, wn_std=0.05), w)
    _say(w, "drawn noise: same (seed, offset) twice, then the next offset")
    run = lambda off: moe.moe_forward(dev["x"], dev["Wg"], dev["b"], dev["Wgate"], dev["Wup"],
                                      dev["Wdown"], k=2, want_z_loss=True, W_noise=Wn,
                                      eps=moe.NoiseDraw(31, off, 1.0))
    a, b, c = run(8), run(8), run(9)
    torch.cuda.synchronize()
    for n in ("y", "idx", "w", "probs", "counts", "f", "p", "loss", "z_loss"):
        assert torch.equal(a[n], b[n]), n
    moved = int(torch.any(torch.sort(a["idx"], 1)[0] != torch.sort(c["idx"], 1)[0], 1).sum())
    assert moved > 0
