"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Every case is seeded and synthetic (workloads/), printed before it runs.
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


def run_tc_case(M, w: W.Workload, inp=None, check_stats=True, sample=None, hidden_fallback=False):
    """Run the token-choice layer on the device and check it against the oracle.

    sample: if given, the number of tokens whose output the oracle evaluates
    (routing is still checked on every token). hidden_fallback: see parity.check_y."""
    _say(w)
    if inp is None:
        inp = W.make_inputs(w)
    dev = PR.device_inputs(inp, w)
    out = M.moe_forward(dev["x"], dev["Wg"], dev["b"], dev["Wgate"], dev["Wup"], dev["Wdown"],
                        k=w.k, renormalize=w.renormalize)
    torch.cuda.synchronize()
    idx, wd, probs, counts = (_np(out[k]) for k in ("idx", "w", "probs", "counts"))
    y = _np(out["y"])
    idx_ref, w_ref, p_ref, s_ref = O.route_tc(inp["x"], inp["Wg"], inp["b"], w.k, w.renormalize)
    np.testing.assert_allclose(probs, p_ref, rtol=0, atol=1e-5 if w.dtype == "bf16" else 1e-6)
    exempt = PR.check_tc_routing(idx, wd, p_ref, w.k, w.renormalize)
    PR.check_counts(counts, idx, idx_ref, exempt, w.E)
    # reference routing: the oracle's, except near-tie tokens take the device's experts
    idx_use = idx_ref.copy()
    idx_use[exempt] = idx[exempt]
    w_use = O.gate_weights(p_ref, idx_use, w.renormalize)
    toks = np.arange(w.T)
    if sample is not None and sample < w.T:
        toks = np.sort(np.random.default_rng(7).choice(w.T, size=sample, replace=False))
    y_ref = O.mix(inp["x"][toks], idx_use[toks], w_use[toks], inp["Wgate"], inp["Wup"], inp["Wdown"])
    hid = (lambda: PR.mix_hidden_bf16(inp["x"][toks], idx_use[toks], w_use[toks], inp["Wgate"],
                                      inp["Wup"], inp["Wdown"])) if hidden_fallback else None
    err = PR.check_y(y[toks], y_ref, w.dtype, hidden_ref=hid)
    if check_stats:
        f_ref, pm_ref, loss_ref, c_ref = O.aux_stats(p_ref, idx_use, w.E, w.k)
        rt = 1e-5
        np.testing.assert_allclose(_np(out["f"]), f_ref, rtol=1e-6, atol=0)
        np.testing.assert_allclose(_np(out["p"]), pm_ref, rtol=rt, atol=1e-7)
        np.testing.assert_allclose(_np(out["loss"])[0], loss_ref, rtol=rt)
    _say(f"  ok: y err {err:.3e}, exempt tokens {int(exempt.sum())}")
    return out, inp


def run_ec_case(M, w: W.Workload, inp=None):
    _say(w)
    if inp is None:
        inp = W.make_inputs(w)
    dev = PR.device_inputs(inp, w)
    out = M.moe_forward(dev["x"], dev["Wg"], dev["b"], dev["Wgate"], dev["Wup"], dev["Wdown"],
                        mode="ec", capacity_factor=w.cf, want_stats=False)
    torch.cuda.synchronize()
    ref = O.forward_ec(inp["x"], inp["Wg"], inp["b"], inp["Wgate"], inp["Wup"], inp["Wdown"], w.cf)
    C = w.capacity
    margin = PR.check_ec_routing(_np(out["idx"]), _np(out["w"]), ref, C)
    assert np.all(_np(out["counts"]) == C)
    np.testing.assert_allclose(_np(out["probs"]), ref["probs"], rtol=1e-4, atol=1e-9)
    if np.all(margin > PR.MARGIN):
        y_ref = ref["y"]
    else:  # near-tie boundary: evaluate the oracle with the device's choice
        y_ref = O.mix_ec(inp["x"], _np(out["idx"]).astype(np.int64),
                         np.take_along_axis(ref["probs"].T, _np(out["idx"]).astype(np.int64), 1),
                         inp["Wgate"], inp["Wup"], inp["Wdown"])
    err = PR.check_y(_np(out["y"]), y_ref, w.dtype)
    _say(f"  ok: y err {err:.3e}")
    return out, inp


# ---------------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------------

def test_tiny_top2_fp32(moe):
    run_tc_case(moe, W.TINY_FP32)


def test_mid_top2_bf16(moe):
    run_tc_case(moe, W.MID_BF16)


def test_fine_grained_e64_top4(moe):
    run_tc_case(moe, W.FINE_GRAINED)


def test_expert_choice_e16(moe):
    run_ec_case(moe, W.EXPERT_CHOICE)


# ---------------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1, 63, 65, 257, 1000])
def test_ragged_tokens_bf16(moe, T):
    run_tc_case(moe, W.custom(f"ragged_T{T}", T=T, d=128, f=192, E=6, k=2, seed=(42, 100 + T)))


def test_fp32_general(moe):
    run_tc_case(moe, W.custom("fp32_k3", dtype="fp32", T=300, d=128, f=256, E=6, k=3,
                              x_std=0.5, wg_std=0.1, seed=(42, 201)))


def test_all_tokens_one_expert_and_empty_experts(moe):
    w = W.custom("collapsed", T=500, d=128, f=128, E=8, k=1, seed=(42, 202))
    inp = W.make_inputs(w)
    inp["b"] = np.zeros(8, dtype=np.float32)
    inp["b"][3] = 50.0
    out, _ = run_tc_case(moe, w, inp=inp)
    assert _np(out["counts"]).tolist() == [0, 0, 0, 500, 0, 0, 0, 0]


def test_single_expert(moe):
    run_tc_case(moe, W.custom("E1k1", T=200, d=64, f=128, E=1, k=1, seed=(42, 203)))


def test_k_equals_E_without_renormalisation_is_dense(moe):
    w = W.custom("dense", T=128, d=64, f=64, E=4, k=4, renormalize=False, wg_std=0.5,
                 seed=(42, 204))
    out, inp = run_tc_case(moe, w)
    y_dense = O.dense_mixture(inp["x"], inp["Wg"], inp["b"], inp["Wgate"], inp["Wup"], inp["Wdown"])
    PR.check_y(_np(out["y"]), y_dense, "bf16", "dense mixture")


def test_max_k_and_E(moe):
    run_tc_case(moe, W.custom("E64k8", T=333, d=128, f=128, E=64, k=8, wg_std=0.2, seed=(42, 205)))


@pytest.mark.parametrize("E,k,d", [(24, 3, 512), (40, 5, 2048)])
def test_router_expert_counts_with_partial_column_blocks(moe, E, k, d):
    # bf16 router with E a multiple of 8 but not of 16: W_g is staged as it lies and the
    # last 16-column block of the MFMA holds padding columns (E = 40: d = 2048 needs two
    # LDS slices of the [k, E] rows)
    run_tc_case(moe, W.custom(f"E{E}k{k}", T=300, d=d, f=128, E=E, k=k, wg_std=0.05,
                              seed=(42, 220 + E)))


def test_zero_input_uniform_routing(moe):
    w = W.custom("zeros", T=70, d=64, f=64, E=8, k=3, seed=(42, 206))
    inp = W.make_inputs(w)
    inp["x"] = np.zeros_like(inp["x"])
    out, _ = run_tc_case(moe, w, inp=inp)
    assert np.all(_np(out["idx"]) == np.array([0, 1, 2]))
    assert np.all(_np(out["y"]) == 0.0)
    assert abs(float(_np(out["loss"])[0]) - 1.0) < 1e-6


def test_empty_batch(moe):
    _say("T=0")
    x = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    Wg = torch.zeros(64, 4, dtype=torch.bfloat16, device="cuda")
    Wgu = torch.zeros(4, 64, 64, dtype=torch.bfloat16, device="cuda")
    out = moe.moe_forward(x, Wg, None, Wgu, Wgu.clone(), Wgu.clone(), k=2)
    torch.cuda.synchronize()
    assert out["y"].shape == (0, 64)
    assert _np(out["counts"]).tolist() == [0, 0, 0, 0]
    assert float(_np(out["loss"])[0]) == 0.0


@pytest.mark.parametrize("T,E,cf", [(1024, 8, 1.0), (1000, 8, 1.25), (96, 1, 1.0), (512, 16, 0.5),
                                    (1000, 10, 0.7)])
def test_expert_choice_shapes(moe, T, E, cf):
    run_ec_case(moe, W.custom(f"ec_T{T}_E{E}_cf{cf}", T=T, d=128, f=128, E=E, mode="ec", cf=cf,
                              k=1, seed=(42, 300 + T + E)))


@pytest.mark.parametrize("d,f", [(64, 128), (192, 320)])
def test_expert_choice_narrow_tiles_bf16(moe, d, f):
    # d_model 64 / 192: the down projection's 256 x 64 column tiles, which also
    # pair each row of h with its residual row (C = 175: a partial second tile of 47
    # tokens per expert); d_ff 320 takes the 256 x 128 gate/up tiles
    run_ec_case(moe, W.custom(f"ec_d{d}_f{f}", T=700, d=d, f=f, E=6, mode="ec", cf=1.5, k=1,
                              bias_std=0.5, seed=(42, 320 + d)))


def test_expert_choice_long_k_bf16(moe):
    # d_ff 8192: 256 K stages per down tile, the length from which a token-choice layer
    # splits its last round of tiles along K; the paired expert-choice tiles stay whole
    # (the workspace holds no stream-K slots for them)
    w = W.custom("ec_f8192", T=640, d=256, f=8192, E=4, mode="ec", cf=1.0, k=1, bias_std=0.5,
                 seed=(42, 350))
    out, _ = run_ec_case(moe, w)
    R, d = w.E * w.capacity, w.d
    shape = out["shape"]
    assert moe.workspace_size(shape) - moe.workspace_offset(shape, moe.WS_O) < R * d * 4 + 4096


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_expert_choice_more_experts_than_row_chunks(moe, dtype):
    # d_model 64: a token's output row is 16 chunks of 4 floats, so the combine's lanes 16
    # and up hold no chunk, while expert e's row and score sit in lane e (E = 40): every
    # expert's rows must still reach y
    run_ec_case(moe, W.custom(f"ec_E40_d64_{dtype}", dtype=dtype, T=900, d=64, f=128, E=40,
                              mode="ec", cf=1.0, k=1, bias_std=0.5, seed=(42, 360)))


def test_expert_choice_fp32_bias_ragged(moe):
    run_ec_case(moe, W.custom("ec_fp32", dtype="fp32", T=333, d=128, f=192, E=5, mode="ec",
                              cf=2.0, k=1, x_std=0.5, wg_std=0.2, bias_std=1.0, seed=(42, 330)))


@pytest.mark.parametrize("T", [12000, 20000, 40000])
def test_expert_choice_long_column(moe, T):
    # the select kernel holds up to 8 logits per thread in registers (T <= 8192, the other
    # tests), up to 16 (T = 12000), stages columns of up to 32768 in LDS (T = 20000), and
    # reads longer ones from HBM in every pass (T = 40000)
    run_ec_case(moe, W.custom(f"ec_T{T}", T=T, d=64, f=64, E=4, mode="ec", cf=1.0, k=1,
                              bias_std=0.3, seed=(42, 340 if T == 40000 else 341 + T % 7)))


def test_expert_choice_boundary_ties_in_one_value_bucket(moe):
    # 2000 tokens repeating 50 rows: every logit value occurs 40 times, and each expert's
    # 250th largest logit sits inside such a group of 40 equal keys (the 50 distinct values are
    # 2.3e-3 or more apart, so fp32 and fp64 order them alike). The select's value bucket holds
    # the group; the lowest 10 token indices of it must be taken, exactly as the oracle's
    # stable order takes them, and every list must match the oracle's.
    w = W.custom("ec_ties", T=2000, d=128, f=128, E=8, k=1, mode="ec", cf=1.0, wg_std=0.3,
                 seed=(42, 713))
    inp = W.make_inputs(w)
    inp["x"][:] = inp["x"][np.arange(w.T) % 50]
    out, _ = run_ec_case(moe, w, inp=inp)
    ref = O.forward_ec(inp["x"], inp["Wg"], inp["b"], inp["Wgate"], inp["Wup"], inp["Wdown"], w.cf)
    assert np.array_equal(_np(out["idx"]), ref["idx"])


def test_dispatch_17_experts(moe):
    # just past 16 experts: the 1024-thread dispatch blocks (every expert's counts in one
    # round), 32 padded experts in the router
    run_tc_case(moe, W.custom("dispatch_E17", T=3000, d=128, f=128, E=17, k=2, wg_std=0.3,
                              bias_std=0.5, seed=(42, 343)))


def test_dispatch_scan_many_blocks(moe):
    # 313 router blocks x 64 experts = 20032 count entries, summed by every block of the
    # fused dispatch kernel
    run_tc_case(moe, W.custom("scan_T20000_E64", T=20000, d=64, f=64, E=64, k=2, wg_std=0.3,
                              seed=(42, 341)))


def test_dispatch_two_kernel_path(moe):
    # 625 router blocks (more than the fused dispatch takes): the dispatch scan, with more
    # than 16 count entries per scan thread (it re-reads them), then the permute kernel
    # (d_model 256, d_ff 512: h rounded to bf16 alone puts this case at 0.011 of the output
    # RMS; at d = d_ff = 64 that rounding alone reaches the 2e-2 bar over 2.56 M outputs)
    run_tc_case(moe, W.custom("scan_T40000_E16", T=40000, d=256, f=512, E=16, k=3, wg_std=0.3,
                              bias_std=0.5, seed=(42, 342)))


@pytest.mark.parametrize("T,d,f,E,k", [(300, 256, 8192, 2, 2), (1500, 512, 8192, 4, 2),
                                       (700, 256, 16384, 3, 1), (5000, 256, 8192, 8, 2)])
def test_stream_k_down_projection(moe, T, d, f, E, k):
    # down projections over d_ff >= 8192 (256 K stages or more): the last round's tiles are
    # split along K over every workgroup of an XCD (T=300: a tile in up to 32 pieces; T=5000:
    # several whole rounds first), and the owner adds the pieces' partial sums to its own in
    # a fixed order; outputs against the oracle, and a second call bitwise equal to the first
    w = W.custom(f"sk_T{T}_d{d}_f{f}", T=T, d=d, f=f, E=E, k=k, bias_std=0.3, seed=(42, 700 + T))
    out, inp = run_tc_case(moe, w)
    dev = PR.device_inputs(inp, w)
    again = moe.moe_forward(dev["x"], dev["Wg"], dev["b"], dev["Wgate"], dev["Wup"], dev["Wdown"],
                            k=k)
    torch.cuda.synchronize()
    assert torch.equal(out["y"], again["y"])


def test_determinism_bitwise(moe):
    w = W.custom("det", T=777, d=256, f=256, E=8, k=2, seed=(42, 207))
    inp = W.make_inputs(w)
    dev = PR.device_inputs(inp, w)
    outs = [moe.moe_forward(dev["x"], dev["Wg"], dev["b"], dev["Wgate"], dev["Wup"], dev["Wdown"], k=2)
            for _ in range(2)]
    torch.cuda.synchronize()
    for key in ("y", "idx", "w", "probs", "counts", "f", "p", "loss"):
        assert torch.equal(outs[0][key], outs[1][key]), key


def test_standalone_aux_loss_matches_fused(moe):
    w = W.custom("aux", T=1500, d=128, f=64, E=16, k=4, seed=(42, 208))
    inp = W.make_inputs(w)
    dev = PR.device_inputs(inp, w)
    fw = moe.moe_forward(dev["x"], dev["Wg"], dev["b"], dev["Wgate"], dev["Wup"], dev["Wdown"], k=4)
    aux = moe.moe_aux_loss(fw["probs"], fw["idx"])
    torch.cuda.synchronize()
    for key in ("f", "p", "loss", "counts"):
        assert torch.equal(aux[key], fw[key]), key
    f_ref, p_ref, loss_ref, c_ref = O.aux_stats(_np(fw["probs"]), _np(fw["idx"]), 16, 4)
    assert _np(aux["counts"]).tolist() == c_ref.tolist()
    np.testing.assert_allclose(_np(aux["loss"])[0], loss_ref, rtol=1e-6)


def test_route_only_matches_forward(moe):
    w = W.custom("route", T=640, d=192, f=64, E=12, k=3, bias_std=1.0, seed=(42, 209))
    inp = W.make_inputs(w)
    dev = PR.device_inputs(inp, w)
    r = moe.moe_route(dev["x"], dev["Wg"], dev["b"], k=3)
    fw = moe.moe_forward(dev["x"], dev["Wg"], dev["b"], dev["Wgate"], dev["Wup"], dev["Wdown"], k=3)
    torch.cuda.synchronize()
    for key in ("idx", "w", "probs", "counts"):
        assert torch.equal(r[key], fw[key]), key


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_dispatch_permutation_is_stable_bijection(moe, dtype):
    w = W.custom(f"perm_{dtype}", dtype=dtype, T=900, d=64, f=64, E=5, k=3, seed=(42, 210))
    inp = W.make_inputs(w)
    dev = PR.device_inputs(inp, w)
    out = moe.moe_forward(dev["x"], dev["Wg"], dev["b"], dev["Wgate"], dev["Wup"], dev["Wdown"], k=3)
    torch.cuda.synchronize()
    ws, shape = out["workspace"], out["shape"]
    R = w.T * w.k

    def grab(which, n, dt):
        off = moe.workspace_offset(shape, which)
        nbytes = n * torch.empty(0, dtype=dt).element_size()
        return ws[off: off + nbytes].view(dt).cpu()

    pos = grab(moe.WS_POS, R, torch.int32).numpy().reshape(w.T, w.k)
    src = grab(moe.WS_SRC, R, torch.int32).numpy()
    offs = grab(moe.WS_OFFSETS, w.E + 1, torch.int32).numpy()
    idx = _np(out["idx"])
    assert np.array_equal(np.sort(pos.ravel()), np.arange(R))            # bijection
    assert np.array_equal(src[pos], np.repeat(np.arange(w.T)[:, None], w.k, 1))
    for e in range(w.E):                                                # grouped + stable
        rows = np.arange(offs[e], offs[e + 1])
        flat = [(t * w.k + j) for t in range(w.T) for j in range(w.k) if idx[t, j] == e]
        assert np.array_equal(pos.ravel()[flat], rows)
    if dtype == "fp32":  # rows copied by the permute
        xperm = grab(moe.WS_XPERM, R * w.d, torch.float32).view(R, w.d)
        assert torch.equal(xperm, dev["x"].cpu()[torch.from_numpy(src).long()])
    else:  # bf16: the gate/up GEMM gathers x[src] itself; there is no copy
        with pytest.raises(moe.MoEError):
            moe.workspace_offset(shape, moe.WS_XPERM)


@pytest.mark.parametrize("mode", ["tc", "tc_capacity", "ec"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_optional_outputs_do_not_change_y(moe, mode, dtype):
    # routing, probabilities and statistics not requested (NULL pointers through the C ABI:
    # the library keeps idx and w in its workspace instead): the same y, bit for bit
    w = W.custom(f"optional_{mode}_{dtype}", dtype=dtype, T=777, d=128, f=192, E=12, k=3 if
                 mode != "ec" else 1, bias_std=0.5, seed=(42, 370))
    inp = W.make_inputs(w)
    dev = PR.device_inputs(inp, w)
    args = (dev["x"], dev["Wg"], dev["b"], dev["Wgate"], dev["Wup"], dev["Wdown"])
    kw = dict(k=w.k, mode=mode, capacity_factor=1.25)
    _say(w, mode, "all outputs, then y alone")
    full = moe.moe_forward(*args, want_stats=mode != "ec", want_z_loss=True, **kw)
    bare = moe.moe_forward(*args, want_routing=False, want_probs=False, want_stats=False, **kw)
    torch.cuda.synchronize()
    assert bare["idx"] is None and bare["probs"] is None
    assert torch.equal(full["y"], bare["y"])


def test_layer_module_batch_seq_input(moe):
    # the layer object on [batch, seq, d_model] input: the same bits as moe_forward on the
    # flattened tokens, for three calls of different token counts sharing its workspace
    w = W.custom("module", T=4 * 75, d=128, f=128, E=8, k=2, seed=(42, 230))
    inp = W.make_inputs(w)
    dev = PR.device_inputs(inp, w)
    layer = moe.SparseMoE(dev["Wg"], dev["Wgate"], dev["Wup"], dev["Wdown"], dev["b"], k=2)
    for B, S in ((4, 75), (2, 33), (4, 75)):
        x = dev["x"][: B * S].reshape(B, S, w.d)
        y = layer(x)
        ref = moe.moe_forward(dev["x"][: B * S], dev["Wg"], dev["b"], dev["Wgate"], dev["Wup"],
                              dev["Wdown"], k=2)
        torch.cuda.synchronize()
        assert y.shape == (B, S, w.d)
        assert torch.equal(y.reshape(B * S, w.d), ref["y"])
        assert torch.equal(layer.last["idx"], ref["idx"])
        assert torch.equal(layer.last["loss"], ref["loss"])


# the full-size case runs last: it is the slowest
def test_mixtral_layer_skewed_full(moe):
    """Full-size Mixtral layer with a skewed router bias: routing, counts, statistics
    and the output y on every token (all 16384 x 4096 outputs against the fp64 oracle)."""
    w = W.MIXTRAL_LAYER
    out, inp = run_tc_case(moe, w)
    counts = _np(out["counts"])
    assert counts.sum() == w.T * w.k
    assert counts.max() > 1.3 * counts.mean()  # the bias skews the load
    # dispatch invariants on the full size
    ws = out["workspace"]
    shape = out["shape"]
    off = moe.workspace_offset(shape, moe.WS_OFFSETS)
    offsets = ws[off: off + 4 * (w.E + 1)].view(torch.int32).cpu().numpy()
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
