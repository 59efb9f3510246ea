"""The allocation-free entry point (moe_forward_noalloc, workspace in the library's fixed
device array) against moe_forward with a caller workspace, through the C ABI: the same
kernels, so every output must be bitwise equal, and y must meet the oracle's bar. Four
calls in a row on one GPU, each smaller than the one before (the array keeps the previous
call's intermediates, which must not leak into the next), then a shape too large for the
array, which is refused before anything is launched."""
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


def _compare(M, w):
    _say("noalloc", w)
    inp = W.make_inputs(w)
    dev = PR.device_inputs(inp, w)
    kw = dict(k=w.k, mode=w.mode, capacity_factor=w.cf, renormalize=w.renormalize,
              want_stats=w.mode != "ec", want_z_loss=True)
    shape = M.make_shape(w.T, w.d, w.f, w.E, w.k, w.mode, w.dtype, w.renormalize, w.cf)
    assert M.workspace_size(shape) <= M.NOALLOC_SCRATCH_BYTES
    a = M.moe_forward_noalloc(dev["x"], dev["Wg"], dev["b"], dev["Wgate"], dev["Wup"],
                              dev["Wdown"], **kw)
    b = M.moe_forward(dev["x"], dev["Wg"], dev["b"], dev["Wgate"], dev["Wup"], dev["Wdown"], **kw)
    torch.cuda.synchronize()
    for key in ("y", "idx", "w", "probs", "counts", "f", "p", "loss", "z_loss"):
        if b[key] is None:
            assert a[key] is None, key
            continue
        assert torch.equal(a[key], b[key]), key
    if w.mode == "ec":
        ref = O.forward_ec(inp["x"], inp["Wg"], inp["b"], inp["Wgate"], inp["Wup"], inp["Wdown"],
                           w.cf)
        idx_use = _np(a["idx"]).astype(np.int64)
        y_ref = O.mix_ec(inp["x"], idx_use, np.take_along_axis(ref["probs"].T, idx_use, 1),
                         inp["Wgate"], inp["Wup"], inp["Wdown"])
    else:
        idx_ref, w_ref, p_ref, _ = O.route_tc(inp["x"], inp["Wg"], inp["b"], w.k, w.renormalize)
        exempt = PR.check_tc_routing(_np(a["idx"]), _np(a["w"]), p_ref, w.k, w.renormalize)
        idx_use = idx_ref.copy()
        idx_use[exempt] = _np(a["idx"])[exempt]
        y_ref = O.mix(inp["x"], idx_use, O.gate_weights(p_ref, idx_use, w.renormalize),
                      inp["Wgate"], inp["Wup"], inp["Wdown"])
    err = PR.check_y(_np(a["y"]), y_ref, w.dtype)
    _say(f"  ok: bitwise equal to moe_forward, y err {err:.3e}")


def test_noalloc_calls_shrinking(moe):
    # four calls, each smaller than the one before: the 16-expert expert-choice layer (its
    # workspace 0.20 GB of the 0.27 GB array), the mid-size layer, a small token-choice one and
    # an fp32 expert-choice one
    _compare(moe, W.EXPERT_CHOICE)
    _compare(moe, W.MID_BF16)
    _compare(moe, W.custom("noalloc_small", T=1000, d=256, f=512, E=8, k=2, bias_std=0.5,
                           seed=(42, 620)))
    _compare(moe, W.custom("noalloc_ec_fp32", dtype="fp32", T=300, d=128, f=192, E=6, mode="ec",
                           cf=1.5, k=1, x_std=0.5, wg_std=0.2, seed=(42, 621)))


def test_noalloc_refuses_a_layer_larger_than_its_array(moe):
    # the Mixtral-size layer needs 1.5 GB of workspace: refused on the host (status 4,
    # MOE_ERR_WORKSPACE_TOO_SMALL), before any launch
    T, d, f, E = 16384, 4096, 14336, 8
    assert moe.workspace_size(moe.make_shape(T, d, f, E, 2)) > moe.NOALLOC_SCRATCH_BYTES
    dev = torch.device("cuda")
    x = torch.empty(T, d, dtype=torch.bfloat16, device=dev)
    Wg = torch.empty(d, E, dtype=torch.bfloat16, device=dev)
    Wgu = torch.empty(E, d, f, dtype=torch.bfloat16, device=dev)
    Wd = torch.empty(E, f, d, dtype=torch.bfloat16, device=dev)
    _say("noalloc refusal", (T, d, f, E))
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_forward_noalloc(x, Wg, None, Wgu, Wgu, Wd, k=2)
    assert ei.value.status == 4
