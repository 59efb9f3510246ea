"""GPU parity at element offsets past 2^31: a bf16 token-choice layer whose input x holds
more than 2^31 elements (T * d_model >= 2^31).

There the rows are no longer gathered from x inside the gate/up GEMM (its per-lane row
offsets are 32-bit): the permute copies them into the workspace's x_perm and the GEMM
reads contiguous rows, so this case is the one that runs that path of the 256 x 256
pipelined kernel, with x_perm offsets near 2^33 elements.

Input: x repeats a seeded block of P = 4099 rows (P prime, so no power-of-two row
shift maps a row onto an equal one). Token t's routing and output are those of block
row t mod P, which the oracle evaluates once for the block: routing, weights and
probabilities are checked on every token, counts and statistics over all tokens, the
output on a sample (including tokens past the 2^31-element boundary and the last
token), and on the device every output row against its block row's.
"""
from __future__ import annotations

import sys
from dataclasses import replace

import numpy as np
import pytest
import torch

import workloads as W
from oracle import moe_oracle as O
from tests import parity as PR

pytestmark = pytest.mark.gpu

P = 4099


@pytest.fixture(scope="module")
def moe():
    import sparse_mixture_experts_sum_amd as M
    M.load_library()
    return M


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def test_bf16_input_past_2_31_elements(moe):
    # T * d = 2^31 + 1000 * 8192 elements; T % 64 = 40 (a ragged router block)
    w = W.custom("large_x_bf16", dtype="bf16", T=(1 << 18) + 1000, d=8192, f=128, E=8, k=2,
                 x_std=1.0, wg_std=0.02, w_std=0.02, seed=(42, 401))
    assert w.T * w.d >= 1 << 31
    _say(w, "x repeats", P, "seeded rows")
    blk = W.make_inputs(replace(w, T=P))  # the block's rows and the layer's weights
    dev = PR.device_inputs(blk, w)
    reps = -(-w.T // P)
    x = dev["x"].repeat(reps, 1)[: w.T].contiguous()
    torch.cuda.synchronize()
    out = moe.moe_forward(x, dev["Wg"], None, dev["Wgate"], dev["Wup"], dev["Wdown"], k=w.k,
                          renormalize=w.renormalize)
    torch.cuda.synchronize()
    _say("  forward done")
    # this shape takes the copying path
    assert moe.workspace_offset(out["shape"], moe.WS_XPERM) > 0

    tok = np.arange(w.T)
    src = tok % P
    idx_b, _, p_b, _ = O.route_tc(blk["x"], blk["Wg"], None, w.k, w.renormalize)
    p_ref = p_b[src]
    idx = out["idx"].cpu().numpy()
    probs = out["probs"].cpu().numpy()
    np.testing.assert_allclose(probs, p_ref, rtol=0, atol=1e-5)
    exempt = PR.check_tc_routing(idx, out["w"].cpu().numpy(), p_ref, w.k, w.renormalize)
    PR.check_counts(out["counts"].cpu().numpy(), idx, idx_b[src], exempt, w.E)
    idx_use = idx_b[src].copy()
    idx_use[exempt] = idx[exempt]
    w_use = O.gate_weights(p_ref, idx_use, w.renormalize)
    f_ref, pm_ref, loss_ref, _ = O.aux_stats(p_ref, idx_use, w.E, w.k)
    np.testing.assert_allclose(out["f"].cpu().numpy(), f_ref, rtol=1e-6, atol=0)
    np.testing.assert_allclose(out["p"].cpu().numpy(), pm_ref, rtol=1e-4, atol=1e-7)
    np.testing.assert_allclose(out["loss"].cpu().numpy()[0], loss_ref, rtol=1e-4)

    # outputs: a sample, with tokens on both sides of the 2^31-element boundary
    edge = (1 << 31) // w.d
    rng = np.random.default_rng(11)
    toks = np.unique(np.concatenate([rng.choice(w.T, size=40, replace=False),
                                     np.arange(edge - 4, edge + 4), [0, w.T - 1]]))
    y = out["y"]
    y_ref = O.mix(blk["x"][src[toks]], idx_use[toks], w_use[toks], blk["Wgate"], blk["Wup"],
                  blk["Wdown"])
    err = PR.check_y(y[torch.from_numpy(toks).to(y.device)].cpu().numpy(), y_ref, w.dtype)
    # every output row against its block row's (rows read from the wrong place would
    # differ by about the output's size)
    rms = y[:P].float().pow(2).mean().sqrt().item()
    worst = 0.0
    for s in range(P, w.T, P):
        n = min(P, w.T - s)
        worst = max(worst, (y[s: s + n] - y[:n]).abs().max().item())
    assert worst <= 1e-4 * rms, f"rows differ from their block rows by {worst / rms:.3e} rms"
    _say(f"  ok: y err {err:.3e}, periodic deviation {worst / rms:.3e} rms, "
         f"exempt tokens {int(exempt.sum())}")
