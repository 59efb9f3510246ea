"""moe_forward under HIP graph capture: the library's launches are plain kernels on the
caller's stream (zeroing is a kernel, never hipMemsetAsync), so a captured layer call can
be replayed. The graph is replayed several times with eager work in between (new x
values written in place), and every replay must equal an eager call on the same x bit
for bit."""
from __future__ import annotations

import sys

import pytest
import torch

import workloads as W
from tests import parity as PR

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import sparse_mixture_experts_sum_amd as M
    M.load_library()
    return M


@pytest.mark.parametrize("mode", ["tc", "tc_capacity", "ec"])
def test_graph_replays_match_eager(moe, mode):
    w = W.custom(f"graph_{mode}", T=1000, d=256, f=256, E=8, k=2 if mode != "ec" else 1,
                 mode=mode, cf=1.0, bias_std=0.5, seed=(42, 400))
    print("[case]", w, flush=True)
    sys.stdout.flush()
    inp = W.make_inputs(w)
    dev = PR.device_inputs(inp, w)
    kw = dict(k=w.k, mode=mode, capacity_factor=w.cf, want_stats=mode != "ec",
              want_z_loss=True)
    x = dev["x"].clone()
    names = ["y", "idx", "w", "probs", "counts", "z_loss"] + (["f", "p", "loss"] if mode != "ec" else [])
    # warm up on a side stream, as graph capture requires, then capture one layer call
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ws = moe.moe_forward(x, dev["Wg"], dev["b"], dev["Wgate"], dev["Wup"], dev["Wdown"],
                             **kw)["workspace"]
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = moe.moe_forward(x, dev["Wg"], dev["b"], dev["Wgate"], dev["Wup"], dev["Wdown"],
                              workspace=ws, **kw)
    gen = torch.Generator(device="cuda").manual_seed(5)
    for rep in range(3):
        # eager work between replays: new token values, written in place
        x.copy_((torch.randn(x.shape, device="cuda", generator=gen) * w.x_std).to(x.dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = moe.moe_forward(x, dev["Wg"], dev["b"], dev["Wgate"], dev["Wup"], dev["Wdown"],
                              **kw)
        torch.cuda.synchronize()
        for n in names:
            assert torch.equal(cap[n], ref[n]), (rep, n)
