"""Pins for the fp64 oracle: checks against facts the pages or mathematics fix.

Each pin takes the oracle module ``O`` (``oracle.moe_oracle`` or a mutated copy
of it) and raises ``AssertionError`` when the oracle disagrees with the fact.
``tests/test_oracle_pins.py`` runs every pin on the real oracle;
``tests/test_oracle_mutants.py`` plants plausible mistakes in a copy of the
oracle and checks that some pin fails for each.

None of these pins retypes the oracle's own formula: each compares it with a
different computation (brute force over subsets, a library routine, a dense
formula with no selection, a closed form, an invariant).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

from oracle import brute as B

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _case(seed, T=6, d=5, f=7, E=4, bias=False, x_std=1.0, wg_std=0.7, w_std=0.5):
    r = _rng(seed)
    return dict(
        x=r.standard_normal((T, d)) * x_std,
        Wg=r.standard_normal((d, E)) * wg_std,
        b=(r.standard_normal(E) if bias else None),
        Wgate=r.standard_normal((E, d, f)) * w_std,
        Wup=r.standard_normal((E, d, f)) * w_std,
        Wdown=r.standard_normal((E, f, d)) * w_std,
    )


def _lists(a):
    return None if a is None else np.asarray(a).tolist()


# ----------------------------------------------------------------------------
# softmax
# ----------------------------------------------------------------------------

def pin_softmax_uniform(O):
    """W_g = 0: every expert gets probability exactly 1/E (E a power of two)."""
    for E in (2, 4, 8, 64):
        x = _rng(1).standard_normal((5, 3))
        p = O.softmax_rows(O.router_logits(x, np.zeros((3, E))))
        assert np.array_equal(p, np.full((5, E), 1.0 / E)), p


def pin_softmax_library(O):
    """Row softmax equals torch.softmax in float64, and a common shift of all
    logits (a bias c * 1) leaves it unchanged."""
    s = _rng(2).standard_normal((9, 6)) * 4
    ref = torch.softmax(torch.from_numpy(s), dim=1).numpy()
    assert np.allclose(O.softmax_rows(s), ref, rtol=1e-13, atol=1e-15)
    x = _rng(3).standard_normal((9, 4))
    Wg = _rng(4).standard_normal((4, 6))
    p0 = O.softmax_rows(O.router_logits(x, Wg))
    p1 = O.softmax_rows(O.router_logits(x, Wg, np.full(6, 3.25)))
    assert np.allclose(p0, p1, rtol=1e-13, atol=1e-15)
    # a non-constant bias must change the probabilities the way exp(b) scales them
    b = np.array([0.0, math.log(2.0), 0.0, 0.0, 0.0, 0.0])
    p2 = O.softmax_rows(O.router_logits(x, Wg, b))
    ratio = (p2[:, 1] / p2[:, 0]) / (p0[:, 1] / p0[:, 0])
    assert np.allclose(ratio, 2.0, rtol=1e-12)


def pin_colsoftmax_library(O):
    """Expert-choice column softmax equals torch.softmax over the token axis."""
    s = _rng(5).standard_normal((11, 4)) * 3
    ref = torch.softmax(torch.from_numpy(s), dim=0).numpy()
    S = O.softmax_cols(s)
    assert np.allclose(S, ref, rtol=1e-13, atol=1e-15)
    assert np.allclose(S.sum(axis=0), 1.0, rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------
# top-k and weights
# ----------------------------------------------------------------------------

def pin_topk_library(O):
    """Without ties, the top-k indices and their order equal torch.topk in float64."""
    for seed, (T, E, k) in enumerate([(20, 8, 2), (20, 64, 4), (7, 5, 5), (10, 16, 1)]):
        p = O.softmax_rows(_rng(10 + seed).standard_normal((T, E)) * 2)
        val, ind = torch.topk(torch.from_numpy(p), k, dim=1, largest=True, sorted=True)
        assert np.array_equal(O.topk_experts(p, k), ind.numpy()), (T, E, k)


def pin_topk_ties_low_index(O):
    """W_g = 0 (all experts tied): every token picks experts 0..k-1 in order.
    A designed tie between two experts picks the lower index first."""
    x = _rng(6).standard_normal((4, 3))
    idx, w, p, _ = O.route_tc(x, np.zeros((3, 8)), None, 3)
    assert np.array_equal(idx, np.tile(np.arange(3), (4, 1))), idx
    # experts 5 and 2 tied at the top, expert 7 third
    b = np.zeros(8)
    b[5] = b[2] = 2.0
    b[7] = 1.0
    idx, w, p, _ = O.route_tc(x, np.zeros((3, 8)), b, 3)
    assert np.array_equal(idx, np.tile([2, 5, 7], (4, 1))), idx


def pin_topk_designed_winners(O):
    """One-hot tokens with a designed W_g: token t's logits are row t of W_g, so
    the winners are known by construction."""
    E, k = 6, 2
    Wg = np.array([[5, 4, 0, 0, 0, 0],
                   [0, 0, 0, 3, 9, 0],
                   [1, 0, 0, 0, 0, 2],
                   [0, 0, 7, 0, 0, 6.5]], dtype=float)
    x = np.eye(4)
    idx, w, p, _ = O.route_tc(x, Wg, None, k)
    assert idx.tolist() == [[0, 1], [4, 3], [5, 0], [2, 5]], idx
    # renormalised weight of the winner is the logistic of the logit gap
    gaps = np.array([1.0, 6.0, 1.0, 0.5])
    assert np.allclose(w[:, 0], 1.0 / (1.0 + np.exp(-gaps)), rtol=1e-14)


def pin_brute_router(O):
    """Router outputs equal the brute force (subset enumeration) on T <= 8."""
    for seed in range(6):
        c = _case(100 + seed, T=8, d=5, E=6, bias=(seed % 2 == 0))
        for k in (1, 2, 3, 6):
            for ren in (True, False):
                idx, w, p, _ = O.route_tc(c["x"], c["Wg"], c["b"], k, ren)
                r = B.forward_tc(_lists(c["x"]), _lists(c["Wg"]), _lists(c["b"]),
                                 _lists(c["Wgate"]), _lists(c["Wup"]), _lists(c["Wdown"]),
                                 k, ren)
                assert idx.tolist() == r["idx"], (seed, k)
                assert np.allclose(w, r["w"], rtol=1e-12, atol=1e-15)
                assert np.allclose(p, r["probs"], rtol=1e-12, atol=1e-15)


def pin_renormalised_weights(O):
    """Renormalised weights sum to 1 and equal the softmax taken over the k
    selected logits alone (the logit-top-k form of the Chinese page's torch
    ``MoELayer``), an independent formula. Without renormalisation they are
    the raw probabilities."""
    x = _rng(7).standard_normal((30, 6))
    Wg = _rng(8).standard_normal((6, 16))
    b = _rng(9).standard_normal(16)
    idx, w, p, s = O.route_tc(x, Wg, b, 4, True)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-14)
    sl = torch.from_numpy(x @ Wg + b)
    val, ind = torch.topk(sl, 4, dim=1)
    assert np.array_equal(idx, ind.numpy())
    assert np.allclose(w, torch.softmax(val, dim=1).numpy(), rtol=1e-12)
    idx0, w0, p0, _ = O.route_tc(x, Wg, b, 4, False)
    assert np.allclose(w0, torch.softmax(sl, dim=1).gather(1, ind).numpy(), rtol=1e-12)


# ----------------------------------------------------------------------------
# experts and combine
# ----------------------------------------------------------------------------

def pin_single_expert_is_dense_swiglu(O):
    """E = 1, k = 1: the layer is one SwiGLU FFN, checked against torch's
    F.silu and matmul in float64."""
    c = _case(11, T=13, d=8, f=12, E=1)
    out = O.forward_tc(c["x"], c["Wg"], None, c["Wgate"], c["Wup"], c["Wdown"], 1)
    X = torch.from_numpy(c["x"])
    ref = (F.silu(X @ torch.from_numpy(c["Wgate"][0])) * (X @ torch.from_numpy(c["Wup"][0]))) \
        @ torch.from_numpy(c["Wdown"][0])
    assert np.allclose(out["y"], ref.numpy(), rtol=1e-12, atol=1e-14)
    assert np.allclose(out["w"], 1.0)


def pin_zero_input(O):
    """x = 0 gives y = 0 (silu(0) = 0), and routing is uniform."""
    c = _case(12, T=4, d=6, f=5, E=4)
    out = O.forward_tc(np.zeros((4, 6)), c["Wg"], None, c["Wgate"], c["Wup"], c["Wdown"], 2)
    assert np.array_equal(out["y"], np.zeros((4, 6)))
    assert np.array_equal(out["probs"], np.full((4, 4), 0.25))


def pin_k_equals_E_is_dense(O):
    """k = E without renormalisation equals the dense softmax mixture of all
    experts (the Chinese page's ``MixtureOfExperts``), computed here in torch."""
    c = _case(13, T=10, d=6, f=9, E=5, bias=True)
    out = O.forward_tc(c["x"], c["Wg"], c["b"], c["Wgate"], c["Wup"], c["Wdown"], 5, False)
    X = torch.from_numpy(c["x"])
    g = torch.softmax(X @ torch.from_numpy(c["Wg"]) + torch.from_numpy(c["b"]), dim=1)
    ref = torch.zeros(10, 6, dtype=torch.float64)
    for e in range(5):
        h = F.silu(X @ torch.from_numpy(c["Wgate"][e])) * (X @ torch.from_numpy(c["Wup"][e]))
        ref += g[:, e:e + 1] * (h @ torch.from_numpy(c["Wdown"][e]))
    assert np.allclose(out["y"], ref.numpy(), rtol=1e-12, atol=1e-14)


def pin_dense_mixture(O):
    """The dense mixture y = sum_e g_e E_e(x) over every expert (the Chinese page's
    ``MixtureOfExperts``) equals the same sum computed in torch float64 with a bias, and
    the literal per-token loops of the brute-force expert on a second case; its gates are
    the full softmax (not a top-k), so a token's output changes when any expert's
    weights change."""
    c = _case(21, T=9, d=6, f=8, E=5, bias=True)
    got = O.dense_mixture(c["x"], c["Wg"], c["b"], c["Wgate"], c["Wup"], c["Wdown"])
    X = torch.from_numpy(c["x"])
    g = torch.softmax(X @ torch.from_numpy(c["Wg"]) + torch.from_numpy(c["b"]), dim=1)
    ref = torch.zeros(9, 6, dtype=torch.float64)
    for e in range(5):
        h = F.silu(X @ torch.from_numpy(c["Wgate"][e])) * (X @ torch.from_numpy(c["Wup"][e]))
        ref += g[:, e:e + 1] * (h @ torch.from_numpy(c["Wdown"][e]))
    assert np.allclose(got, ref.numpy(), rtol=1e-12, atol=1e-14)
    c = _case(22, T=4, d=3, f=5, E=3, bias=False, wg_std=2.0)
    got = O.dense_mixture(c["x"], c["Wg"], None, c["Wgate"], c["Wup"], c["Wdown"])
    for t in range(4):
        s = [sum(c["x"][t, i] * c["Wg"][i, e] for i in range(3)) for e in range(3)]
        m = max(s)
        ex = [math.exp(v - m) for v in s]
        want = [0.0] * 3
        for e in range(3):
            out = B.expert(_lists(c["x"][t]), _lists(c["Wgate"][e]), _lists(c["Wup"][e]),
                           _lists(c["Wdown"][e]))
            for j in range(3):
                want[j] += ex[e] / sum(ex) * out[j]
        assert np.allclose(got[t], want, rtol=1e-12, atol=1e-14), t


def pin_brute_layer(O):
    """Whole token-choice layer equals the literal-loop brute force on T <= 8
    to 1e-12 relative."""
    for seed in range(4):
        c = _case(200 + seed, T=7, d=6, f=5, E=5, bias=(seed % 2 == 1))
        for k, ren in ((2, True), (3, False), (1, True)):
            out = O.forward_tc(c["x"], c["Wg"], c["b"], c["Wgate"], c["Wup"], c["Wdown"], k, ren)
            r = B.forward_tc(_lists(c["x"]), _lists(c["Wg"]), _lists(c["b"]), _lists(c["Wgate"]),
                             _lists(c["Wup"]), _lists(c["Wdown"]), k, ren)
            y = np.asarray(r["y"])
            assert np.max(np.abs(out["y"] - y)) <= 1e-12 * np.max(np.abs(y)), (seed, k)


def pin_linearity_and_equivariance(O):
    """y is linear in W_down; permuting tokens permutes rows of y and idx;
    relabelling experts (permuting W_g columns and expert stacks) relabels idx
    and leaves y unchanged."""
    c = _case(14, T=12, d=6, f=7, E=6, bias=True)
    args = (c["Wgate"], c["Wup"], c["Wdown"])
    base = O.forward_tc(c["x"], c["Wg"], c["b"], *args, 2)
    scaled = O.forward_tc(c["x"], c["Wg"], c["b"], c["Wgate"], c["Wup"], 2.5 * c["Wdown"], 2)
    assert np.allclose(scaled["y"], 2.5 * base["y"], rtol=1e-12, atol=1e-14)
    perm = _rng(15).permutation(12)
    pt = O.forward_tc(c["x"][perm], c["Wg"], c["b"], *args, 2)
    assert np.array_equal(pt["idx"], base["idx"][perm])
    assert np.allclose(pt["y"], base["y"][perm], rtol=1e-13, atol=1e-15)
    relab = _rng(16).permutation(6)          # new expert i is old expert relab[i]
    inv = np.argsort(relab)
    pe = O.forward_tc(c["x"], c["Wg"][:, relab], c["b"][relab], c["Wgate"][relab],
                      c["Wup"][relab], c["Wdown"][relab], 2)
    assert np.array_equal(relab[pe["idx"]], base["idx"])
    assert np.allclose(pe["y"], base["y"], rtol=1e-12, atol=1e-14)
    assert inv.shape == (6,)


# ----------------------------------------------------------------------------
# load-balancing statistics
# ----------------------------------------------------------------------------

def pin_aux_invariants(O):
    """sum f = k, sum p = 1, sum counts = T*k, 0 < loss <= E."""
    for seed, (T, E, k) in enumerate([(40, 8, 2), (64, 64, 4), (9, 3, 1)]):
        x = _rng(300 + seed).standard_normal((T, 5))
        Wg = _rng(400 + seed).standard_normal((5, E))
        idx, w, p, _ = O.route_tc(x, Wg, None, k)
        f, pm, loss, cnt = O.aux_stats(p, idx, E, k)
        assert cnt.sum() == T * k
        assert np.isclose(f.sum(), k, rtol=1e-14)
        assert np.isclose(pm.sum(), 1.0, rtol=1e-14)
        assert 0.0 < loss <= E + 1e-12
        # counts against a direct per-expert tally over the flattened slots
        tally = [sum(1 for v in idx.ravel() if v == e) for e in range(E)]
        assert cnt.tolist() == tally


def pin_aux_uniform_probs(O):
    """Uniform router probabilities (W_g = 0) give loss = 1 for any f, and the
    first page's scale E * sum(f * p) gives its stated ideal value top_k."""
    for E, k in ((8, 2), (16, 4), (4, 1)):
        x = _rng(17).standard_normal((32, 3))
        idx, w, p, _ = O.route_tc(x, np.zeros((3, E)), None, k)
        f, pm, loss, cnt = O.aux_stats(p, idx, E, k)
        assert loss == 1.0, loss
        assert np.isclose(E * np.sum(f * pm), k, rtol=1e-15)


def pin_aux_uniform_counts(O):
    """Perfectly balanced assignments (T = m*E tokens, token t routed to experts
    t mod E .. t+k-1 mod E by construction) give loss = sum p = 1 whatever p is."""
    E, k, m = 8, 2, 5
    T = m * E
    x = np.eye(E)[np.arange(T) % E] * 10.0        # token t is one-hot at t mod E
    Wg = np.zeros((E, E))
    for r in range(E):
        Wg[r, r] = 3.0
        Wg[r, (r + 1) % E] = 2.0                  # second choice: the next expert
        Wg[r, (r + 2) % E] = -1.0
    idx, w, p, _ = O.route_tc(x, Wg, None, k)
    assert idx.tolist() == [[t % E, (t + 1) % E] for t in range(T)]
    f, pm, loss, cnt = O.aux_stats(p, idx, E, k)
    assert cnt.tolist() == [m * k] * E
    assert np.isclose(loss, 1.0, rtol=1e-14), loss


def pin_golden_page_values(O):
    """Values the pages state, from tests/golden/page_values.json."""
    with open(os.path.join(GOLDEN, "page_values.json")) as fh:
        g = json.load(fh)
    d = g["p1_ideal_loss_is_top_k"]
    x = _rng(18).standard_normal((d["T"], d["d_model"])) * 0.5
    idx, w, p, _ = O.route_tc(x, np.zeros((d["d_model"], d["E"])), None, d["k"])
    f, pm, loss, cnt = O.aux_stats(p, idx, d["E"], d["k"])
    assert np.isclose(d["E"] * np.sum(f * pm), d["value"], rtol=1e-15)
    d = g["p1_ideal_tokens_per_expert"]
    # a balanced assignment reaches the ideal count T*k/E for every expert
    T, E, k = d["T"], d["E"], d["k"]
    idx = np.array([[(t * k + j) % E for j in range(k)] for t in range(T)])
    assert O.expert_counts(idx, E).tolist() == [d["value"]] * E
    d = g["p3_expert_capacity"]
    assert O.capacity(d["T"], d["E"], d["capacity_factor"]) == d["value"]
    d = g["p3_expert_capacity_truncates"]
    assert O.capacity(d["T"], d["E"], d["capacity_factor"]) == d["value"]


# ----------------------------------------------------------------------------
# expert choice
# ----------------------------------------------------------------------------

def pin_ec_brute(O):
    """Expert-choice routing and output equal the brute force (enumerating all
    C-subsets of tokens per expert) on T <= 8, with exactly C tokens per expert."""
    for seed in range(4):
        c = _case(500 + seed, T=8, d=5, f=6, E=4, bias=(seed % 2 == 0))
        for cf in (1.0, 2.0, 1.5, 0.5):
            out = O.forward_ec(c["x"], c["Wg"], c["b"], c["Wgate"], c["Wup"], c["Wdown"], cf)
            C = int(8 * cf / 4)
            r = B.forward_ec(_lists(c["x"]), _lists(c["Wg"]), _lists(c["b"]), _lists(c["Wgate"]),
                             _lists(c["Wup"]), _lists(c["Wdown"]), cf)
            assert out["idx"].shape == (4, C)
            assert out["idx"].tolist() == r["idx"], (seed, cf)
            assert np.allclose(out["w"], r["w"], rtol=1e-12)
            y = np.asarray(r["y"])
            assert np.max(np.abs(out["y"] - y)) <= 1e-12 * max(1e-300, np.max(np.abs(y)))


def pin_ec_single_expert_closed_form(O):
    """E = 1, cf = 1: C = T, every token is taken, and y_t = S_t * E_1(x_t) with
    S the softmax of the single logit column over all tokens (torch in float64)."""
    c = _case(19, T=9, d=4, f=6, E=1)
    out = O.forward_ec(c["x"], c["Wg"], None, c["Wgate"], c["Wup"], c["Wdown"], 1.0)
    assert out["idx"].tolist() == [list(range(9))]
    X = torch.from_numpy(c["x"])
    S = torch.softmax((X @ torch.from_numpy(c["Wg"]))[:, 0], dim=0)
    h = F.silu(X @ torch.from_numpy(c["Wgate"][0])) * (X @ torch.from_numpy(c["Wup"][0]))
    ref = S[:, None] * (h @ torch.from_numpy(c["Wdown"][0]))
    assert np.allclose(out["y"], ref.numpy(), rtol=1e-12, atol=1e-15)


def pin_ec_uncovered_tokens_zero(O):
    """A token that no expert selects gets y = 0; a designed token with the
    largest logit in every column is selected by every expert."""
    T, E = 8, 2
    x = np.zeros((T, 2))
    x[:, 0] = np.arange(T)          # logit of expert 0 grows with t
    x[:, 1] = -np.arange(T)         # logit of expert 1 grows with -t
    Wg = np.eye(2)
    r = _rng(20)
    Wgate, Wup = r.standard_normal((E, 2, 3)), r.standard_normal((E, 2, 3))
    Wdown = r.standard_normal((E, 3, 2))
    out = O.forward_ec(x, Wg, None, Wgate, Wup, Wdown, 0.5)  # C = 2
    assert out["idx"].tolist() == [[6, 7], [0, 1]]
    assert np.array_equal(out["y"][2:6], np.zeros((4, 2)))
    assert np.any(out["y"][7] != 0)


def pin_margins(O):
    """Top-k margin is the gap between the k-th and (k+1)-th probability and
    +inf when k = E; expert-choice margin is the gap of the C-th and (C+1)-th
    logit of each column and +inf when C = T."""
    p = np.array([[0.05, 0.45, 0.2, 0.3], [0.25, 0.25, 0.25, 0.25]])
    assert np.allclose(O.topk_margin(p, 2), [0.1, 0.0])
    assert np.all(np.isinf(O.topk_margin(p, 4)))
    s = np.array([[1.0, 0.0], [3.0, 2.0], [2.5, 5.0]])
    assert np.allclose(O.ec_margin(s, 1), [0.5, 3.0])
    assert np.all(np.isinf(O.ec_margin(s, 3)))



# ----------------------------------------------------------------------------
# token choice with an expert capacity
# ----------------------------------------------------------------------------

def pin_capacity_golden(O):
    """The capacity of the page's own call (tests/golden/page_values.json), and the
    truncation of the product at a few exact points."""
    with open(os.path.join(GOLDEN, "page_values.json")) as fh:
        d = json.load(fh)["p5_capacity_of_page_call"]
    assert O.tc_capacity(d["T"], d["E"], d["k"], d["capacity_factor"]) == d["value"]
    for T, E, k, cf, C in [(64, 8, 1, 1.0, 8), (10, 4, 2, 1.0, 5), (7, 8, 1, 1.0, 0),
                           (1000, 8, 2, 1.25, 312), (12, 8, 2, 1.0, 3)]:
        assert O.tc_capacity(T, E, k, cf) == C, (T, E, k, cf)


def pin_capacity_unlimited_is_plain_tc(O):
    """A capacity of at least T*k drops nothing: routing equals plain token choice."""
    c = _case(31, T=9, E=5, bias=True)
    for renorm in (True, False):
        idx, w, kept, p, s, load = O.route_tc_capacity(c["x"], c["Wg"], c["b"], 2, 1e6, renorm)
        idx0, w0, p0, s0 = O.route_tc(c["x"], c["Wg"], c["b"], 2, renorm)
        assert kept.all()
        assert np.array_equal(idx, idx0)
        assert np.allclose(w, w0, rtol=1e-15, atol=0)
        assert load.tolist() == np.bincount(idx0.ravel(), minlength=5).tolist()


def pin_capacity_brute(O):
    """Output, weights, kept slots and loads equal the literal-loop brute force
    (subset enumeration for top-k, a running count per expert) under tight
    capacities, with and without renormalisation."""
    for seed, cf, T, E, k in [(32, 0.5, 7, 4, 2), (33, 0.75, 8, 3, 2), (34, 0.4, 6, 4, 1),
                              (35, 1.0, 8, 4, 3)]:
        c = _case(seed, T=T, E=E, bias=True, wg_std=1.5)
        for renorm in (True, False):
            ref = B.forward_tc_capacity(_lists(c["x"]), _lists(c["Wg"]), _lists(c["b"]),
                                        _lists(c["Wgate"]), _lists(c["Wup"]), _lists(c["Wdown"]),
                                        k, cf, renorm)
            got = O.forward_tc_capacity(c["x"], c["Wg"], c["b"], c["Wgate"], c["Wup"],
                                        c["Wdown"], k, cf, renorm)
            assert got["idx"].tolist() == ref["idx"]
            assert got["kept"].tolist() == ref["kept"]
            assert got["load"].tolist() == ref["load"]
            assert np.allclose(got["w"], np.array(ref["w"]), rtol=1e-12, atol=1e-15)
            assert np.allclose(got["y"], np.array(ref["y"]), rtol=1e-10, atol=1e-12)


def pin_capacity_one_expert_closed_form(O):
    """Every token routed to one expert with k = 1: the first C tokens keep weight 1
    and that expert's output; the others get weight 0 and y = 0."""
    T, E, cf = 10, 4, 1.2   # C = int(10 / 4 * 1.2 * 1) = 3
    c = _case(36, T=T, E=E)
    b = np.zeros(E)
    b[2] = 60.0
    got = O.forward_tc_capacity(c["x"], c["Wg"], b, c["Wgate"], c["Wup"], c["Wdown"], 1, cf)
    assert got["idx"][:, 0].tolist() == [2] * T
    assert got["kept"][:, 0].tolist() == [True] * 3 + [False] * (T - 3)
    assert got["w"][:, 0].tolist() == [1.0] * 3 + [0.0] * (T - 3)
    for t in range(T):
        want = B.expert(_lists(c["x"][t]), _lists(c["Wgate"][2]), _lists(c["Wup"][2]),
                        _lists(c["Wdown"][2])) if t < 3 else [0.0] * c["x"].shape[1]
        assert np.allclose(got["y"][t], want, rtol=1e-10, atol=1e-12), t


def pin_capacity_zero_drops_everything(O):
    """Capacity 0 (int() of a product below 1): every slot dropped, all weights and
    outputs exactly 0, no NaN from an empty renormalisation."""
    c = _case(37, T=5, E=8)
    got = O.forward_tc_capacity(c["x"], c["Wg"], None, c["Wgate"], c["Wup"], c["Wdown"], 1, 1.0)
    assert not got["kept"].any()
    assert np.all(got["w"] == 0.0) and np.all(got["y"] == 0.0)
    assert got["load"].tolist() == [0] * 8


def pin_capacity_keeps_earliest_tokens(O):
    """Invariants: each expert keeps min(count, C) assignments, and they are its
    earliest tokens; each token's kept weights sum to 1 (or it has none)."""
    c = _case(38, T=40, d=6, E=5, bias=True, wg_std=1.0)
    idx, w, kept, p, s, load = O.route_tc_capacity(c["x"], c["Wg"], c["b"], 2, 0.6)
    C = O.tc_capacity(40, 5, 2, 0.6)
    for e in range(5):
        tt, jj = np.nonzero(idx == e)
        order = np.argsort(tt, kind="stable")
        flags = kept[tt[order], jj[order]]
        n = min(len(tt), C)
        assert flags.tolist() == [True] * n + [False] * (len(tt) - n), e
        assert load[e] == n
    sums = w.sum(axis=1)
    assert np.allclose(sums[kept.any(axis=1)], 1.0, rtol=1e-14)
    assert np.all(sums[~kept.any(axis=1)] == 0.0)


# ----------------------------------------------------------------------------
# router z-loss
# ----------------------------------------------------------------------------

def pin_zloss_brute(O):
    """Equals the token-by-token scalar computation, with and without a bias."""
    for seed, T, E, bias in [(41, 7, 4, True), (42, 5, 8, False), (43, 1, 3, True)]:
        c = _case(seed, T=T, E=E, bias=bias, wg_std=1.3)
        s = O.router_logits(c["x"], c["Wg"], c["b"])
        ref = B.router_z_loss(_lists(c["x"]), _lists(c["Wg"]), _lists(c["b"]))
        assert math.isclose(O.router_z_loss(s), ref, rel_tol=1e-12), (seed, ref)


def pin_zloss_library(O):
    """Equals torch.logsumexp squared and averaged over tokens."""
    r = _rng(44)
    for T, E in [(33, 8), (5, 64), (16, 1)]:
        s = r.standard_normal((T, E)) * 3.0
        ref = float((torch.logsumexp(torch.from_numpy(s), dim=-1) ** 2).mean())
        assert math.isclose(O.router_z_loss(s), ref, rel_tol=1e-12)


def pin_zloss_closed_forms(O):
    """Equal logits c: (c + log E)^2 per token; one expert: mean of s^2; a per-token
    shift c_t moves each log-partition by c_t; no tokens: 0."""
    for E, c in [(8, 0.0), (4, -2.5), (64, 1.25)]:
        assert math.isclose(O.router_z_loss(np.full((3, E), c)), (c + math.log(E)) ** 2,
                            rel_tol=1e-13)
    s1 = np.array([[0.5], [-2.0], [3.0]])
    assert math.isclose(O.router_z_loss(s1), (0.25 + 4.0 + 9.0) / 3, rel_tol=1e-14)
    r = _rng(45)
    s = r.standard_normal((6, 5))
    lse = [math.log(sum(math.exp(v) for v in row)) for row in s.tolist()]
    shift = r.standard_normal(6)
    want = sum((a + b) ** 2 for a, b in zip(lse, shift.tolist())) / 6
    assert math.isclose(O.router_z_loss(s + shift[:, None]), want, rel_tol=1e-12)
    assert O.router_z_loss(np.zeros((0, 4))) == 0.0


# ----------------------------------------------------------------------------
# noisy top-k gating
# ----------------------------------------------------------------------------

def _noise_case(seed, T=6, d=5, E=4, bias=True, eps_std=1.0):
    c = _case(seed, T=T, E=E, d=d, bias=bias, wg_std=0.8)
    r = _rng(seed + 1000)
    c["Wn"] = r.standard_normal((d, E)) * 0.6
    c["eps"] = r.standard_normal((T, E)) * eps_std
    return c


def pin_softplus_library(O):
    """softplus equals torch's (whose linear cut-off is moved past the range), log 2
    at 0, and softplus(z) - softplus(-z) = z."""
    z = np.linspace(-30.0, 30.0, 241)
    ref = F.softplus(torch.from_numpy(z), beta=1.0, threshold=100.0).numpy()
    assert np.allclose(O.softplus(z), ref, rtol=1e-12, atol=1e-300)
    assert math.isclose(float(O.softplus(np.array(0.0))), math.log(2.0), rel_tol=1e-15)
    assert np.allclose(O.softplus(z) - O.softplus(-z), z, rtol=1e-12, atol=1e-12)


def pin_noisy_brute(O):
    """Noisy routing and layer equal the literal-loop brute force, with the P3
    softplus scale and with additive noise (Wn = None)."""
    for seed, T, E, k, use_wn in [(51, 6, 4, 2, True), (52, 7, 5, 1, True), (53, 5, 4, 3, False)]:
        c = _noise_case(seed, T=T, E=E, eps_std=2.0)
        Wn = c["Wn"] if use_wn else None
        ref = B.forward_tc(_lists(c["x"]), _lists(c["Wg"]), _lists(c["b"]), _lists(c["Wgate"]),
                           _lists(c["Wup"]), _lists(c["Wdown"]), k, True, _lists(Wn),
                           _lists(c["eps"]))
        idx, w, p, s = O.route_tc_noisy(c["x"], c["Wg"], c["b"], Wn, c["eps"], k)
        assert idx.tolist() == ref["idx"]
        assert np.allclose(w, np.array(ref["w"]), rtol=1e-12, atol=1e-15)
        assert np.allclose(p, np.array(ref["probs"]), rtol=1e-12, atol=1e-15)
        y = O.mix(c["x"], idx, w, c["Wgate"], c["Wup"], c["Wdown"])
        assert np.allclose(y, np.array(ref["y"]), rtol=1e-10, atol=1e-12)


def pin_noisy_special_cases(O):
    """eps = 0 is plain routing; W_noise = 0 scales the draw by log 2; a draw that
    is constant over a token's experts changes none of its probabilities; a large
    draw on one expert selects it."""
    c = _noise_case(54, T=8, E=6)
    plain = O.route_tc(c["x"], c["Wg"], c["b"], 2)
    zero = O.route_tc_noisy(c["x"], c["Wg"], c["b"], c["Wn"], np.zeros((8, 6)), 2)
    assert np.array_equal(zero[0], plain[0]) and np.allclose(zero[2], plain[2], rtol=1e-15)
    s0 = O.noisy_logits(c["x"], c["Wg"], c["b"], np.zeros((5, 6)), c["eps"])
    s_ref = torch.from_numpy(c["x"]) @ torch.from_numpy(c["Wg"]) + torch.from_numpy(c["b"])
    assert np.allclose(s0, s_ref.numpy() + math.log(2.0) * c["eps"], rtol=1e-13, atol=1e-14)
    shift = np.repeat(_rng(55).standard_normal((8, 1)) * 5.0, 6, axis=1)
    moved = O.route_tc_noisy(c["x"], c["Wg"], c["b"], None, shift, 2)
    assert np.allclose(moved[2], plain[2], rtol=1e-12, atol=1e-15)
    spike = np.zeros((8, 6))
    spike[:, 4] = 50.0
    assert np.all(O.route_tc_noisy(c["x"], c["Wg"], c["b"], c["Wn"], spike, 1)[0][:, 0] == 4)


def pin_philox_known_answers(O):
    """Philox4x32-10 reproduces the generator's published known-answer vectors
    (tests/golden/philox4x32_10_kat.json), one counter at a time and as a batch."""
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.json")) as fh:
        vec = json.load(fh)["vectors"]
    ctr = np.array([[int(h, 16) for h in v["counter"]] for v in vec], dtype=np.uint64)
    for i, v in enumerate(vec):
        key = tuple(int(h, 16) for h in v["key"])
        out = O.philox4x32_10(ctr[i], key)
        assert [int(u) for u in out] == [int(h, 16) for h in v["out"]], v


def pin_noise_draw_is_standard_normal(O):
    """One million draws of the in-kernel noise definition pass as independent
    standard normals: mean, variance, a Kolmogorov-Smirnov test against N(0, 1), the
    tail mass beyond 3, and no correlation between a token's neighbouring experts
    (the cosine and sine of one Box-Muller pair, and the pairs of one Philox call)."""
    from scipy import stats
    eps = O.noise_draw(65536, 16, seed=0x5EED5EED1234, offset=3)
    n = eps.size
    flat = eps.ravel()
    assert abs(flat.mean()) < 5.0 / math.sqrt(n)
    assert abs(flat.var() - 1.0) < 5.0 * math.sqrt(2.0 / n)
    assert stats.kstest(flat, "norm").pvalue > 1e-4
    tail = float(np.mean(np.abs(flat) > 3.0))
    assert abs(tail - 2.0 * stats.norm.sf(3.0)) < 6.0 * math.sqrt(2.0 * stats.norm.sf(3.0) / n)
    for a, b in ((0, 1), (2, 3), (0, 2), (1, 3), (3, 4)):
        rho = np.corrcoef(eps[:, a], eps[:, b])[0, 1]
        assert abs(rho) < 5.0 / math.sqrt(eps.shape[0]), (a, b, rho)


def pin_noise_draw_counter_based(O):
    """The draw of (t, e) depends on (seed, offset, t, e) only: a smaller batch or
    fewer experts read the same numbers, a new offset or seed draws new ones, scale
    multiplies, and the vectorised draw equals the scalar evaluation of the
    definition in pure Python (oracle/brute.py) element by element."""
    big = O.noise_draw(300, 12, seed=77, offset=5)
    assert np.array_equal(O.noise_draw(7, 12, seed=77, offset=5), big[:7])
    assert np.array_equal(O.noise_draw(300, 5, seed=77, offset=5), big[:, :5])
    other = O.noise_draw(300, 12, seed=77, offset=6)
    assert np.mean(other == big) < 0.01
    assert np.mean(O.noise_draw(300, 12, seed=78, offset=5) == big) < 0.01
    assert np.allclose(O.noise_draw(300, 12, seed=77, offset=5, scale=-2.5), -2.5 * big,
                       rtol=1e-15, atol=0.0)
    for t, e in ((0, 0), (1, 3), (17, 6), (299, 11), (123, 9)):
        ref = B.noise_draw_one(t, e, seed=77, offset=5)
        assert math.isclose(float(big[t, e]), ref, rel_tol=1e-12, abs_tol=1e-12), (t, e)
    hi = O.noise_draw(4, 8, seed=(3 << 32) | 9, offset=(5 << 32) | 1)
    for t, e in ((0, 0), (3, 7), (2, 5)):
        ref = B.noise_draw_one(t, e, seed=(3 << 32) | 9, offset=(5 << 32) | 1)
        assert math.isclose(float(hi[t, e]), ref, rel_tol=1e-12, abs_tol=1e-12), (t, e)


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
