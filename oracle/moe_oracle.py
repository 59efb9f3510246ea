"""fp64 CPU oracle for the sparse Mixture-of-Experts layer forward.

TEST INFRASTRUCTURE ONLY. This module is the checker, not the product: only
``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import or call it. It shares no code with the HIP library and
imports nothing from it.

Every function is the plain definition written out in NumPy float64, one step
per statement, in the order the pages give the steps. Inputs are the exact
values the device sees (bf16 or fp32 values widened to float64; nothing is
re-rounded). Library routines used as steps: ``@`` (matmul), ``np.exp``,
``np.argsort(kind="stable")``.

Pages cited (by title):
  P1 "Mixture of Experts（MoE）の理論と実装 — 条件付き計算でLLMを効率化する"
     (classes ``Expert`` and ``MoELayer``: ``route``, ``forward``,
     ``load_balancing_loss``)
  P2 "MoE" primer on qiita (section "ゲート / ルーターって何者？", the four
     router equations s = W_g x, g = softmax(s), TopK(g), y = sum g_i E_i(x))
  P3 "Sparse Mixture of Experts(MoE) 아키텍처 심층 분석" (``SwiGLUExpert``,
     ``TopKGating``, ``ExpertChoiceGating``, ``compute_load_balancing_loss``,
     ``MoELayerWithAuxLoss``)
  P5 "机器学习基础系列——混合专家模型" (``GatingNetwork`` with bias,
     ``MixtureOfExperts`` dense mixture, ``SparseMoE``,
     ``expert_capacity_routing``)

Readings where the pages leave a step open or disagree:
  * renormalisation: P1/P3 code renormalise the selected weights, P2's
    equations do not; both are provided (``renormalize`` flag).
  * ties: experts with equal probability are ordered by lower index; in
    expert-choice mode tokens with equal score are ordered by lower token index.
  * slot order: descending probability (P1 ``route``, P3 ``TopKGating``).
  * f = count/T so that sum(f) = k (P1 ``load_balancing_loss``); the loss is
    E * sum((f/k) * p), which is P3's scale (sum(f/k) = 1) and equals 1 under
    uniform routing.
  * expert choice: softmax over tokens of each expert's logit column, top-C
    tokens per expert with C = floor(T*cf/E), outputs combined with the
    selected scores and no renormalisation; a token no expert picks gets 0.
  * noisy top-k gating (P3 ``TopKGating`` training branch): the noise is added
    to the logits, bias included, before the softmax; the normal draw eps is an
    input. P5's fixed-scale noise is the same with Wn = None and eps scaled by
    the caller. Token choice only (P3's ``ExpertChoiceGating`` has no noise).
    The pages draw eps with torch's generator; a draw that both sides can make
    without passing it is the counter-based one of ``noise_draw`` (Philox4x32-10
    and the Box-Muller transform, from their published definitions, not from
    the pages).
  * router z-loss (P3 ``router_z_loss``) is taken on the logits the softmax sees,
    bias included, for every routing mode (it depends on the logits only); with
    no tokens it is 0. P5 prints another quantity under the same name (a mean
    sum of squared gates); it conflicts with P3 and is not provided.
  * token choice with an expert capacity (P5 ``expert_capacity_routing``):
    capacity = int((T / E) * cf * k); assignments are taken token by token and
    kept while the expert is below capacity. The page walks a token's slots
    from its smallest selected gate up; a token's slots go to distinct
    experts, so that order decides nothing. Kept gates are renormalised over
    the token's kept slots (zeros stay zeros); with renormalize=False (not on
    the page, which always renormalises) the kept slots keep the raw gates.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def _f64(a):
    return None if a is None else np.asarray(a, dtype=F64)


# --------------------------------------------------------------------------
# Router (token choice)
# --------------------------------------------------------------------------

def router_logits(x, Wg, b=None):
    """s = x W_g (+ b). P2 first router equation (written as x @ W in P1
    ``MoELayer.route``); the optional bias is P5 ``GatingNetwork.forward``."""
    s = _f64(x) @ _f64(Wg)
    if b is not None:
        s = s + _f64(b)[None, :]
    return s


def softmax_rows(s):
    """g = softmax(s) over the experts of each token, shifted by the row max
    (P1 ``MoELayer.route``; P2 second router equation)."""
    s = _f64(s)
    z = s - s.max(axis=1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=1, keepdims=True)


def topk_experts(p, k):
    """TopK(g): the k experts of largest probability per token, listed by
    descending probability, lower expert index first among equals (P1
    ``route``, P3 ``TopKGating``; tie order is this implementation's reading)."""
    p = _f64(p)
    order = np.argsort(-p, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def gate_weights(p, idx, renormalize=True):
    """Weights of the selected experts: g_i (P2 fourth equation) or g_i divided
    by the sum over the selected set (P1 ``route``, P3 ``TopKGating``)."""
    sel = np.take_along_axis(_f64(p), idx, axis=1)
    if renormalize:
        sel = sel / sel.sum(axis=1, keepdims=True)
    return sel


def route_tc(x, Wg, b, k, renormalize=True):
    """Token-choice routing: returns (idx [T,k], w [T,k], probs [T,E], logits [T,E])."""
    s = router_logits(x, Wg, b)
    p = softmax_rows(s)
    idx = topk_experts(p, k)
    w = gate_weights(p, idx, renormalize)
    return idx, w, p, s


def softplus(z):
    """softplus(z) = log(1 + exp(z)), the noise scale of P3 ``TopKGating``."""
    z = _f64(z)
    with np.errstate(over="ignore"):
        return np.log1p(np.exp(z))


def noisy_logits(x, Wg, b, Wn, eps):
    """Router logits with training noise. P3 ``TopKGating`` (training branch):
    s + softplus(x W_noise) * eps, eps a standard normal draw per (token,
    expert). P5 ``MoELayer`` (training branch) adds noise_std * eps instead: that
    is Wn = None with the scaled draw passed as eps. The draw is an input, so
    that every implementation sees the same numbers."""
    s = router_logits(x, Wg, b)
    if Wn is None:
        return s + _f64(eps)
    return s + softplus(_f64(x) @ _f64(Wn)) * _f64(eps)


# Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy
# as 1, 2, 3", SC 2011): a counter of four 32-bit words and a key of two go through
# ten rounds; a round multiplies counter words 0 and 2 by two fixed odd constants
# into 64-bit products and rebuilds the counter from their halves, the two other
# words and the key; between rounds the key takes a Weyl step (the golden-ratio
# and sqrt(3) - 1 constants).
PHILOX_M = (0xD2511F53, 0xCD9E8D57)
PHILOX_W = (0x9E3779B9, 0xBB67AE85)


def philox4x32_10(counter, key):
    """Philox4x32-10 of arrays of counters: counter uint [..., 4], key (k0, k1).
    Returns uint64 [..., 4] holding the four 32-bit output words."""
    c = [np.asarray(counter, dtype=np.uint64)[..., i] & 0xFFFFFFFF for i in range(4)]
    k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
    lo32 = np.uint64(0xFFFFFFFF)
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + PHILOX_W[0]) & 0xFFFFFFFF
            k1 = (k1 + PHILOX_W[1]) & 0xFFFFFFFF
        prod0 = np.uint64(PHILOX_M[0]) * c[0]   # < 2^64: no wrap
        prod1 = np.uint64(PHILOX_M[1]) * c[2]
        hi0, lo0 = prod0 >> np.uint64(32), prod0 & lo32
        hi1, lo1 = prod1 >> np.uint64(32), prod1 & lo32
        c = [hi1 ^ c[1] ^ np.uint64(k0), lo1, hi0 ^ c[3] ^ np.uint64(k1), lo0]
    return np.stack(c, axis=-1)


def noise_draw(T, E, seed, offset=0, scale=1.0):
    """The counter-based normal draw eps [T, E] (float64) that the library makes in
    its router when no eps is passed: for token t and expert e = 4q + 2h + c,
    Philox4x32-10 of counter (t, q, offset mod 2^32, offset div 2^32) under key
    (seed mod 2^32, seed div 2^32) gives words r0..r3; u_i = (floor(r_i / 2^8) +
    1/2) / 2^24; and the Box-Muller transform (Box and Muller, 1958) of the pair
    (u_2h, u_2h+1) gives sqrt(-2 ln u_2h) times cos (c = 0) or sin (c = 1) of
    2 pi u_2h+1. eps = scale * that."""
    Q = (E + 3) // 4
    t = np.arange(T, dtype=np.uint64)[:, None]
    q = np.arange(Q, dtype=np.uint64)[None, :]
    ctr = np.zeros((T, Q, 4), dtype=np.uint64)
    ctr[..., 0] = t
    ctr[..., 1] = q
    ctr[..., 2] = int(offset) & 0xFFFFFFFF
    ctr[..., 3] = (int(offset) >> 32) & 0xFFFFFFFF
    r = philox4x32_10(ctr, (int(seed) & 0xFFFFFFFF, (int(seed) >> 32) & 0xFFFFFFFF))
    u = ((r >> np.uint64(8)).astype(F64) + 0.5) / float(1 << 24)   # [T, Q, 4], in (0, 1)
    n = np.empty((T, Q, 4), dtype=F64)
    for h in range(2):
        rad = np.sqrt(-2.0 * np.log(u[..., 2 * h]))
        ang = 2.0 * np.pi * u[..., 2 * h + 1]
        n[..., 2 * h] = rad * np.cos(ang)
        n[..., 2 * h + 1] = rad * np.sin(ang)
    return float(scale) * n.reshape(T, 4 * Q)[:, :E]


def route_tc_noisy(x, Wg, b, Wn, eps, k, renormalize=True):
    """Noisy top-k gating (P3 ``TopKGating`` training branch): softmax, top-k
    and weights as in ``route_tc``, on the noisy logits. Returns (idx, w,
    probs, logits)."""
    s = noisy_logits(x, Wg, b, Wn, eps)
    p = softmax_rows(s)
    idx = topk_experts(p, k)
    w = gate_weights(p, idx, renormalize)
    return idx, w, p, s


def topk_margin(p, k):
    """p_(k) - p_(k+1) per token (descending order); +inf when k equals E."""
    p = _f64(p)
    E = p.shape[1]
    if k >= E:
        return np.full(p.shape[0], np.inf)
    ps = -np.sort(-p, axis=1)
    return ps[:, k - 1] - ps[:, k]


# --------------------------------------------------------------------------
# Experts
# --------------------------------------------------------------------------

def silu(z):
    """silu(z) = z / (1 + exp(-z)) (P1 ``Expert.forward``)."""
    z = _f64(z)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(X, Wgate, Wup, Wdown):
    """E_i(x) = (silu(x W_gate) * (x W_up)) W_down for the rows of X (P1
    ``Expert.forward`` with W1 = W_up and W2 = W_down; P3 ``SwiGLUExpert``)."""
    X = _f64(X)
    g = silu(X @ _f64(Wgate))
    u = X @ _f64(Wup)
    return (g * u) @ _f64(Wdown)


def mix(x, idx, w, Wgate, Wup, Wdown):
    """y_t = sum_j w[t,j] * E_{idx[t,j]}(x_t) (P2 fourth equation; P1
    ``MoELayer.forward``). Rows of each expert are gathered and run through
    that expert once; expert weights are widened to float64 one expert at a
    time so that large stacks need not be held in float64 all at once."""
    x = _f64(x)
    idx = np.asarray(idx)
    w = _f64(w)
    T = x.shape[0]
    d_out = Wdown.shape[2]
    y = np.zeros((T, d_out), dtype=F64)
    for e in np.unique(idx):
        tt, jj = np.nonzero(idx == e)
        out = expert_ffn(x[tt], Wgate[e], Wup[e], Wdown[e])
        np.add.at(y, tt, w[tt, jj][:, None] * out)
    return y


def forward_tc(x, Wg, b, Wgate, Wup, Wdown, k, renormalize=True):
    """Token-choice layer forward. Returns dict with y, idx, w, probs, logits."""
    idx, w, p, s = route_tc(x, Wg, b, k, renormalize)
    y = mix(x, idx, w, Wgate, Wup, Wdown)
    return {"y": y, "idx": idx, "w": w, "probs": p, "logits": s}


# --------------------------------------------------------------------------
# Load-balancing statistics
# --------------------------------------------------------------------------

def expert_counts(idx, E):
    """Number of (token, slot) assignments per expert (P1 ``load_balancing_loss``
    dispatch count; P3 ``tokens_per_expert``)."""
    return np.bincount(np.asarray(idx).ravel(), minlength=E).astype(np.int64)


def aux_stats(probs, idx, E, k):
    """f_e = count_e / T (sum f = k, P1), p_e = mean_t probs[t,e] (P1, P3),
    loss = E * sum_e (f_e / k) * p_e (P3 ``compute_load_balancing_loss`` scale).
    Returns (f, p, loss, counts)."""
    probs = _f64(probs)
    T = probs.shape[0]
    c = expert_counts(idx, E)
    f = c.astype(F64) / T
    p = probs.mean(axis=0)
    loss = E * np.sum((f / k) * p)
    return f, p, float(loss), c


def router_z_loss(s):
    """Router z-loss (P3 ``router_z_loss``, the ST-MoE form): the mean over tokens
    of the squared log-partition log(sum_e exp(s_te)) of the router logits. The
    logits are the ones the softmax normalises, bias included. No tokens: 0."""
    s = _f64(s)
    if s.shape[0] == 0:
        return 0.0
    lse = np.log(np.exp(s).sum(axis=1))
    return float(np.mean(lse ** 2))


# --------------------------------------------------------------------------
# Expert choice
# --------------------------------------------------------------------------

def capacity(T, E, cf):
    """C = int(T * cf / E) (P3 ``ExpertChoiceGating``)."""
    return int(T * cf / E)


def softmax_cols(s):
    """Each expert's softmax over the tokens of its logit column (P3
    ``ExpertChoiceGating``: softmax of the transposed logits)."""
    s = _f64(s)
    z = s - s.max(axis=0, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=0, keepdims=True)


def route_ec(x, Wg, b, cf):
    """Expert-choice routing (P3 ``ExpertChoiceGating``): expert e takes the C
    tokens of largest column-softmax score, lower token first among equals;
    idx [E,C] lists each expert's tokens in ascending token order and score
    [E,C] their scores. Returns (idx, score, S [T,E], logits [T,E])."""
    return route_ec_logits(router_logits(x, Wg, b), cf)


def route_ec_logits(s, cf):
    """The part of ``route_ec`` after the router projection, from the logits s [T,E]
    (so that a caller holding the logits of repeated rows need not hold the rows).
    Returns (idx, score, S [T,E], logits [T,E])."""
    s = _f64(s)
    S = softmax_cols(s)
    T, E = S.shape
    C = capacity(T, E, cf)
    idx = np.empty((E, C), dtype=np.int64)
    score = np.empty((E, C), dtype=F64)
    for e in range(E):
        chosen = np.argsort(-S[:, e], kind="stable")[:C]
        chosen = np.sort(chosen)
        idx[e] = chosen
        score[e] = S[chosen, e]
    return idx, score, S, s


def ec_margin(logits, C):
    """Per expert, l_(C) - l_(C+1) on its descending logit column; +inf when C = T."""
    s = _f64(logits)
    T = s.shape[0]
    if C >= T:
        return np.full(s.shape[1], np.inf)
    ss = -np.sort(-s, axis=0)
    return ss[C - 1, :] - ss[C, :]


def mix_ec(x, idx, score, Wgate, Wup, Wdown):
    """y_t = sum over experts e that chose t of score[e,t] * E_e(x_t); tokens no
    expert chose get y_t = 0 (the dispatch mask of P3 ``ExpertChoiceGating``
    applied to the expert outputs)."""
    x = _f64(x)
    T = x.shape[0]
    E = idx.shape[0]
    y = np.zeros((T, Wdown.shape[2]), dtype=F64)
    for e in range(E):
        tt = np.asarray(idx[e])
        out = expert_ffn(x[tt], Wgate[e], Wup[e], Wdown[e])
        y[tt] += _f64(score[e])[:, None] * out
    return y


def forward_ec(x, Wg, b, Wgate, Wup, Wdown, cf):
    """Expert-choice layer forward. Returns dict with y, idx, score, probs, logits."""
    idx, score, S, s = route_ec(x, Wg, b, cf)
    y = mix_ec(x, idx, score, Wgate, Wup, Wdown)
    return {"y": y, "idx": idx, "w": score, "probs": S, "logits": s}


# --------------------------------------------------------------------------
# Token choice with an expert capacity
# --------------------------------------------------------------------------

def tc_capacity(T, E, k, cf):
    """capacity = int((T / E) * cf * k) (P5 ``expert_capacity_routing``), the
    product taken in that order in float64 as on the page."""
    return int((T / E) * cf * k)


def capacity_keep(idx, E, cap):
    """Which assignments survive an expert capacity (P5 ``expert_capacity_routing``):
    tokens are visited in order and each of a token's assignments is kept while its
    expert has taken fewer than `cap`. Returns (kept [T,k] bool, load [E])."""
    idx = np.asarray(idx)
    T, k = idx.shape
    load = np.zeros(E, dtype=np.int64)
    kept = np.zeros(idx.shape, dtype=bool)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            if load[e] < cap:
                kept[t, j] = True
                load[e] += 1
    return kept, load


def capacity_weights(p, idx, kept, renormalize=True):
    """Gate weights after the capacity: the kept slots' probabilities, divided by
    their sum over the token's kept slots (a sum of 0 is divided by 1) when
    renormalising; dropped slots weigh 0."""
    idx = np.asarray(idx, dtype=np.int64)
    g = np.where(kept, np.take_along_axis(p, idx, axis=1), 0.0)
    if renormalize:
        rows = g.sum(axis=1, keepdims=True)
        rows[rows == 0] = 1.0
        g = g / rows
    return g


def route_tc_capacity(x, Wg, b, k, cf, renormalize=True):
    """Token choice with an expert capacity (P5 ``expert_capacity_routing``).
    Each token's top-k experts (as in ``route_tc``) are visited token by token;
    an assignment is kept while its expert has taken fewer than `capacity`
    assignments, and dropped otherwise. The kept gates, divided by their sum
    over the token's kept slots (a sum of 0 is divided by 1), are the weights;
    dropped slots weigh 0. Returns (idx [T,k], w [T,k], kept [T,k], probs,
    logits, load [E]) with load the kept assignments per expert."""
    s = router_logits(x, Wg, b)
    p = softmax_rows(s)
    idx = topk_experts(p, k)
    T, E = p.shape
    cap = tc_capacity(T, E, k, cf)
    kept, load = capacity_keep(idx, E, cap)
    g = capacity_weights(p, idx, kept, renormalize)
    return idx, g, kept, p, s, load


def forward_tc_capacity(x, Wg, b, Wgate, Wup, Wdown, k, cf, renormalize=True):
    """Capacity-limited token-choice layer forward: y_t = sum over the token's
    kept slots of w * E_e(x_t) (dropped slots weigh 0). Returns dict with y,
    idx, w, kept, probs, logits, load."""
    idx, w, kept, p, s, load = route_tc_capacity(x, Wg, b, k, cf, renormalize)
    y = mix(x, idx, w, Wgate, Wup, Wdown)
    return {"y": y, "idx": idx, "w": w, "kept": kept, "probs": p, "logits": s, "load": load}


# --------------------------------------------------------------------------
# Dense mixture (used as an independent pin)
# --------------------------------------------------------------------------

def dense_mixture(x, Wg, b, Wgate, Wup, Wdown):
    """All experts run on every token, y = sum_e g_e E_e(x) (P5
    ``MixtureOfExperts.forward``)."""
    g = softmax_rows(router_logits(x, Wg, b))
    x = _f64(x)
    y = np.zeros((x.shape[0], Wdown.shape[2]), dtype=F64)
    for e in range(g.shape[1]):
        y += g[:, e:e + 1] * expert_ffn(x, Wgate[e], Wup[e], Wdown[e])
    return y
