"""Brute-force MoE forward for tiny inputs (T <= 8), pure Python loops.

TEST INFRASTRUCTURE ONLY (see ``oracle/moe_oracle.py``): used to pin the
vectorised oracle. It imports nothing from the HIP library nor from the
vectorised oracle.

Differences from the vectorised oracle, on purpose:
  * every dot product is an explicit Python loop over scalars;
  * the top-k set is found by enumerating all C(E,k) expert subsets and keeping
    the one of largest total probability (the set maximising sum g_i is the
    top-k set of P2's ``TopK(g)`` equation); among equal totals the
    lexicographically smallest index tuple wins, which is the lower-index tie
    rule;
  * expert choice enumerates all C-subsets of tokens per expert the same way.

Pages cited by title as in ``oracle/moe_oracle.py``.
"""
from __future__ import annotations

import itertools
import math


def _dot_col(row, M, col):
    acc = 0.0
    for i in range(len(row)):
        acc += float(row[i]) * float(M[i][col])
    return acc


def _vecmat(row, M):
    return [_dot_col(row, M, j) for j in range(len(M[0]))]


def _softmax(v):
    m = max(v)
    ex = [math.exp(a - m) for a in v]
    s = 0.0
    for a in ex:
        s += a
    return [a / s for a in ex]


def _silu(z):
    # z / (1 + e^-z), written to avoid overflow for very negative z
    if z >= 0:
        return z / (1.0 + math.exp(-z))
    ez = math.exp(z)
    return z * ez / (ez + 1.0)


def expert(xrow, Wgate, Wup, Wdown):
    """(silu(x W_gate) * (x W_up)) W_down, P1 ``Expert.forward``."""
    g = _vecmat(xrow, Wgate)
    u = _vecmat(xrow, Wup)
    h = [_silu(g[i]) * u[i] for i in range(len(g))]
    return _vecmat(h, Wdown)


def _best_subset(values, size):
    """Subset of ``size`` positions maximising the sum of ``values``; the sum is
    taken over the values in ascending order so that equal multisets give equal
    sums; ties go to the lexicographically smallest position tuple."""
    best, best_sum = None, -math.inf
    for comb in itertools.combinations(range(len(values)), size):
        s = 0.0
        for v in sorted(values[i] for i in comb):
            s += v
        if s > best_sum:
            best, best_sum = comb, s
    return list(best)


def forward_tc(x, Wg, b, Wgate, Wup, Wdown, k, renormalize=True, Wn=None, eps=None):
    """Token-choice forward by literal loops. Returns dict(y, idx, w, probs).
    With eps, the training noise of P3 ``TopKGating`` is added to each logit:
    log(1 + e^z) * eps with z = x W_noise, or eps alone when Wn is None."""
    T, E = len(x), len(Wg[0])
    ys, idxs, ws, ps = [], [], [], []
    for t in range(T):
        s = _vecmat(x[t], Wg)
        if b is not None:
            s = [s[e] + float(b[e]) for e in range(E)]
        if eps is not None:
            zn = _vecmat(x[t], Wn) if Wn is not None else None
            for e in range(E):
                scale = math.log(1.0 + math.exp(zn[e])) if zn is not None else 1.0
                s[e] = s[e] + scale * float(eps[t][e])
        p = _softmax(s)
        chosen = _best_subset(p, k)
        # slot order: descending probability, lower index first on ties
        chosen.sort(key=lambda e: (-p[e], e))
        wsel = [p[e] for e in chosen]
        if renormalize:
            tot = 0.0
            for v in wsel:
                tot += v
            wsel = [v / tot for v in wsel]
        y = [0.0] * len(Wdown[0][0])
        for j, e in enumerate(chosen):
            out = expert(x[t], Wgate[e], Wup[e], Wdown[e])
            for c in range(len(y)):
                y[c] += wsel[j] * out[c]
        ys.append(y)
        idxs.append(chosen)
        ws.append(wsel)
        ps.append(p)
    return {"y": ys, "idx": idxs, "w": ws, "probs": ps}


def forward_ec(x, Wg, b, Wgate, Wup, Wdown, cf):
    """Expert-choice forward by literal loops. Returns dict(y, idx, w)."""
    T, E = len(x), len(Wg[0])
    C = int(T * cf / E)
    logits = []
    for t in range(T):
        s = _vecmat(x[t], Wg)
        if b is not None:
            s = [s[e] + float(b[e]) for e in range(E)]
        logits.append(s)
    idx, score = [], []
    ys = [[0.0] * len(Wdown[0][0]) for _ in range(T)]
    for e in range(E):
        col = _softmax([logits[t][e] for t in range(T)])
        chosen = sorted(_best_subset(col, C))
        idx.append(chosen)
        score.append([col[t] for t in chosen])
        for t in chosen:
            out = expert(x[t], Wgate[e], Wup[e], Wdown[e])
            for c in range(len(out)):
                ys[t][c] += col[t] * out[c]
    return {"y": ys, "idx": idx, "w": score}


def forward_tc_capacity(x, Wg, b, Wgate, Wup, Wdown, k, cf, renormalize=True):
    """Capacity-limited token choice by literal loops (P5
    ``expert_capacity_routing``): a running count per expert, tokens in order,
    an assignment kept while its expert's count is below int((T / E) * cf * k).
    Returns dict(y, idx, w, kept, load)."""
    T, E = len(x), len(Wg[0])
    cap = int((T / E) * cf * k)
    load = [0] * E
    ys, idxs, ws, kepts = [], [], [], []
    for t in range(T):
        s = _vecmat(x[t], Wg)
        if b is not None:
            s = [s[e] + float(b[e]) for e in range(E)]
        p = _softmax(s)
        chosen = _best_subset(p, k)
        chosen.sort(key=lambda e: (-p[e], e))
        keep = []
        for e in chosen:
            if load[e] < cap:
                load[e] += 1
                keep.append(True)
            else:
                keep.append(False)
        wsel = [p[e] if kp else 0.0 for e, kp in zip(chosen, keep)]
        if renormalize:
            tot = 0.0
            for v in wsel:
                tot += v
            if tot > 0.0:
                wsel = [v / tot for v in wsel]
        y = [0.0] * len(Wdown[0][0])
        for j, e in enumerate(chosen):
            if not keep[j]:
                continue
            out = expert(x[t], Wgate[e], Wup[e], Wdown[e])
            for c in range(len(y)):
                y[c] += wsel[j] * out[c]
        ys.append(y)
        idxs.append(chosen)
        ws.append(wsel)
        kepts.append(keep)
    return {"y": ys, "idx": idxs, "w": ws, "kept": kepts, "load": load}



def router_z_loss(x, Wg, b):
    """Mean over tokens of (log sum_e exp(s_te))^2 with s = x W_g (+ b), token by
    token with scalar exp and log (P3 ``router_z_loss``)."""
    T = len(x)
    if T == 0:
        return 0.0
    acc = 0.0
    for t in range(T):
        s = _vecmat(x[t], Wg)
        if b is not None:
            s = [s[e] + float(b[e]) for e in range(len(s))]
        z = 0.0
        for v in s:
            z += math.exp(v)
        lz = math.log(z)
        acc += lz * lz
    return acc / T


def noise_draw_one(t, e, seed, offset=0):
    """One element of the in-kernel training-noise draw, evaluated with Python
    integers and the math module: Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
    SC 2011) of counter (t, e // 4, low and high 32 bits of offset) under key (low and
    high 32 bits of seed), the 24-bit uniforms u = (r >> 8 + 1/2) / 2^24 of its four
    words, and the Box-Muller transform (Box and Muller, 1958) of the pair that
    expert e falls in: cosine for even e, sine for odd e."""
    m32 = (1 << 32) - 1
    c = [t & m32, e // 4, offset & m32, (offset >> 32) & m32]
    k0, k1 = seed & m32, (seed >> 32) & m32
    for rnd in range(10):
        if rnd:
            k0 = (k0 + 0x9E3779B9) & m32
            k1 = (k1 + 0xBB67AE85) & m32
        a = 0xD2511F53 * c[0]
        b = 0xCD9E8D57 * c[2]
        c = [((b >> 32) ^ c[1] ^ k0) & m32, b & m32, ((a >> 32) ^ c[3] ^ k1) & m32, a & m32]
    j = e % 4
    pair = j // 2
    u0 = ((c[2 * pair] >> 8) + 0.5) / float(1 << 24)
    u1 = ((c[2 * pair + 1] >> 8) + 0.5) / float(1 << 24)
    r = math.sqrt(-2.0 * math.log(u0))
    return r * (math.cos(2.0 * math.pi * u1) if j % 2 == 0 else math.sin(2.0 * math.pi * u1))
