"""Seeded synthetic inputs for the sparse MoE layer forward.

This module is shared by the oracle's tests, the GPU parity tests and the
benchmark. It only draws random numbers and rounds them to the storage type;
it holds none of the layer's arithmetic.

Recipe (the same for every workload):
  * one ``numpy.random.SeedSequence(seed)`` per workload, ``seed = (42, i)`` with
    ``i`` its place (1-5) in the list below (42 is the seed both NumPy pages use), spawned into six child streams in the order
    x, W_g, b, W_gate, W_up, W_down;
  * each tensor is ``standard_normal(dtype=float32)`` times its standard
    deviation; expert stacks are drawn expert by expert, one ``[rows, cols]``
    block per expert, from that tensor's stream;
  * bf16 workloads round every activation and weight to bfloat16
    (round-to-nearest-even) and keep the rounded values in float32 arrays, so
    that ``float32 -> bfloat16`` on the device and ``float32 -> float64`` in the
    oracle are both exact. The router bias stays float32.

The five fixed workloads (``WORKLOADS``, by name) take their layer shapes from
the pages: the NumPy demo of "Mixture of Experts（MoE）の理論と実装"
(``TINY_FP32``), the ``MoEConfig`` of "Sparse Mixture of Experts(MoE) 아키텍처
심층 분석" (``MID_BF16``), the Mixtral 8x7B dictionary of "机器学习基础系列——混合
专家模型" (``MIXTRAL_LAYER``), the 64 fine-grained sub-experts with top-4 of
"細粒度専門家分割がもたらす訓練コスト削減" (``FINE_GRAINED``), and the
``ExpertChoiceGating`` of the Korean page (``EXPERT_CHOICE``).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    """One MoE layer workload: shapes, routing mode and input distributions."""

    name: str
    dtype: str                 # "fp32" or "bf16": storage type of x and all weights
    T: int                     # tokens
    d: int                     # d_model
    f: int                     # d_ff per expert
    E: int                     # experts
    k: int = 2                 # top-k (token choice)
    mode: str = "tc"           # "tc" token choice, "ec" expert choice,
                               # "tc_capacity" token choice with an expert capacity
    cf: float = 1.0            # capacity factor (expert choice, token choice with capacity)
    renormalize: bool = True   # renormalise the selected top-k weights
    x_std: float = 1.0
    wg_std: float = 0.02
    bias_std: Optional[float] = None
    w_std: float = 0.02
    seed: tuple = field(default=(42, 0))

    @property
    def capacity(self) -> int:
        """floor(T * cf / E): tokens each expert takes in expert-choice mode."""
        return int(self.T * self.cf / self.E)

    @property
    def rows(self) -> int:
        """Rows the dispatch lays out: T*k (token choice; with a capacity, the kept
        rows are a prefix of them) or E*C (expert choice)."""
        return self.E * self.capacity if self.mode == "ec" else self.T * self.k


TINY_FP32 = Workload("tiny_top2_fp32", "fp32", T=256, d=64, f=128, E=8, k=2,
                     x_std=0.5, wg_std=0.1, w_std=0.02, seed=(42, 1))
MID_BF16 = Workload("mid_top2_bf16", "bf16", T=4096, d=1024, f=4096, E=8, k=2,
                    x_std=1.0, wg_std=0.02, w_std=0.02, seed=(42, 2))
MIXTRAL_LAYER = Workload("mixtral_layer_skewed_top2_bf16", "bf16", T=16384, d=4096, f=14336,
                         E=8, k=2, x_std=1.0, wg_std=0.02, bias_std=1.0, w_std=0.01,
                         seed=(42, 3))
FINE_GRAINED = Workload("fine_grained_e64_top4_bf16", "bf16", T=8192, d=2048, f=1408, E=64, k=4,
                        x_std=1.0, wg_std=0.02, w_std=0.02, seed=(42, 4))
EXPERT_CHOICE = Workload("expert_choice_e16_cf1_bf16", "bf16", T=8192, d=1024, f=4096, E=16, k=1,
                         mode="ec", cf=1.0, x_std=1.0, wg_std=0.02, w_std=0.02, seed=(42, 5))

WORKLOADS = {w.name: w for w in (TINY_FP32, MID_BF16, MIXTRAL_LAYER, FINE_GRAINED, EXPERT_CHOICE)}


def custom(name: str = "custom", **kw) -> Workload:
    """A workload outside the five fixed ones (edge cases, small parity cases)."""
    base = dict(dtype="bf16", T=64, d=64, f=64, E=4, k=2)
    base.update(kw)
    return Workload(name, **base)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    r = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _draw(rng: np.random.Generator, shape, std: float, bf16: bool) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    a *= np.float32(std)
    return round_bf16(a) if bf16 else a


def _stack(rng: np.random.Generator, E: int, shape, std: float, bf16: bool) -> np.ndarray:
    out = np.empty((E,) + tuple(shape), dtype=np.float32)
    for e in range(E):
        out[e] = _draw(rng, shape, std, bf16)
    return out


def make_inputs(w: Workload, experts: bool = True) -> dict:
    """Draw the workload's inputs as float32 NumPy arrays.

    Returns ``x [T,d]``, ``Wg [d,E]``, ``b [E]`` (or None), and when ``experts``
    is true ``Wgate [E,d,f]``, ``Wup [E,d,f]``, ``Wdown [E,f,d]``.
    """
    ss = np.random.SeedSequence(list(w.seed))
    kids = ss.spawn(6)
    rngs = [np.random.default_rng(s) for s in kids]
    bf = w.dtype == "bf16"
    jobs = {
        "x": lambda: _draw(rngs[0], (w.T, w.d), w.x_std, bf),
        "Wg": lambda: _draw(rngs[1], (w.d, w.E), w.wg_std, bf),
        "b": lambda: (rngs[2].standard_normal(w.E, dtype=np.float32) * np.float32(w.bias_std)
                      if w.bias_std is not None else None),
    }
    if experts:
        jobs["Wgate"] = lambda: _stack(rngs[3], w.E, (w.d, w.f), w.w_std, bf)
        jobs["Wup"] = lambda: _stack(rngs[4], w.E, (w.d, w.f), w.w_std, bf)
        jobs["Wdown"] = lambda: _stack(rngs[5], w.E, (w.f, w.d), w.w_std, bf)
    # each tensor has its own stream, so drawing them concurrently changes nothing
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        futs = {k: ex.submit(fn) for k, fn in jobs.items()}
        return {k: f.result() for k, f in futs.items()}


def make_noise(w: Workload, wn_std: Optional[float] = 0.02, eps_scale: float = 1.0) -> dict:
    """Training-noise inputs of a workload: ``Wn [d,E]`` (the noise projection, drawn
    like W_g and rounded like it; None when ``wn_std`` is None) and ``eps [T,E]``, a
    standard normal draw times ``eps_scale`` (float32). Streams: the workload's seed
    with a trailing 1, spawned into two (Wn, eps), so the layer's own inputs are the
    same with or without noise."""
    kids = np.random.SeedSequence(list(w.seed) + [1]).spawn(2)
    r_wn, r_eps = (np.random.default_rng(k) for k in kids)
    Wn = _draw(r_wn, (w.d, w.E), wn_std, w.dtype == "bf16") if wn_std is not None else None
    eps = r_eps.standard_normal((w.T, w.E), dtype=np.float32) * np.float32(eps_scale)
    return {"Wn": Wn, "eps": eps}


def with_seed(w: Workload, seed) -> Workload:
    return replace(w, seed=tuple(seed))
