"""Each plausible mistake planted in a copy of the oracle makes some pin fail.

The mistakes are planted on the CPU, in a private copy of the oracle's source
(text replacement, then exec into a fresh module); the real oracle is untouched.
"""
import inspect
import types

import pytest

from oracle import moe_oracle
from tests.pins import PINS

SRC = inspect.getsource(moe_oracle)

MUTANTS = {
    "no_renormalise": ("sel = sel / sel.sum(axis=1, keepdims=True)", "sel = sel"),
    "renormalise_always": ("if renormalize:\n        sel = sel / sel",
                           "if True:\n        sel = sel / sel"),
    "softmax_no_shift_wrong_axis": ("return e / e.sum(axis=1, keepdims=True)",
                                    "return e / e.sum(axis=0, keepdims=True)"),
    "topk_ascending": ("order = np.argsort(-p, axis=1, kind=\"stable\")",
                       "order = np.argsort(p, axis=1, kind=\"stable\")"),
    "ties_to_higher_index": ("order = np.argsort(-p, axis=1, kind=\"stable\")",
                             "order = (p.shape[1] - 1) - np.argsort(-p[:, ::-1], axis=1, kind=\"stable\")"),
    "silu_sign": ("return z / (1.0 + np.exp(-z))", "return z / (1.0 + np.exp(z))"),
    "silu_is_sigmoid": ("return z / (1.0 + np.exp(-z))", "return 1.0 / (1.0 + np.exp(-z))"),
    "gate_up_swapped": ("g = silu(X @ _f64(Wgate))\n    u = X @ _f64(Wup)",
                        "g = silu(X @ _f64(Wup))\n    u = X @ _f64(Wgate)"),
    "silu_on_up": ("return (g * u) @ _f64(Wdown)", "return (g * silu(u)) @ _f64(Wdown)"),
    "bias_dropped": ("s = s + _f64(b)[None, :]", "s = s"),
    "weight_wrong_slot": ("w[tt, jj][:, None] * out", "w[tt, 0][:, None] * out"),
    "f_over_Tk": ("f = c.astype(F64) / T", "f = c.astype(F64) / (T * k)"),
    "loss_missing_k": ("loss = E * np.sum((f / k) * p)", "loss = E * np.sum(f * p)"),
    "p_is_sum": ("p = probs.mean(axis=0)", "p = probs.sum(axis=0)"),
    "capacity_rounds_up": ("return int(T * cf / E)", "return -(-int(T * cf) // E)"),
    "ec_softmax_rows": ("z = s - s.max(axis=0, keepdims=True)\n    e = np.exp(z)\n    return e / e.sum(axis=0, keepdims=True)",
                        "z = s - s.max(axis=1, keepdims=True)\n    e = np.exp(z)\n    return e / e.sum(axis=1, keepdims=True)"),
    "ec_smallest_scores": ("chosen = np.argsort(-S[:, e], kind=\"stable\")[:C]",
                           "chosen = np.argsort(S[:, e], kind=\"stable\")[:C]"),
    "ec_unsorted_tokens": ("chosen = np.sort(chosen)\n", "\n"),
    "ec_score_unweighted": ("y[tt] += _f64(score[e])[:, None] * out", "y[tt] += out"),
    "margin_off_by_one": ("return ps[:, k - 1] - ps[:, k]", "return ps[:, k] - ps[:, k + 1 if k + 1 < E else k]"),
    "tc_capacity_keeps_one_more": ("if load[e] < cap:", "if load[e] <= cap:"),
    "noise_no_softplus": ("return s + softplus(_f64(x) @ _f64(Wn)) * _f64(eps)",
                          "return s + (_f64(x) @ _f64(Wn)) * _f64(eps)"),
    "noise_subtracted": ("return s + softplus(_f64(x) @ _f64(Wn)) * _f64(eps)",
                         "return s - softplus(_f64(x) @ _f64(Wn)) * _f64(eps)"),
    "noise_from_gate_weights": ("return s + softplus(_f64(x) @ _f64(Wn)) * _f64(eps)",
                                "return s + softplus(_f64(x) @ _f64(Wg)) * _f64(eps)"),
    "softplus_is_exp": ("return np.log1p(np.exp(z))", "return np.exp(z)"),
    "noise_on_probs": ("    s = noisy_logits(x, Wg, b, Wn, eps)\n    p = softmax_rows(s)",
                       "    s = noisy_logits(x, Wg, b, Wn, eps)\n    p = softmax_rows(router_logits(x, Wg, b)) + (s - router_logits(x, Wg, b))"),
    "additive_noise_dropped": ("    if Wn is None:\n        return s + _f64(eps)",
                               "    if Wn is None:\n        return s"),
    "zloss_no_square": ("return float(np.mean(lse ** 2))", "return float(np.mean(lse))"),
    "zloss_no_log": ("lse = np.log(np.exp(s).sum(axis=1))", "lse = np.exp(s).sum(axis=1)"),
    "zloss_sum_not_mean": ("return float(np.mean(lse ** 2))", "return float(np.sum(lse ** 2))"),
    "zloss_over_tokens": ("lse = np.log(np.exp(s).sum(axis=1))", "lse = np.log(np.exp(s).sum(axis=0))"),
    "zloss_max_not_lse": ("lse = np.log(np.exp(s).sum(axis=1))", "lse = s.max(axis=1)"),
    "tc_capacity_no_zero_guard": ("rows[rows == 0] = 1.0", "rows = rows"),
    "tc_capacity_dropped_keep_gate": ("g = np.where(kept, np.take_along_axis(p, idx, axis=1), 0.0)",
                                      "g = np.take_along_axis(p, idx, axis=1)"),
    "tc_capacity_truncates_factors": ("return int((T / E) * cf * k)", "return int(T / E) * int(cf * k)"),
    "dense_mixture_drops_gate": ("y += g[:, e:e + 1] * expert_ffn(x, Wgate[e], Wup[e], Wdown[e])",
                                 "y += expert_ffn(x, Wgate[e], Wup[e], Wdown[e])"),
    "dense_mixture_drops_bias": ("g = softmax_rows(router_logits(x, Wg, b))",
                                 "g = softmax_rows(router_logits(x, Wg, None))"),
    "dense_mixture_skips_last_expert": ("for e in range(g.shape[1]):",
                                        "for e in range(g.shape[1] - 1):"),
    "philox_no_key_step": ("            k0 = (k0 + PHILOX_W[0]) & 0xFFFFFFFF\n            k1 = (k1 + PHILOX_W[1]) & 0xFFFFFFFF",
                           "            pass"),
    "philox_multipliers_swapped": ("prod0 = np.uint64(PHILOX_M[0]) * c[0]",
                                   "prod0 = np.uint64(PHILOX_M[1]) * c[0]"),
    "philox_nine_rounds": ("for rnd in range(10):\n        if rnd > 0:", "for rnd in range(9):\n        if rnd > 0:"),
    "box_muller_no_minus_two": ("rad = np.sqrt(-2.0 * np.log(u[..., 2 * h]))",
                                "rad = np.sqrt(-np.log(u[..., 2 * h]))"),
    "box_muller_angle_from_radius_uniform": ("ang = 2.0 * np.pi * u[..., 2 * h + 1]",
                                             "ang = 2.0 * np.pi * u[..., 2 * h]"),
    "box_muller_half_turn": ("ang = 2.0 * np.pi * u[..., 2 * h + 1]", "ang = np.pi * u[..., 2 * h + 1]"),
    "noise_draw_ignores_offset": ("ctr[..., 2] = int(offset) & 0xFFFFFFFF", "ctr[..., 2] = 0"),
    "noise_draw_counter_runs_over_experts": ("ctr[..., 1] = q", "ctr[..., 1] = t * Q + q"),
    "tc_capacity_renorm_over_all_slots":("rows = g.sum(axis=1, keepdims=True)",
                                          "rows = np.take_along_axis(p, idx, axis=1).sum(axis=1, keepdims=True)"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) >= 1, f"mutation site for {name} not found"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(SRC.replace(old, new, 1), mod.__name__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    M = _mutant(name)
    caught = []
    for pin in PINS:
        try:
            pin(M)
        except Exception:
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"
