"""The Python binding checks every tensor's full shape before anything reaches the C ABI
(which sees only raw pointers, so an undersized tensor would be read or written out of
bounds on the device). Runs on the CPU: the shape checks come before the device checks,
so CPU tensors with a wrong shape raise ValueError, and CPU tensors of the right shape
raise TypeError (not a device tensor); nothing is launched either way."""
import pytest
import torch

import sparse_mixture_experts_sum_amd as M

T, d, f, E, k = 10, 64, 128, 4, 2


def _layer(**over):
    t = dict(
        x=torch.zeros(T, d, dtype=torch.bfloat16),
        W_g=torch.zeros(d, E, dtype=torch.bfloat16),
        b_g=torch.zeros(E),
        W_gate=torch.zeros(E, d, f, dtype=torch.bfloat16),
        W_up=torch.zeros(E, d, f, dtype=torch.bfloat16),
        W_down=torch.zeros(E, f, d, dtype=torch.bfloat16),
    )
    t.update(over)
    return t


def _forward(t, **kw):
    return M.moe_forward(t["x"], t["W_g"], t["b_g"], t["W_gate"], t["W_up"], t["W_down"], k=k,
                         **kw)


BAD_FORWARD = {
    "W_g_rows": dict(W_g=torch.zeros(d - 8, E, dtype=torch.bfloat16)),
    "W_g_cols": dict(W_g=torch.zeros(d, E - 1, dtype=torch.bfloat16)),
    "b_g": dict(b_g=torch.zeros(E - 1)),
    "W_gate_d": dict(W_gate=torch.zeros(E, d - 64, f, dtype=torch.bfloat16)),
    "W_up_f": dict(W_up=torch.zeros(E, d, f - 64, dtype=torch.bfloat16)),
    "W_up_E": dict(W_up=torch.zeros(E - 1, d, f, dtype=torch.bfloat16)),
    "W_down": dict(W_down=torch.zeros(E, f, d - 64, dtype=torch.bfloat16)),
    "W_down_T": dict(W_down=torch.zeros(E, d, f, dtype=torch.bfloat16)),
    "x_3d": dict(x=torch.zeros(1, T, d, dtype=torch.bfloat16)),
}


@pytest.mark.parametrize("name", sorted(BAD_FORWARD))
def test_forward_rejects_undersized_tensors(name):
    with pytest.raises(ValueError):
        _forward(_layer(**BAD_FORWARD[name]))


def test_forward_rejects_wrong_y_and_noise():
    t = _layer()
    with pytest.raises(ValueError):
        _forward(t, y=torch.zeros(T - 1, d))
    with pytest.raises(ValueError):
        _forward(t, eps=torch.zeros(T, E - 1))
    with pytest.raises(ValueError):
        _forward(t, eps=torch.zeros(T, E), W_noise=torch.zeros(d, E - 1, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        _forward(t, W_noise=torch.zeros(d, E, dtype=torch.bfloat16))  # no draw


def test_route_rejects_undersized_tensors():
    t = _layer()
    with pytest.raises(ValueError):
        M.moe_route(t["x"], torch.zeros(d - 8, E, dtype=torch.bfloat16), None, k=k)
    with pytest.raises(ValueError):
        M.moe_route(t["x"], t["W_g"], torch.zeros(E + 1), k=k)
    with pytest.raises(ValueError):
        M.moe_route(t["x"], t["W_g"], None, k=k, eps=torch.zeros(T + 1, E))
    with pytest.raises(ValueError):
        M.moe_route(t["x"], t["W_g"], None, k=k, eps=torch.zeros(T, E),
                    W_noise=torch.zeros(d, E + 1, dtype=torch.bfloat16))


def test_aux_loss_rejects_mismatched_idx():
    with pytest.raises(ValueError):
        M.moe_aux_loss(torch.zeros(T, E), torch.zeros(T - 1, k, dtype=torch.int32))
    with pytest.raises(ValueError):
        M.moe_aux_loss(torch.zeros(T, E), torch.zeros(T * k, dtype=torch.int32))


def test_right_shapes_on_the_cpu_are_refused_as_host_tensors():
    # shapes pass; the device check then refuses host memory before any library call
    with pytest.raises(TypeError):
        _forward(_layer())
    t = _layer()
    with pytest.raises(TypeError):
        M.moe_route(t["x"], t["W_g"], t["b_g"], k=k)
    with pytest.raises(TypeError):
        M.moe_aux_loss(torch.zeros(T, E), torch.zeros(T, k, dtype=torch.int32))


def test_noise_draw_arguments():
    # the in-kernel draw: seed and offset are 64-bit unsigned; W_noise still checked
    with pytest.raises(ValueError):
        M.NoiseDraw(-1)
    with pytest.raises(ValueError):
        M.NoiseDraw(1, offset=1 << 64)
    t = _layer()
    with pytest.raises(ValueError):
        _forward(t, eps=M.NoiseDraw(3), W_noise=torch.zeros(d, E - 1, dtype=torch.bfloat16))
    with pytest.raises(TypeError):  # right shapes, host tensors
        _forward(t, eps=M.NoiseDraw(3, 4, 0.5), W_noise=torch.zeros(d, E, dtype=torch.bfloat16))
