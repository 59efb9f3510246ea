"""MI355X (gfx950) sparse Mixture-of-Experts layer forward.

A thin ctypes binding over the C ABI in ``include/moe.h`` (``libmoe_hip.so``, built
in-tree by ``python -m sparse_mixture_experts_sum_amd.build``). Every step of the
layer runs in the library's HIP kernels; this module only checks tensor
metadata, allocates outputs and the workspace with torch (device memory), and
passes pointers and the current HIP stream. There is no fallback: if the library
is missing, importing the binding's functions raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "moe_route", "moe_forward", "moe_forward_noalloc", "moe_aux_loss", "NoiseDraw", "make_shape",
    "workspace_size", "capacity",
    "workspace_offset", "profile_enable", "profile_read", "stage_names", "SparseMoE",
    "MoEError", "load_library", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_hip.so")

MOE_FP32, MOE_BF16 = 0, 1
MOE_TOKEN_CHOICE, MOE_EXPERT_CHOICE, MOE_TOKEN_CHOICE_CAPACITY = 0, 1, 2
# mode names: token choice, expert choice, token choice with an expert capacity
MODES = {"tc": MOE_TOKEN_CHOICE, "ec": MOE_EXPERT_CHOICE, "tc_capacity": MOE_TOKEN_CHOICE_CAPACITY}
NUM_STAGES = 8
WS_OFFSETS, WS_POS, WS_SRC, WS_XPERM, WS_H, WS_O = range(6)

# every symbol include/moe.h declares
EXPORTS = (
    "moe_status_string", "moe_capacity", "moe_workspace_size", "moe_workspace_offset",
    "moe_route", "moe_forward", "moe_aux_loss", "moe_profile_enable", "moe_profile_read",
    "moe_stage_name", "moe_forward_noalloc",
)


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: status {status} ({msg})")
        self.status = status


class MoeShape(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64),
        ("d_model", ctypes.c_int64),
        ("d_ff", ctypes.c_int64),
        ("E", ctypes.c_int32),
        ("k", ctypes.c_int32),
        ("mode", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("renormalize", ctypes.c_int32),
        ("capacity_factor", ctypes.c_double),
    ]


class MoeNoise(ctypes.Structure):
    _fields_ = [("W_noise", ctypes.c_void_p), ("eps", ctypes.c_void_p), ("seed", ctypes.c_uint64),
                ("offset", ctypes.c_uint64), ("scale", ctypes.c_float)]


class NoiseDraw:
    """Pass as ``eps`` to have the router kernel draw the training noise itself:
    eps[t, e] = scale * n(t, e) with n the counter-based normal draw of (seed, offset)
    that include/moe.h defines (Philox4x32-10 and the Box-Muller transform). A new draw
    per training step takes a new offset."""

    def __init__(self, seed: int, offset: int = 0, scale: float = 1.0):
        if not (0 <= int(seed) < 1 << 64 and 0 <= int(offset) < 1 << 64):
            raise ValueError("seed and offset must fit in 64 unsigned bits")
        self.seed, self.offset, self.scale = int(seed), int(offset), float(scale)

    def __repr__(self):
        return f"NoiseDraw(seed={self.seed}, offset={self.offset}, scale={self.scale})"


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmoe_hip.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} not found: build it with `python -m sparse_mixture_experts_sum_amd.build`")
    lib = ctypes.CDLL(path)
    P, S, I32, I64, F = ctypes.c_void_p, ctypes.POINTER(MoeShape), ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [I32]
    lib.moe_stage_name.restype = ctypes.c_char_p
    lib.moe_stage_name.argtypes = [I32]
    lib.moe_capacity.argtypes = [S, ctypes.POINTER(I64)]
    lib.moe_workspace_size.argtypes = [S, ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_workspace_offset.argtypes = [S, I32, ctypes.POINTER(ctypes.c_size_t)]
    N = ctypes.POINTER(MoeNoise)
    lib.moe_route.argtypes = [S, P, P, P, N, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.moe_forward.argtypes = [S, P, P, P, N, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                ctypes.c_size_t, P]
    lib.moe_aux_loss.argtypes = [S, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.moe_forward_noalloc.argtypes = [S, P, P, P, N, P, P, P, P, P, P, P, P, P, P, P, P, P]
    lib.moe_profile_enable.argtypes = [I32]
    lib.moe_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I64), I32]
    for name in ("moe_capacity", "moe_workspace_size", "moe_workspace_offset", "moe_route",
                 "moe_forward", "moe_forward_noalloc", "moe_aux_loss", "moe_profile_enable",
                 "moe_profile_read"):
        getattr(lib, name).restype = I32
    _lib = lib
    return lib


def _check(fn: str, st: int):
    if st != 0:
        msg = load_library().moe_status_string(st).decode()
        raise MoEError(fn, st, msg)


def make_shape(T, d_model, d_ff, E, k=2, mode="tc", dtype="bf16", renormalize=True,
               capacity_factor=1.0) -> MoeShape:
    if mode not in MODES:
        raise ValueError(f"mode must be one of {sorted(MODES)}, got {mode!r}")
    return MoeShape(T=int(T), d_model=int(d_model), d_ff=int(d_ff), E=int(E), k=int(k),
                    mode=MODES[mode],
                    dtype=MOE_BF16 if dtype in ("bf16", torch.bfloat16) else MOE_FP32,
                    renormalize=1 if renormalize else 0,
                    capacity_factor=float(capacity_factor))


def workspace_size(shape: MoeShape) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_workspace_size", load_library().moe_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def workspace_offset(shape: MoeShape, which: int) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_workspace_offset",
           load_library().moe_workspace_offset(ctypes.byref(shape), int(which), ctypes.byref(n)))
    return n.value


def capacity(shape: MoeShape) -> int:
    c = ctypes.c_int64(0)
    _check("moe_capacity", load_library().moe_capacity(ctypes.byref(shape), ctypes.byref(c)))
    return c.value


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dtype_name(t: torch.Tensor) -> str:
    if t.dtype == torch.bfloat16:
        return "bf16"
    if t.dtype == torch.float32:
        return "fp32"
    raise TypeError(f"unsupported dtype {t.dtype}: x and weights must be bfloat16 or float32")


def _shape_is(t, name, shape):
    """Full shape check, before anything reaches the library: the C ABI sees only raw
    pointers, so an undersized tensor would be read or written out of bounds on the
    device."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _need(t, name, dtype=None, dev=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")


def _x_shape(x):
    if not isinstance(x, torch.Tensor):
        raise TypeError("x must be a tensor")
    if x.dim() != 2:
        raise ValueError(f"x must be [T, d_model], got shape {tuple(x.shape)}")
    return x.shape


def _noise_shapes(T, d, E, W_noise, eps):
    if eps is None:
        if W_noise is not None:
            raise ValueError("W_noise needs eps, the normal draw (a tensor or a NoiseDraw)")
        return
    if not isinstance(eps, NoiseDraw):
        _shape_is(eps, "eps", (T, E))
    _shape_is(W_noise, "W_noise", (d, E))


def _noise(x, W_noise, eps, dev):
    """moe_noise for training noise: eps [T,E] fp32 or a NoiseDraw (required for any
    noise) and optionally W_noise [d,E] of x's dtype; None when eps is None. Shapes are
    checked by _noise_shapes first."""
    if eps is None:
        return None
    _need(W_noise, "W_noise", x.dtype, dev)
    wn = None if W_noise is None else W_noise.data_ptr()
    if isinstance(eps, NoiseDraw):
        return ctypes.byref(MoeNoise(W_noise=wn, eps=None, seed=eps.seed, offset=eps.offset,
                                     scale=eps.scale))
    _need(eps, "eps", torch.float32, dev)
    return ctypes.byref(MoeNoise(W_noise=wn, eps=eps.data_ptr()))


def _workspace(shape: MoeShape, dev, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    n = workspace_size(shape)
    if workspace is not None:
        _need(workspace, "workspace", dev=dev)
        if workspace.numel() * workspace.element_size() >= n:
            return workspace
    return torch.empty(max(n, 16), dtype=torch.uint8, device=dev)


def moe_route(x, W_g, b_g=None, *, k=2, mode="tc", capacity_factor=1.0, renormalize=True,
              want_probs=True, want_counts=True, want_z_loss=False, W_noise=None, eps=None,
              workspace=None) -> dict:
    """Router only. Token choice (with or without capacity) returns idx/w [T,k];
    expert choice idx/w [E,C]. want_z_loss adds the router z-loss (fp32 [1]); eps
    (and W_noise) add the training noise of noisy top-k gating: eps an fp32 [T,E] draw,
    or a NoiseDraw for the router kernel to draw it."""
    T, d = _x_shape(x)
    if not isinstance(W_g, torch.Tensor) or W_g.dim() != 2:
        raise ValueError("W_g must be [d_model, E]")
    E = W_g.shape[1]
    _shape_is(W_g, "W_g", (d, E))
    _shape_is(b_g, "b_g", (E,))
    _noise_shapes(T, d, E, W_noise, eps)
    dev = x.device
    dt = x.dtype
    _need(x, "x", dev=dev)
    _need(W_g, "W_g", dt, dev)
    _need(b_g, "b_g", torch.float32, dev)
    shape = make_shape(T, d, 64, E, k, mode, _dtype_name(x), renormalize, capacity_factor)
    ws = _workspace(shape, dev, workspace)
    if mode != "ec":
        idx = torch.empty(T, k, dtype=torch.int32, device=dev)
        w = torch.empty(T, k, dtype=torch.float32, device=dev)
    else:
        C = capacity(shape)
        idx = torch.empty(E, C, dtype=torch.int32, device=dev)
        w = torch.empty(E, C, dtype=torch.float32, device=dev)
    probs = torch.empty(T, E, dtype=torch.float32, device=dev) if want_probs else None
    counts = torch.empty(E, dtype=torch.int32, device=dev) if want_counts else None
    z = torch.empty(1, dtype=torch.float32, device=dev) if want_z_loss else None
    noise = _noise(x, W_noise, eps, dev)
    _check("moe_route", load_library().moe_route(
        ctypes.byref(shape), _ptr(x), _ptr(W_g), _ptr(b_g), noise, _ptr(idx), _ptr(w), _ptr(probs),
        _ptr(counts), _ptr(z), _ptr(ws), ws.numel(), _stream(dev)))
    return {"idx": idx, "w": w, "probs": probs, "counts": counts, "z_loss": z}


def moe_forward(x, W_g, b_g, W_gate, W_up, W_down, *, k=2, mode="tc", capacity_factor=1.0,
                renormalize=True, want_routing=True, want_probs=True, want_stats=True,
                want_z_loss=False, W_noise=None, eps=None, workspace=None, y=None) -> dict:
    """Whole layer forward. Returns y (fp32 [T,d]) and, on request, idx, w, probs,
    counts, (token choice) f, p, loss, and the router z-loss. eps (and W_noise) add
    the training noise of noisy top-k gating: eps an fp32 [T,E] draw, or a NoiseDraw
    for the router kernel to draw it."""
    return _forward(x, W_g, b_g, W_gate, W_up, W_down, k, mode, capacity_factor, renormalize,
                    want_routing, want_probs, want_stats, want_z_loss, W_noise, eps, workspace, y,
                    noalloc=False)


def moe_forward_noalloc(x, W_g, b_g, W_gate, W_up, W_down, *, k=2, mode="tc",
                        capacity_factor=1.0, renormalize=True, want_routing=True, want_probs=True,
                        want_stats=True, want_z_loss=False, W_noise=None, eps=None,
                        y=None) -> dict:
    """moe_forward through the library's allocation-free entry point: its workspace is the
    library's own fixed device array (NOALLOC_SCRATCH_BYTES per GPU), which every such
    call on a GPU shares (overlapping calls race). The outputs requested here are still
    allocated by torch unless passed in (y); the library call itself allocates nothing."""
    return _forward(x, W_g, b_g, W_gate, W_up, W_down, k, mode, capacity_factor, renormalize,
                    want_routing, want_probs, want_stats, want_z_loss, W_noise, eps, None, y,
                    noalloc=True)


NOALLOC_SCRATCH_BYTES = 256 << 20  # MOE_NOALLOC_SCRATCH_BYTES of include/moe.h


def _forward(x, W_g, b_g, W_gate, W_up, W_down, k, mode, capacity_factor, renormalize,
             want_routing, want_probs, want_stats, want_z_loss, W_noise, eps, workspace, y,
             noalloc):
    T, d = _x_shape(x)
    if not isinstance(W_gate, torch.Tensor) or W_gate.dim() != 3:
        raise ValueError("W_gate must be [E, d_model, d_ff]")
    E, _, f = W_gate.shape
    _shape_is(W_gate, "W_gate", (E, d, f))
    _shape_is(W_up, "W_up", (E, d, f))
    _shape_is(W_down, "W_down", (E, f, d))
    _shape_is(W_g, "W_g", (d, E))
    _shape_is(b_g, "b_g", (E,))
    _shape_is(y, "y", (T, d))
    _noise_shapes(T, d, E, W_noise, eps)
    dev = x.device
    dt = x.dtype
    _need(x, "x", dev=dev)
    for t, nm in ((W_g, "W_g"), (W_gate, "W_gate"), (W_up, "W_up"), (W_down, "W_down")):
        _need(t, nm, dt, dev)
    _need(b_g, "b_g", torch.float32, dev)
    _need(y, "y", torch.float32, dev)
    shape = make_shape(T, d, f, E, k, mode, _dtype_name(x), renormalize, capacity_factor)
    ws = None if noalloc else _workspace(shape, dev, workspace)
    if y is None:
        y = torch.empty(T, d, dtype=torch.float32, device=dev)
    idx = w = probs = counts = fo = po = lo = None
    if want_routing:
        if mode != "ec":
            idx = torch.empty(T, k, dtype=torch.int32, device=dev)
            w = torch.empty(T, k, dtype=torch.float32, device=dev)
        else:
            C = capacity(shape)
            idx = torch.empty(E, C, dtype=torch.int32, device=dev)
            w = torch.empty(E, C, dtype=torch.float32, device=dev)
        counts = torch.empty(E, dtype=torch.int32, device=dev)
    if want_probs:
        probs = torch.empty(T, E, dtype=torch.float32, device=dev)
    if want_stats and mode != "ec":
        fo = torch.empty(E, dtype=torch.float32, device=dev)
        po = torch.empty(E, dtype=torch.float32, device=dev)
        lo = torch.empty(1, dtype=torch.float32, device=dev)
    z = torch.empty(1, dtype=torch.float32, device=dev) if want_z_loss else None
    noise = _noise(x, W_noise, eps, dev)
    lib = load_library()
    if noalloc:
        _check("moe_forward_noalloc", lib.moe_forward_noalloc(
            ctypes.byref(shape), _ptr(x), _ptr(W_g), _ptr(b_g), noise, _ptr(W_gate), _ptr(W_up),
            _ptr(W_down), _ptr(y), _ptr(idx), _ptr(w), _ptr(probs), _ptr(counts), _ptr(fo),
            _ptr(po), _ptr(lo), _ptr(z), _stream(dev)))
    else:
        _check("moe_forward", lib.moe_forward(
            ctypes.byref(shape), _ptr(x), _ptr(W_g), _ptr(b_g), noise, _ptr(W_gate), _ptr(W_up),
            _ptr(W_down),
            _ptr(y), _ptr(idx), _ptr(w), _ptr(probs), _ptr(counts), _ptr(fo), _ptr(po), _ptr(lo),
            _ptr(z), _ptr(ws), ws.numel(), _stream(dev)))
    return {"y": y, "idx": idx, "w": w, "probs": probs, "counts": counts, "f": fo, "p": po,
            "loss": lo, "z_loss": z, "workspace": ws, "shape": shape}


def moe_aux_loss(probs, idx, *, workspace=None) -> dict:
    """f, p, loss and counts from router outputs probs [T,E] and idx [T,k] (token choice)."""
    if not isinstance(probs, torch.Tensor) or probs.dim() != 2:
        raise ValueError("probs must be [T, E]")
    if not isinstance(idx, torch.Tensor) or idx.dim() != 2:
        raise ValueError("idx must be [T, k]")
    T, E = probs.shape
    k = idx.shape[1]
    _shape_is(idx, "idx", (T, k))
    dev = probs.device
    _need(probs, "probs", torch.float32, dev)
    _need(idx, "idx", torch.int32, dev)
    shape = make_shape(T, 64, 64, E, k, "tc", "fp32")
    ws = _workspace(shape, dev, workspace)
    f = torch.empty(E, dtype=torch.float32, device=dev)
    p = torch.empty(E, dtype=torch.float32, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    _check("moe_aux_loss", load_library().moe_aux_loss(
        ctypes.byref(shape), _ptr(probs), _ptr(idx), _ptr(f), _ptr(p), _ptr(loss), _ptr(counts),
        _ptr(ws), ws.numel(), _stream(dev)))
    return {"f": f, "p": p, "loss": loss, "counts": counts}


def profile_enable(on: bool = True):
    _check("moe_profile_enable", load_library().moe_profile_enable(1 if on else 0))


def stage_names():
    lib = load_library()
    return [lib.moe_stage_name(i).decode() for i in range(NUM_STAGES)]


def profile_read() -> dict:
    """Per-stage totals since the last read: {stage: (total_ms, launches)}."""
    ms = (ctypes.c_double * NUM_STAGES)()
    n = (ctypes.c_int64 * NUM_STAGES)()
    _check("moe_profile_read", load_library().moe_profile_read(ms, n, NUM_STAGES))
    return {nm: (ms[i], n[i]) for i, nm in enumerate(stage_names())}


class SparseMoE:
    """One sparse MoE layer with its weights held as device tensors.

    ``layer(x)`` runs ``moe_forward`` and returns the fp32 output y. x may carry leading
    dimensions, [..., d_model] (the [batch, seq, d_model] input of the pages' layer
    modules): the tokens are those dimensions flattened (a view of the contiguous x), and
    y comes back with x's leading shape. The workspace is kept and reused while it is
    large enough; ``last`` holds the full result of the latest call (routing, f, p, loss)."""

    def __init__(self, W_g, W_gate, W_up, W_down, b_g=None, *, k=2, mode="tc",
                 capacity_factor=1.0, renormalize=True):
        self.W_g, self.W_gate, self.W_up, self.W_down, self.b_g = W_g, W_gate, W_up, W_down, b_g
        self.k, self.mode, self.cf, self.renormalize = k, mode, capacity_factor, renormalize
        self._ws = None
        self.last = None

    def __call__(self, x, **kw):
        _need(x, "x")
        lead, d = x.shape[:-1], x.shape[-1]
        out = moe_forward(x.view(-1, d), self.W_g, self.b_g, self.W_gate, self.W_up,
                          self.W_down, k=self.k, mode=self.mode, capacity_factor=self.cf,
                          renormalize=self.renormalize, workspace=self._ws, **kw)
        self._ws = out["workspace"]
        self.last = out
        return out["y"].view(*lead, d)
