"""C ABI checks that need no GPU: the library loads, exports every symbol that
include/moe.h declares, and validates arguments on the host (these calls return
before any HIP call, so they run on a machine without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def M():
    import sparse_mixture_experts_sum_amd as M
    if not os.path.exists(M.LIB_PATH):
        from sparse_mixture_experts_sum_amd import build
        build.build()
    M.load_library()
    return M


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("moe_route", "moe_forward", "moe_aux_loss", "moe_workspace_size", "moe_capacity"):
        assert must in names


def test_exports_every_declared_symbol(M):
    lib = ctypes.CDLL(M.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} not exported"
    assert set(declared_functions()) == set(M.EXPORTS)


def test_status_strings(M):
    lib = M.load_library()
    for st in range(7):
        assert lib.moe_status_string(st)
    assert lib.moe_status_string(99) == b"unknown status"
    assert lib.moe_stage_name(3) == b"gemm_gate_up"


def _status(M, fn, *args):
    return getattr(M.load_library(), fn)(*args)


def test_shape_validation(M):
    ok = M.make_shape(64, 128, 256, 8, 2)
    assert M.workspace_size(ok) > 0
    bad = [
        dict(T=-1), dict(d_model=100), dict(d_ff=96), dict(E=0), dict(k=0), dict(k=9),
    ]
    for b in bad:
        kw = dict(T=64, d_model=128, d_ff=256, E=8, k=2)
        kw.update(b)
        s = M.make_shape(**kw)
        with pytest.raises(M.MoEError) as ei:
            M.workspace_size(s)
        assert ei.value.status in (2, 3)
    # tile limits of the kernels, not of the method: unsupported rather than a bad shape
    for kw in (dict(d_model=100), dict(d_ff=96), dict(d_model=72, d_ff=136)):
        a = dict(T=64, d_model=128, d_ff=256, E=8, k=2)
        a.update(kw)
        with pytest.raises(M.MoEError) as ei:
            M.workspace_size(M.make_shape(**a))
        assert ei.value.status == 3, kw
    s = M.make_shape(64, 128, 256, 65, 2)
    with pytest.raises(M.MoEError) as ei:
        M.workspace_size(s)
    assert ei.value.status == 3  # E > 64 unsupported
    s = M.make_shape(64, 128, 256, 16, 9)
    with pytest.raises(M.MoEError) as ei:
        M.workspace_size(s)
    assert ei.value.status == 3  # k > 8 unsupported
    # d_model, d_ff at most 2^20
    with pytest.raises(M.MoEError) as ei:
        M.workspace_size(M.make_shape(64, 1 << 21, 256, 8, 2))
    assert ei.value.status == 2
    # fp32 layers: at most 64 * (65535 - E) routed rows; bf16 has no such limit
    E, k = 8, 2
    T_max = 64 * (65535 - E) // k
    assert M.workspace_size(M.make_shape(T_max, 64, 64, E, k, dtype="fp32")) > 0
    with pytest.raises(M.MoEError) as ei:
        M.workspace_size(M.make_shape(T_max + 32, 64, 64, E, k, dtype="fp32"))
    assert ei.value.status == 3
    assert M.workspace_size(M.make_shape(T_max + 32, 64, 64, E, k, dtype="bf16")) > 0
    s = M.make_shape(64 * 65535, 64, 64, 16, mode="ec", dtype="fp32", capacity_factor=1.0)
    with pytest.raises(M.MoEError) as ei:
        M.workspace_size(s)
    assert ei.value.status == 3


def test_capacity(M):
    assert M.capacity(M.make_shape(8192, 1024, 4096, 16, mode="ec", capacity_factor=1.0)) == 512
    assert M.capacity(M.make_shape(100, 64, 64, 8, mode="ec", capacity_factor=1.25)) == 15
    # the factor travels as a double: factors that binary floating point cannot hold give
    # the pages' int(T * cf / E) in double (0.7 as a float would give 69 here)
    from oracle import moe_oracle as O
    for T, E, cf in ((1000, 10, 0.7), (1000, 10, 0.3), (777, 7, 1.1), (4096, 64, 0.9)):
        s = M.make_shape(T, 64, 64, E, mode="ec", capacity_factor=cf)
        assert M.capacity(s) == O.capacity(T, E, cf) == int(T * cf / E), (T, E, cf)
    assert M.capacity(M.make_shape(1000, 64, 64, 10, mode="ec", capacity_factor=0.7)) == 70
    with pytest.raises(M.MoEError):
        M.capacity(M.make_shape(4, 64, 64, 8, mode="ec", capacity_factor=1.0))  # C = 0
    with pytest.raises(M.MoEError):
        M.capacity(M.make_shape(64, 64, 64, 8, mode="tc"))


def test_token_choice_capacity_host_checks(M):
    # the page's example call of the capacity routing: T=100, E=8, k=2, cf=1.25 -> 31
    import json
    from oracle import moe_oracle as O
    with open(os.path.join(ROOT, "tests", "golden", "page_values.json")) as fh:
        g = json.load(fh)["p5_capacity_of_page_call"]
    s = M.make_shape(g["T"], 64, 64, g["E"], g["k"], mode="tc_capacity",
                     capacity_factor=g["capacity_factor"])
    assert M.capacity(s) == g["value"]
    # int((T / E) * cf * k) in double, the product in that order
    for T, E, k, cf in ((8192, 8, 2, 1.0), (4096, 64, 4, 0.5), (7, 8, 1, 1.0), (1000, 3, 2, 1.1),
                        (1000, 10, 2, 0.9), (1000, 10, 1, 0.7), (333, 6, 3, 0.35)):
        s = M.make_shape(T, 64, 64, E, k, mode="tc_capacity", capacity_factor=cf)
        assert M.capacity(s) == int((T / E) * cf * k) == O.tc_capacity(T, E, k, cf)
    assert M.capacity(M.make_shape(7, 64, 64, 8, 1, mode="tc_capacity")) == 0  # valid: drops all
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(M.MoEError) as ei:
            M.workspace_size(M.make_shape(64, 64, 64, 8, 2, mode="tc_capacity",
                                          capacity_factor=bad))
        assert ei.value.status == 2
    s = M.make_shape(1000, 256, 512, 8, 2, mode="tc_capacity", capacity_factor=1.0)
    assert M.workspace_size(s) == M.workspace_size(M.make_shape(1000, 256, 512, 8, 2, mode="tc"))
    assert M.workspace_offset(s, M.WS_POS) >= 0
    with pytest.raises(ValueError):
        M.make_shape(64, 64, 64, 8, 2, mode="capacity")


def test_expert_choice_bf16_near_the_row_limit_is_sized(M):
    # bf16 expert choice carries h's residual as E * C more rows; only E * C itself must stay
    # below 2^31 (the residual rows are addressed from their own base, not by row index)
    T = (1 << 31) - 2
    s = M.make_shape(T, 64, 64, 2, 1, mode="ec", capacity_factor=1.0)
    R = 2 * (T // 2)
    assert M.workspace_size(s) >= 2 * R * 64 * 2 + R * 64 * 4  # h and its residual, o
    with pytest.raises(M.MoEError) as ei:  # C = T = 2^30 + 2, E * C = 2^31 + 4: out of range
        M.workspace_size(M.make_shape((1 << 30) + 2, 64, 64, 2, 1, mode="ec", capacity_factor=2.0))
    assert ei.value.status == 2


def test_workspace_offsets_are_inside(M):
    for mode in ("tc", "ec"):
        s = M.make_shape(1000, 256, 512, 8, 2, mode=mode)
        n = M.workspace_size(s)
        for which in (M.WS_OFFSETS, M.WS_SRC, M.WS_H, M.WS_O):
            off = M.workspace_offset(s, which)
            assert 0 <= off < n and off % 256 == 0
        # bf16 rows are gathered from x inside the GEMM: no copy to inspect; fp32 copies them
        with pytest.raises(M.MoEError) as ei:
            M.workspace_offset(s, M.WS_XPERM)
        assert ei.value.status == 3
        s32 = M.make_shape(1000, 256, 512, 8, 2, mode=mode, dtype="fp32")
        off = M.workspace_offset(s32, M.WS_XPERM)
        assert 0 <= off < M.workspace_size(s32) and off % 256 == 0
    # the gathered layout needs no copy buffer: past the shared regions the bf16 workspace
    # holds no x_perm (its h follows src directly); bf16 adds the down projection's stream-K
    # partial slots (256 x 256 KB) and flags once d_ff reaches 256 K stages of 32 (8192),
    # the shortest K the down projection splits
    s16 = M.make_shape(1000, 256, 512, 8, 2)
    s32 = M.make_shape(1000, 256, 512, 8, 2, dtype="fp32")
    R, d = 2000, 256
    assert M.workspace_offset(s32, M.WS_H) - M.workspace_offset(s32, M.WS_SRC) >= R * d * 4
    assert M.workspace_offset(s16, M.WS_H) - M.workspace_offset(s16, M.WS_SRC) < 256 * 64
    sk = 256 * 256 * 256 * 4 + 256 * 4
    assert M.workspace_offset(s16, M.WS_O) + R * d * 4 <= M.workspace_size(s16)
    assert M.workspace_size(s16) < M.workspace_offset(s16, M.WS_O) + R * d * 4 + sk
    for f, with_sk in ((8128, False), (8192, True)):
        sf = M.make_shape(1000, 256, f, 8, 2)
        end_o = M.workspace_offset(sf, M.WS_O) + R * d * 4
        assert (M.workspace_size(sf) >= end_o + sk) == with_sk, f
    # bf16 expert choice: h holds 2R rows (h, then its bf16 residual), o R rows (each row's
    # two products summed in the down projection's epilogue), and no stream-K region
    se = M.make_shape(1000, 256, 8192, 8, 1, mode="ec", capacity_factor=1.0)
    Re = 8 * 125
    assert M.workspace_offset(se, M.WS_O) - M.workspace_offset(se, M.WS_H) >= 2 * Re * 8192 * 2
    assert M.workspace_size(se) - M.workspace_offset(se, M.WS_O) < Re * d * 4 + 4096
    with pytest.raises(M.MoEError):
        M.workspace_offset(M.make_shape(1000, 256, 512, 8, 2, mode="ec"), M.WS_POS)


def test_forward_argument_errors_before_any_hip_call(M):
    lib = M.load_library()
    s = M.make_shape(64, 128, 256, 8, 2)
    n = M.workspace_size(s)
    P = ctypes.c_void_p
    good = P(4096)  # never dereferenced: every call below fails validation first
    args = dict(x=good, Wg=good, b=None, Wgate=good, Wup=good, Wdown=good, y=good)

    def call(shape=s, ws=good, ws_bytes=n, **over):
        a = dict(args)
        a.update(over)
        return lib.moe_forward(ctypes.byref(shape), a["x"], a["Wg"], a["b"], a.get("noise"),
                               a["Wgate"], a["Wup"],
                               a["Wdown"], a["y"], None, None, None, None, None, None, None, None,
                               ws, ws_bytes, None)

    assert call(x=None) == 1
    assert call(Wdown=None) == 1
    assert call(ws=None) == 1
    assert call(y=P(4100)) == 5                      # misaligned
    assert call(ws_bytes=n - 1) == 4                 # workspace too small
    assert lib.moe_forward(None, *([None] * 17), 0, None) == 1
    ec = M.make_shape(64, 128, 256, 8, mode="ec")
    f = P(8192)
    assert lib.moe_forward(ctypes.byref(ec), good, good, None, None, good, good, good, good, None,
                           None, None, None, f, None, None, None, good, n, None) == 3
    assert lib.moe_route(ctypes.byref(s), good, good, None, None, None, good, None, None, None, good,
                         n, None) == 1
    # training noise: expert choice refuses it (given or drawn), an in-kernel draw with a
    # non-finite scale is refused, and a misaligned projection is caught
    ecn = M.make_shape(64, 128, 256, 8, mode="ec", capacity_factor=1.0)
    nz = M.MoeNoise(W_noise=None, eps=8192)
    assert lib.moe_route(ctypes.byref(ecn), good, good, None, ctypes.byref(nz), good, good, None,
                         None, None, good, n * 4, None) == 3
    nzd = M.MoeNoise(W_noise=None, eps=None, seed=1, offset=2, scale=1.0)
    assert lib.moe_route(ctypes.byref(ecn), good, good, None, ctypes.byref(nzd), good, good, None,
                         None, None, good, n * 4, None) == 3
    for bad in (float("nan"), float("inf"), -float("inf")):
        nzb = M.MoeNoise(W_noise=8192, eps=None, seed=1, offset=2, scale=bad)
        assert call(noise=ctypes.byref(nzb)) == 2
    assert call(noise=ctypes.byref(M.MoeNoise(W_noise=8196, eps=8192))) == 5
    assert call(noise=ctypes.byref(M.MoeNoise(W_noise=8196, eps=None, scale=1.0))) == 5
    assert lib.moe_aux_loss(ctypes.byref(ec), good, good, good, good, good, None, good, n, None) == 3
    assert lib.moe_aux_loss(ctypes.byref(s), good, good, None, good, good, None, good, n, None) == 1


def test_profile_read_without_records(M):
    M.profile_enable(False)
    d = M.profile_read()
    assert set(d) == set(M.stage_names()) and all(v == (0.0, 0) for v in d.values())


def test_noalloc_refusals_before_any_hip_call(M):
    # the allocation-free entry point: moe_forward's argument checks, then the size of its
    # fixed scratch (a shape needing more returns MOE_ERR_WORKSPACE_TOO_SMALL); none of
    # these calls reaches a HIP call, so they run without a GPU
    lib = M.load_library()
    P = ctypes.c_void_p
    good = P(4096)

    def call(shape, **over):
        a = dict(x=good, Wg=good, Wgate=good, Wup=good, Wdown=good, y=good, f=None)
        a.update(over)
        return lib.moe_forward_noalloc(ctypes.byref(shape), a["x"], a["Wg"], None, None,
                                       a["Wgate"], a["Wup"], a["Wdown"], a["y"], None, None, None,
                                       None, a["f"], None, None, None, None)

    big = M.make_shape(16384, 4096, 14336, 8, 2)
    assert M.workspace_size(big) > M.NOALLOC_SCRATCH_BYTES
    assert call(big) == 4
    fits = M.make_shape(4096, 1024, 4096, 8, 2)
    assert M.workspace_size(fits) <= M.NOALLOC_SCRATCH_BYTES
    assert call(fits, x=None) == 1
    assert call(fits, y=P(4100)) == 5
    assert call(M.make_shape(64, 100, 64, 8, 2)) == 3
    assert call(M.make_shape(64, 128, 256, 8, mode="ec"), f=P(8192)) == 3
    assert lib.moe_forward_noalloc(None, *([None] * 16), None) == 1
