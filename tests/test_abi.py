"""CPU tests of the C ABI: the library loads, exports every entry point the
header declares, and rejects bad arguments with the documented status codes
before touching any device."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "s4dplr.h")
LIB = os.path.join(ROOT, "structured_state_space_dplr_amd", "libs4dplr.so")

OK, ERR_NULL, ERR_SHAPE, ERR_WORKSPACE, ERR_UNSUPPORTED, ERR_HIP, ERR_ALIAS = range(7)
ERR_TOO_LARGE, ERR_ALIGN = 7, 8


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from structured_state_space_dplr_amd.build import build
        build()
    import torch  # noqa: F401  (the HIP runtime the library shares)
    L = ctypes.CDLL(LIB)
    vp = ctypes.c_void_p
    L.s4dplr_plan_create.argtypes = [ctypes.POINTER(vp), ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_uint]
    L.s4dplr_plan_workspace_bytes.argtypes = [vp, ctypes.POINTER(ctypes.c_size_t)]
    L.s4dplr_plan_init.argtypes = [vp, vp, vp]
    L.s4dplr_kernel_gen.argtypes = [vp] * 10
    L.s4dplr_conv_fwd.argtypes = [vp] * 7
    L.s4dplr_forward.argtypes = [vp] * 13
    L.s4dplr_conv_apply.argtypes = [vp] * 5
    L.s4dplr_recurrent_prepare.argtypes = [vp] * 9
    L.s4dplr_recurrent_scan.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp, vp, vp]
    L.s4dplr_conv_bwd.argtypes = [vp] * 10
    L.s4dplr_kernel_gen_bwd.argtypes = [vp] * 16
    L.s4dplr_block_forward.argtypes = [vp] * 16
    L.s4dplr_plan_destroy.argtypes = [vp]
    L.s4dplr_status_string.restype = ctypes.c_char_p
    return L


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(s4dplr_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["s4dplr_abi_version", "s4dplr_status_string", "s4dplr_plan_create",
              "s4dplr_plan_workspace_bytes", "s4dplr_plan_init", "s4dplr_kernel_gen",
              "s4dplr_conv_fwd", "s4dplr_forward", "s4dplr_plan_destroy",
              "s4dplr_last_hip_error", "s4dplr_conv_apply", "s4dplr_recurrent_prepare",
              "s4dplr_recurrent_scan", "s4dplr_conv_bwd", "s4dplr_kernel_gen_bwd",
              "s4dplr_block_forward", "s4dplr_generating_function", "s4dplr_forward_noalloc"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(lib, n)


def test_version_and_status_strings(lib):
    assert lib.s4dplr_abi_version() == 1
    for s in range(9):
        assert lib.s4dplr_status_string(s) != b"unknown status"
    assert lib.s4dplr_status_string(99) == b"unknown status"


def _create(lib, H, N, L, B, flags=0):
    h = ctypes.c_void_p()
    st = lib.s4dplr_plan_create(ctypes.byref(h), H, N, L, B, flags)
    return st, h


@pytest.mark.parametrize("H,N,L,B,flags,expect", [
    (4, 16, 256, 2, 0, OK),
    (1, 1, 2, 1, 0, OK),
    (3, 256, 64, 5, 1, OK),
    (1, 64, 16384, 1, 0, OK),
    (0, 16, 256, 2, 0, ERR_SHAPE),
    (4, 0, 256, 2, 0, ERR_SHAPE),
    (4, 257, 256, 2, 0, ERR_SHAPE),
    (4, 16, 255, 2, 0, ERR_SHAPE),
    (4, 16, 1, 2, 0, ERR_SHAPE),
    (4, 16, 131072, 2, 0, ERR_SHAPE),
    (4, 16, 256, 0, 0, ERR_SHAPE),
    (4096, 16, 65536, 16, 0, ERR_SHAPE),     # batch*H*L >= 2^31
    (4, 16, 256, 2, 3, OK),                  # diagonal + zero-order hold
    (4, 16, 256, 2, 2, ERR_UNSUPPORTED),     # zero-order hold needs the diagonal flag
    (4, 16, 256, 2, 4, OK),                  # block buffers
    (4, 16, 256, 2, 8, ERR_UNSUPPORTED),
])
def test_plan_create_validation(lib, H, N, L, B, flags, expect):
    st, h = _create(lib, H, N, L, B, flags)
    assert st == expect
    if st == OK:
        n = ctypes.c_size_t()
        assert lib.s4dplr_plan_workspace_bytes(h, ctypes.byref(n)) == OK
        assert n.value > 0 and n.value % 256 == 0
        lib.s4dplr_plan_destroy(h)
    else:
        assert h.value is None


def test_null_arguments(lib):
    assert lib.s4dplr_plan_create(None, 4, 16, 256, 2, 0) == ERR_NULL
    assert lib.s4dplr_plan_workspace_bytes(None, None) == ERR_NULL
    st, h = _create(lib, 4, 16, 256, 2)
    n = ctypes.c_size_t()
    assert lib.s4dplr_plan_workspace_bytes(h, None) == ERR_NULL
    lib.s4dplr_plan_workspace_bytes(h, ctypes.byref(n))
    fake = 1 << 20          # an aligned, never-dereferenced address
    ws = 1 << 30
    # plan_init
    assert lib.s4dplr_plan_init(None, ws, None) == ERR_NULL
    assert lib.s4dplr_plan_init(h, None, None) == ERR_NULL
    assert lib.s4dplr_plan_init(h, ws + 16, None) == ERR_WORKSPACE
    # kernel_gen: lambda, P, Q, B, C, dt, K required except Q
    args = [fake] * 7
    for i in [0, 1, 3, 4, 5, 6]:
        a = list(args)
        a[i] = None
        assert lib.s4dplr_kernel_gen(h, *a, ws, None) == ERR_NULL
    assert lib.s4dplr_kernel_gen(h, *args, None, None) == ERR_NULL
    assert lib.s4dplr_kernel_gen(h, *args, ws + 8, None) == ERR_WORKSPACE
    # conv_fwd: u, K, y required; D optional
    assert lib.s4dplr_conv_fwd(h, None, fake, None, fake + 4096, ws, None) == ERR_NULL
    assert lib.s4dplr_conv_fwd(h, fake, None, None, fake + 4096, ws, None) == ERR_NULL
    assert lib.s4dplr_conv_fwd(h, fake, fake, None, None, ws, None) == ERR_NULL
    # conv_apply: u, y required
    assert lib.s4dplr_conv_apply(h, None, fake, ws, None) == ERR_NULL
    assert lib.s4dplr_conv_apply(h, fake, None, ws, None) == ERR_NULL
    assert lib.s4dplr_conv_apply(h, fake, fake + 8192, None, None) == ERR_NULL
    assert lib.s4dplr_conv_apply(h, fake, fake + 8192, ws + 4, None) == ERR_WORKSPACE
    # forward: K and D optional
    assert lib.s4dplr_forward(h, None, fake, None, fake, fake, fake, None, fake, None, fake, ws, None) == ERR_NULL
    assert lib.s4dplr_forward(h, fake, fake, None, fake, fake, fake, None, None, None, fake, ws, None) == ERR_NULL
    lib.s4dplr_plan_destroy(h)
    lib.s4dplr_plan_destroy(None)


def test_diagonal_plan_needs_no_P(lib):
    st, h = _create(lib, 2, 8, 64, 1, flags=1)
    assert st == OK
    ws = 1 << 30
    # P missing is fine for the diagonal flag; the remaining NULL checks still apply
    assert lib.s4dplr_kernel_gen(h, None, None, None, 1 << 20, 1 << 20, 1 << 20, 1 << 21, ws, None) == ERR_NULL
    st2, h2 = _create(lib, 2, 8, 64, 1, flags=0)
    assert lib.s4dplr_kernel_gen(h2, 1 << 20, None, None, 1 << 20, 1 << 20, 1 << 20, 1 << 21, ws, None) == ERR_NULL
    lib.s4dplr_plan_destroy(h)
    lib.s4dplr_plan_destroy(h2)


def test_aliasing_is_rejected_before_launch(lib):
    H, N, L, B = 4, 16, 256, 2
    st, h = _create(lib, H, N, L, B)
    n = ctypes.c_size_t()
    lib.s4dplr_plan_workspace_bytes(h, ctypes.byref(n))
    ws = 1 << 32
    u = 1 << 24
    ub = 4 * B * H * L
    K = u + 4 * ub
    # y == u, y overlapping the tail of u, y overlapping K, y inside the workspace
    for y in (u, u + ub - 4, K, ws + 256):
        assert lib.s4dplr_conv_fwd(h, u, K, None, y, ws, None) == ERR_ALIAS
    assert lib.s4dplr_conv_apply(h, u, u + 4, ws, None) == ERR_ALIAS
    assert lib.s4dplr_conv_apply(h, u, ws, ws, None) == ERR_ALIAS
    # forward: y over u; K over y; K inside the workspace
    y = K + 4 * 4 * H * L
    assert lib.s4dplr_forward(h, 1, 1, None, 1, 1, 1, None, u, None, u, ws, None) == ERR_ALIAS
    assert lib.s4dplr_forward(h, 1, 1, None, 1, 1, 1, None, u, y, y, ws, None) == ERR_ALIAS
    assert lib.s4dplr_forward(h, 1, 1, None, 1, 1, 1, None, u, ws, y, ws, None) == ERR_ALIAS
    assert lib.s4dplr_kernel_gen(h, 1, 1, None, 1, 1, 1, ws + 512, ws, None) == ERR_ALIAS
    lib.s4dplr_plan_destroy(h)


def test_misaligned_buffers_are_rejected_before_launch(lib):
    """Every device buffer is 8-byte aligned (the kernels move float pairs):
    one buffer off by 4 bytes returns ERR_ALIGN before anything is enqueued.
    Each call below has exactly one misaligned pointer, so none reaches a
    launch."""
    H, N, L, B = 4, 16, 256, 2
    st, h = _create(lib, H, N, L, B)
    n = ctypes.c_size_t()
    lib.s4dplr_plan_workspace_bytes(h, ctypes.byref(n))
    ws = 1 << 32
    a = [(1 << 20) * (i + 1) for i in range(16)]       # disjoint, aligned, never read
    lam, P, Bv, C, dt, D, u, K, y = a[:9]
    for i in [0, 1, 3, 4, 5, 6]:                        # every buffer but the absent Q
        args = [lam, P, None, Bv, C, dt, K]
        args[i] += 4
        assert lib.s4dplr_kernel_gen(h, *args, ws, None) == ERR_ALIGN
    for i in range(4):
        args = [u, K, D, y]
        args[i] += 4
        assert lib.s4dplr_conv_fwd(h, *args, ws, None) == ERR_ALIGN
    fwd = [lam, P, None, Bv, C, dt, D, u, K, y]
    for i in [0, 1, 3, 4, 5, 6, 7, 8, 9]:
        args = list(fwd)
        args[i] += 4
        assert lib.s4dplr_forward(h, *args, ws, None) == ERR_ALIGN
    assert lib.s4dplr_conv_apply(h, u + 4, y, ws, None) == ERR_ALIGN
    assert lib.s4dplr_conv_apply(h, u, y + 4, ws, None) == ERR_ALIGN
    lib.s4dplr_plan_destroy(h)


def test_hip_error_is_reported_without_a_device(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; the no-device error path cannot be forced")
    st, h = _create(lib, 4, 16, 256, 2)
    assert lib.s4dplr_plan_init(h, 1 << 30, None) == ERR_HIP
    assert lib.s4dplr_last_hip_error() != 0
    lib.s4dplr_plan_destroy(h)


def test_recurrent_validation(lib):
    H, N, L, B = 4, 16, 256, 2
    st, h = _create(lib, H, N, L, B)
    fake, ws = 1 << 20, 1 << 32
    # prepare: lambda, P, B, C, dt required; Q optional
    args = [fake] * 6
    for i in [0, 1, 3, 4, 5]:
        a = list(args)
        a[i] = None
        assert lib.s4dplr_recurrent_prepare(h, *a, ws, None) == ERR_NULL
    assert lib.s4dplr_recurrent_prepare(h, *args, None, None) == ERR_NULL
    assert lib.s4dplr_recurrent_prepare(h, *args, ws + 64, None) == ERR_WORKSPACE
    assert lib.s4dplr_recurrent_prepare(None, *args, ws, None) == ERR_NULL
    # scan: state always required; u and y unless T = 0; D optional
    u, T = 1 << 24, 100
    ub = 4 * B * H * T
    state = u + 2 * ub
    y = state + 8 * B * H * N
    assert lib.s4dplr_recurrent_scan(h, None, u, T, None, y, ws, None) == ERR_NULL
    assert lib.s4dplr_recurrent_scan(h, None, None, T, state, y, ws, None) == ERR_NULL
    assert lib.s4dplr_recurrent_scan(h, None, u, T, state, None, ws, None) == ERR_NULL
    assert lib.s4dplr_recurrent_scan(h, None, u, T, state, y, None, None) == ERR_NULL
    assert lib.s4dplr_recurrent_scan(h, None, u, T, state, y, ws + 8, None) == ERR_WORKSPACE
    assert lib.s4dplr_recurrent_scan(h, None, u, -1, state, y, ws, None) == ERR_SHAPE
    assert lib.s4dplr_recurrent_scan(h, None, u, (1 << 31) // (B * H), state, y, ws, None) == ERR_SHAPE
    # T = 0 enqueues nothing, so it succeeds even without a device
    assert lib.s4dplr_recurrent_scan(h, None, None, 0, state, None, ws, None) == OK
    # aliasing: y over u, y over the state, the state over u, the state inside the workspace
    assert lib.s4dplr_recurrent_scan(h, None, u, T, state, u + 4, ws, None) == ERR_ALIAS
    assert lib.s4dplr_recurrent_scan(h, None, u, T, state, state + 8, ws, None) == ERR_ALIAS
    assert lib.s4dplr_recurrent_scan(h, None, u, T, u + ub - 8, y, ws, None) == ERR_ALIAS
    assert lib.s4dplr_recurrent_scan(h, None, u, T, ws + 256, y, ws, None) == ERR_ALIAS
    assert lib.s4dplr_recurrent_scan(h, None, u, T, state, ws + 256, ws, None) == ERR_ALIAS
    lib.s4dplr_plan_destroy(h)


def test_backward_validation(lib):
    H, N, L, B = 4, 16, 256, 2
    st, h = _create(lib, H, N, L, B)
    ws = 1 << 32
    u = 1 << 24
    ub, kb = 4 * B * H * L, 4 * H * L
    dy, K, du, dK, dD = u + ub, u + 2 * ub, u + 3 * ub, u + 4 * ub, u + 4 * ub + kb
    # conv_bwd: dy always; K for du; u for dK / dD
    assert lib.s4dplr_conv_bwd(h, u, K, None, None, du, dK, dD, ws, None) == ERR_NULL
    assert lib.s4dplr_conv_bwd(h, u, None, None, dy, du, None, None, ws, None) == ERR_NULL
    assert lib.s4dplr_conv_bwd(h, None, K, None, dy, None, dK, None, ws, None) == ERR_NULL
    assert lib.s4dplr_conv_bwd(h, None, K, None, dy, None, None, dD, ws, None) == ERR_NULL
    assert lib.s4dplr_conv_bwd(h, u, K, None, dy, du, dK, dD, ws + 4, None) == ERR_WORKSPACE
    # outputs over inputs, over each other, inside the workspace
    assert lib.s4dplr_conv_bwd(h, u, K, None, dy, dy + 4, None, None, ws, None) == ERR_ALIAS
    assert lib.s4dplr_conv_bwd(h, u, K, None, dy, du, u, None, ws, None) == ERR_ALIAS
    assert lib.s4dplr_conv_bwd(h, u, K, None, dy, du, du + 8, None, ws, None) == ERR_ALIAS
    assert lib.s4dplr_conv_bwd(h, u, K, None, dy, None, dK, dK + 4, ws, None) == ERR_ALIAS
    assert lib.s4dplr_conv_bwd(h, u, K, None, dy, ws + 512, None, None, ws, None) == ERR_ALIAS
    # kernel_gen_bwd: parameters and dK required; outputs disjoint from inputs and each other
    f = 1 << 20
    cb = 8 * H * N
    prm = [f, f + cb, None, f + 2 * cb, f + 3 * cb, f + 4 * cb]      # lambda P Q B C dt
    dKi = f + 5 * cb
    o0 = 1 << 28
    outs = [o0, o0 + cb, None, o0 + 2 * cb, o0 + 3 * cb, o0 + 4 * cb]  # dlam dP dQ dB dC ddt
    assert lib.s4dplr_kernel_gen_bwd(h, *prm, None, *outs, ws, None) == ERR_NULL
    bad = list(prm)
    bad[0] = None
    assert lib.s4dplr_kernel_gen_bwd(h, *bad, dKi, *outs, ws, None) == ERR_NULL
    for i, target in [(0, f), (3, dKi), (1, o0 + 8), (5, ws + 1024)]:
        o = list(outs)
        o[i] = target
        assert lib.s4dplr_kernel_gen_bwd(h, *prm, dKi, *o, ws, None) == ERR_ALIAS, i
    lib.s4dplr_plan_destroy(h)


def test_block_validation(lib):
    H, N, L, B = 4, 16, 256, 2
    st, h = _create(lib, H, N, L, B)                 # no block flag
    st, hb = _create(lib, H, N, L, B, flags=4)
    ws = 1 << 32
    f = 1 << 20
    x = 1 << 24
    ub = 4 * B * H * L
    args = lambda out: [x, f, f, f, f, None, f, f, f, None, f, f, out, ws, None]
    assert lib.s4dplr_block_forward(h, *args(x + ub)) == ERR_UNSUPPORTED
    assert lib.s4dplr_block_forward(hb, *args(None)) == ERR_NULL
    a = args(x + ub)
    a[1] = None                                      # gamma
    assert lib.s4dplr_block_forward(hb, *a) == ERR_NULL
    # out may be x itself, but not a shifted view of it, an input or the workspace
    assert lib.s4dplr_block_forward(hb, *args(x + 4)) == ERR_ALIAS
    assert lib.s4dplr_block_forward(hb, *args(f)) == ERR_ALIAS
    assert lib.s4dplr_block_forward(hb, *args(ws + 256)) == ERR_ALIAS
    lib.s4dplr_plan_destroy(h)
    lib.s4dplr_plan_destroy(hb)
