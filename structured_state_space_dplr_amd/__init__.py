"""Python binding of libs4dplr (S4 DPLR convolution-mode forward on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libs4dplr.so``.  The functions carry the names of the C entry
points in ``include/s4dplr.h`` (without the ``s4dplr_`` prefix).  Tensors are
float32, contiguous, on the GPU and 8-byte aligned (a view that starts at an
odd element is refused with status 8); complex parameters are [H, N, 2]
(interleaved re, im).  PyTorch supplies device memory and the current stream.

There is no fallback: if the library is missing or fails to load, importing
this package raises.

Preconditions that the kernels do not test on the device -- Re(Lambda) < 0
(stable poles), dt > 0 and every value finite -- are checked on the host
before the call when the environment variable ``S4DPLR_VALIDATE`` is ``1``;
a violation raises ``S4DPLRPreconditionError``.  The check copies the
inputs to host memory and synchronizes, so it is for debugging, not for the
timed path.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime that libs4dplr then shares

__all__ = [
    "S4DPLRError", "S4DPLRPreconditionError", "check_preconditions", "validation_enabled",
    "DIAGONAL", "ZOH", "BLOCK", "abi_version", "status_string", "plan_create",
    "plan_workspace_bytes", "plan_init", "kernel_gen", "generating_function", "conv_fwd",
    "forward", "forward_noalloc",
    "conv_apply", "recurrent_prepare", "recurrent_scan", "conv_bwd", "kernel_gen_bwd",
    "block_forward",
    "plan_destroy", "Plan", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libs4dplr.so")
DIAGONAL = 1
ZOH = 2
BLOCK = 4
RANK_SHIFT = 8

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python structured_state_space_dplr_amd/build.py` "
        "(or __graft_entry__.build()) first")

_lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_lib.s4dplr_abi_version.restype = ctypes.c_int
_lib.s4dplr_abi_version.argtypes = []
_lib.s4dplr_status_string.restype = ctypes.c_char_p
_lib.s4dplr_status_string.argtypes = [ctypes.c_int]
_lib.s4dplr_last_hip_error.restype = ctypes.c_int
_lib.s4dplr_last_hip_error.argtypes = []
_lib.s4dplr_plan_create.restype = ctypes.c_int
_lib.s4dplr_plan_create.argtypes = [ctypes.POINTER(_p), ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_uint]
_lib.s4dplr_plan_workspace_bytes.restype = ctypes.c_int
_lib.s4dplr_plan_workspace_bytes.argtypes = [_p, ctypes.POINTER(ctypes.c_size_t)]
_lib.s4dplr_plan_init.restype = ctypes.c_int
_lib.s4dplr_plan_init.argtypes = [_p, _p, _p]
_lib.s4dplr_kernel_gen.restype = ctypes.c_int
_lib.s4dplr_kernel_gen.argtypes = [_p] * 10
_lib.s4dplr_generating_function.restype = ctypes.c_int
_lib.s4dplr_generating_function.argtypes = [_p] * 10
_lib.s4dplr_conv_fwd.restype = ctypes.c_int
_lib.s4dplr_conv_fwd.argtypes = [_p] * 7
_lib.s4dplr_forward.restype = ctypes.c_int
_lib.s4dplr_forward.argtypes = [_p] * 13
_lib.s4dplr_forward_noalloc.restype = ctypes.c_int
_lib.s4dplr_forward_noalloc.argtypes = [_p] * 12
_lib.s4dplr_conv_apply.restype = ctypes.c_int
_lib.s4dplr_conv_apply.argtypes = [_p] * 5
_lib.s4dplr_recurrent_prepare.restype = ctypes.c_int
_lib.s4dplr_recurrent_prepare.argtypes = [_p] * 9
_lib.s4dplr_recurrent_scan.restype = ctypes.c_int
_lib.s4dplr_recurrent_scan.argtypes = [_p, _p, _p, ctypes.c_int, _p, _p, _p, _p]
_lib.s4dplr_conv_bwd.restype = ctypes.c_int
_lib.s4dplr_conv_bwd.argtypes = [_p] * 10
_lib.s4dplr_kernel_gen_bwd.restype = ctypes.c_int
_lib.s4dplr_kernel_gen_bwd.argtypes = [_p] * 16
_lib.s4dplr_block_forward.restype = ctypes.c_int
_lib.s4dplr_block_forward.argtypes = [_p] * 16
_lib.s4dplr_plan_destroy.restype = None
_lib.s4dplr_plan_destroy.argtypes = [_p]


class S4DPLRError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = status_string(status)
        if status == 5:
            msg += f" (hipError_t {_lib.s4dplr_last_hip_error()})"
        super().__init__(f"{where}: status {status}: {msg}")
        self.status = status


def _check(status: int, where: str) -> None:
    if status != 0:
        raise S4DPLRError(status, where)


VALIDATE_ENV = "S4DPLR_VALIDATE"


class S4DPLRPreconditionError(ValueError):
    """An input violates a precondition the kernels do not check: Re(Lambda)
    < 0 ("The S4 kernel, from scratch", section 6 keeps the real parts of the
    poles negative; "ML//SSM//S4": a stable discrete system needs its
    eigenvalues inside the unit circle, which the bilinear map gives exactly
    for Re(Lambda) < 0), dt > 0, or finite values.  Raised only with
    S4DPLR_VALIDATE=1."""

    def __init__(self, where: str, what: str):
        super().__init__(f"{where}: {what}")
        self.where, self.what = where, what


def validation_enabled() -> bool:
    return os.environ.get(VALIDATE_ENV, "") == "1"


def _host(t):
    return torch.as_tensor(t).detach().to(device="cpu", dtype=torch.float64)


def check_preconditions(where: str = "check_preconditions", lam=None, dt=None, **tensors) -> None:
    """Raise S4DPLRPreconditionError for the first violated precondition:
    every given tensor finite, Re(lam[..., 0]) < 0 strictly, dt > 0 strictly.
    Tensors may live on any device (they are copied to host memory); None is
    skipped."""
    named = dict(tensors)
    named["lam"], named["dt"] = lam, dt
    for name, t in named.items():
        if t is None:
            continue
        h = _host(t)
        bad = ~torch.isfinite(h)
        if bool(bad.any()):
            idx = tuple(int(i) for i in bad.nonzero()[0])
            raise S4DPLRPreconditionError(where, f"{name} is not finite at index {idx}")
    if lam is not None:
        re = _host(lam)[..., 0]
        bad = re >= 0
        if bool(bad.any()):
            idx = tuple(int(i) for i in bad.nonzero()[0])
            raise S4DPLRPreconditionError(
                where, f"Re(lam) must be < 0 (stable pole); lam{list(idx)} has Re = "
                       f"{float(re[idx]):g}")
    if dt is not None:
        d = _host(dt)
        bad = d <= 0
        if bool(bad.any()):
            idx = int(bad.nonzero()[0][0])
            raise S4DPLRPreconditionError(where, f"dt must be > 0; dt[{idx}] = {float(d[idx]):g}")


def _validate(where: str, **kw) -> None:
    if validation_enabled():
        check_preconditions(where, **kw)


def abi_version() -> int:
    return _lib.s4dplr_abi_version()


def status_string(status: int) -> str:
    return _lib.s4dplr_status_string(status).decode()


def plan_create(H: int, N: int, L: int, batch: int, flags: int = 0) -> int:
    h = _p()
    _check(_lib.s4dplr_plan_create(ctypes.byref(h), H, N, L, batch, flags), "plan_create")
    return h.value


def plan_workspace_bytes(plan: int) -> int:
    n = ctypes.c_size_t()
    _check(_lib.s4dplr_plan_workspace_bytes(plan, ctypes.byref(n)), "plan_workspace_bytes")
    return n.value


def plan_destroy(plan: int) -> None:
    _lib.s4dplr_plan_destroy(plan)


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t, name, shape=None):
    """Device pointer of a float32 contiguous GPU tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if t.dtype != torch.float32:
        raise TypeError(f"{name}: must be float32, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _ws_ptr(ws) -> int:
    if isinstance(ws, torch.Tensor):
        return ws.data_ptr()
    return int(ws)


def plan_init(plan: int, ws, stream=None) -> None:
    _check(_lib.s4dplr_plan_init(plan, _ws_ptr(ws), _stream(stream)), "plan_init")


def kernel_gen(plan: "Plan | int", lam, P, Q, B, C, dt, K, ws, stream=None) -> None:
    _validate("kernel_gen", lam=lam, dt=dt, P=P, Q=Q, B=B, C=C)
    p, (H, N, L, _) = _dims(plan)
    cplx = (H, N, 2)
    lr = _lowrank_shape(plan)
    _check(_lib.s4dplr_kernel_gen(
        p, _ptr(lam, "lam", cplx), _ptr(P, "P", lr), _ptr(Q, "Q", lr), _ptr(B, "B", cplx),
        _ptr(C, "C", cplx), _ptr(dt, "dt", (H,)), _ptr(K, "K", (H, L)), _ws_ptr(ws),
        _stream(stream)), "kernel_gen")


def generating_function(plan: "Plan | int", lam, P, Q, B, C, dt, khat, ws, stream=None) -> None:
    """K-hat at the L roots of unity into ``khat`` ([H, L, 2] float32)."""
    _validate("generating_function", lam=lam, dt=dt, P=P, Q=Q, B=B, C=C)
    p, (H, N, L, _) = _dims(plan)
    cplx = (H, N, 2)
    lr = _lowrank_shape(plan)
    _check(_lib.s4dplr_generating_function(
        p, _ptr(lam, "lam", cplx), _ptr(P, "P", lr), _ptr(Q, "Q", lr), _ptr(B, "B", cplx),
        _ptr(C, "C", cplx), _ptr(dt, "dt", (H,)), _ptr(khat, "khat", (H, L, 2)), _ws_ptr(ws),
        _stream(stream)), "generating_function")


def conv_fwd(plan: "Plan | int", u, K, D, y, ws, stream=None) -> None:
    _validate("conv_fwd", u=u, K=K, D=D)
    p, (H, N, L, batch) = _dims(plan)
    _check(_lib.s4dplr_conv_fwd(
        p, _ptr(u, "u", (batch, H, L)), _ptr(K, "K", (H, L)), _ptr(D, "D", (H,)),
        _ptr(y, "y", (batch, H, L)), _ws_ptr(ws), _stream(stream)), "conv_fwd")


def forward(plan: "Plan | int", lam, P, Q, B, C, dt, D, u, K, y, ws, stream=None) -> None:
    _validate("forward", lam=lam, dt=dt, P=P, Q=Q, B=B, C=C, D=D, u=u)
    p, (H, N, L, batch) = _dims(plan)
    cplx = (H, N, 2)
    lr = _lowrank_shape(plan)
    _check(_lib.s4dplr_forward(
        p, _ptr(lam, "lam", cplx), _ptr(P, "P", lr), _ptr(Q, "Q", lr), _ptr(B, "B", cplx),
        _ptr(C, "C", cplx), _ptr(dt, "dt", (H,)), _ptr(D, "D", (H,)),
        _ptr(u, "u", (batch, H, L)), _ptr(K, "K", (H, L)), _ptr(y, "y", (batch, H, L)),
        _ws_ptr(ws), _stream(stream)), "forward")


def forward_noalloc(plan: "Plan | int", lam, P, Q, B, C, dt, D, u, K, y, stream=None) -> None:
    """``forward`` on the library's static device scratch (no workspace)."""
    _validate("forward_noalloc", lam=lam, dt=dt, P=P, Q=Q, B=B, C=C, D=D, u=u)
    p, (H, N, L, batch) = _dims(plan)
    cplx = (H, N, 2)
    lr = _lowrank_shape(plan)
    _check(_lib.s4dplr_forward_noalloc(
        p, _ptr(lam, "lam", cplx), _ptr(P, "P", lr), _ptr(Q, "Q", lr), _ptr(B, "B", cplx),
        _ptr(C, "C", cplx), _ptr(dt, "dt", (H,)), _ptr(D, "D", (H,)),
        _ptr(u, "u", (batch, H, L)), _ptr(K, "K", (H, L)), _ptr(y, "y", (batch, H, L)),
        _stream(stream)), "forward_noalloc")


def conv_apply(plan: "Plan | int", u, y, ws, stream=None) -> None:
    _validate("conv_apply", u=u)
    p, (H, N, L, batch) = _dims(plan)
    _check(_lib.s4dplr_conv_apply(
        p, _ptr(u, "u", (batch, H, L)), _ptr(y, "y", (batch, H, L)), _ws_ptr(ws),
        _stream(stream)), "conv_apply")


def recurrent_prepare(plan: "Plan | int", lam, P, Q, B, C, dt, ws, stream=None) -> None:
    _validate("recurrent_prepare", lam=lam, dt=dt, P=P, Q=Q, B=B, C=C)
    p, (H, N, L, _) = _dims(plan)
    cplx = (H, N, 2)
    lr = _lowrank_shape(plan)
    _check(_lib.s4dplr_recurrent_prepare(
        p, _ptr(lam, "lam", cplx), _ptr(P, "P", lr), _ptr(Q, "Q", lr), _ptr(B, "B", cplx),
        _ptr(C, "C", cplx), _ptr(dt, "dt", (H,)), _ws_ptr(ws), _stream(stream)),
        "recurrent_prepare")


def recurrent_scan(plan: "Plan | int", D, u, state, y, ws, stream=None) -> None:
    """T = u.shape[-1] steps from ``state`` ([batch, H, N, 2], updated in place)."""
    p, (H, N, L, batch) = _dims(plan)
    _validate("recurrent_scan", D=D, u=u, state=state)
    if u is None or u.dim() != 3:
        raise ValueError("u: expected a [batch, H, T] tensor")
    T = int(u.shape[-1])
    _check(_lib.s4dplr_recurrent_scan(
        p, _ptr(D, "D", (H,)), _ptr(u, "u", (batch, H, T)), T,
        _ptr(state, "state", (batch, H, N, 2)), _ptr(y, "y", (batch, H, T)), _ws_ptr(ws),
        _stream(stream)), "recurrent_scan")


def conv_bwd(plan: "Plan | int", u, K, D, dy, du, dK, dD, ws, stream=None) -> None:
    _validate("conv_bwd", u=u, K=K, D=D, dy=dy)
    p, (H, N, L, batch) = _dims(plan)
    _check(_lib.s4dplr_conv_bwd(
        p, _ptr(u, "u", (batch, H, L)), _ptr(K, "K", (H, L)), _ptr(D, "D", (H,)),
        _ptr(dy, "dy", (batch, H, L)), _ptr(du, "du", (batch, H, L)), _ptr(dK, "dK", (H, L)),
        _ptr(dD, "dD", (H,)), _ws_ptr(ws), _stream(stream)), "conv_bwd")


def kernel_gen_bwd(plan: "Plan | int", lam, P, Q, B, C, dt, dK, dlam, dP, dQ, dB, dC, ddt, ws,
                   stream=None) -> None:
    _validate("kernel_gen_bwd", lam=lam, dt=dt, P=P, Q=Q, B=B, C=C, dK=dK)
    p, (H, N, L, _) = _dims(plan)
    cplx = (H, N, 2)
    lr = _lowrank_shape(plan)
    _check(_lib.s4dplr_kernel_gen_bwd(
        p, _ptr(lam, "lam", cplx), _ptr(P, "P", lr), _ptr(Q, "Q", lr), _ptr(B, "B", cplx),
        _ptr(C, "C", cplx), _ptr(dt, "dt", (H,)), _ptr(dK, "dK", (H, L)),
        _ptr(dlam, "dlam", cplx), _ptr(dP, "dP", lr), _ptr(dQ, "dQ", lr),
        _ptr(dB, "dB", cplx), _ptr(dC, "dC", cplx), _ptr(ddt, "ddt", (H,)), _ws_ptr(ws),
        _stream(stream)), "kernel_gen_bwd")


def block_forward(plan: "Plan | int", x, gamma, beta, lam, P, Q, B, C, dt, D, W, bias, out, ws,
                  stream=None) -> None:
    _validate("block_forward", lam=lam, dt=dt, x=x, gamma=gamma, beta=beta, P=P, Q=Q, B=B, C=C,
              D=D, W=W, bias=bias)
    p, (H, N, L, batch) = _dims(plan)
    cplx = (H, N, 2)
    lr = _lowrank_shape(plan)
    _check(_lib.s4dplr_block_forward(
        p, _ptr(x, "x", (batch, H, L)), _ptr(gamma, "gamma", (H,)), _ptr(beta, "beta", (H,)),
        _ptr(lam, "lam", cplx), _ptr(P, "P", lr), _ptr(Q, "Q", lr), _ptr(B, "B", cplx),
        _ptr(C, "C", cplx), _ptr(dt, "dt", (H,)), _ptr(D, "D", (H,)), _ptr(W, "W", (2 * H, H)),
        _ptr(bias, "bias", (2 * H,)), _ptr(out, "out", (batch, H, L)), _ws_ptr(ws),
        _stream(stream)), "block_forward")


def _dims(plan):
    if isinstance(plan, Plan):
        return plan.handle, (plan.H, plan.N, plan.L, plan.batch)
    raise TypeError("pass a Plan (its sizes are needed to check tensor shapes)")


def _lowrank_shape(plan):
    """Shape of P and Q: [H, N, 2] at rank 1, [H, r, N, 2] at rank r > 1."""
    if plan.rank == 1:
        return (plan.H, plan.N, 2)
    return (plan.H, plan.rank, plan.N, 2)


class Plan:
    """Owns a plan handle and (optionally) a workspace tensor on one device."""

    def __init__(self, H: int, N: int, L: int, batch: int, diagonal: bool = False,
                 device=None, zoh: bool = False, block: bool = False, rank: int = 1):
        self.H, self.N, self.L, self.batch = H, N, L, batch
        self.diagonal, self.zoh, self.block, self.rank = diagonal, zoh, block, rank
        self.handle = plan_create(H, N, L, batch, (DIAGONAL if diagonal else 0)
                                  | (ZOH if zoh else 0) | (BLOCK if block else 0)
                                  | ((rank << RANK_SHIFT) if rank != 1 else 0))
        self.workspace_bytes = plan_workspace_bytes(self.handle)
        self.device = torch.device("cuda" if device is None else device)
        self._ws_store = None
        self._ws = None

    def workspace(self, stream=None):
        """A 256-byte aligned workspace tensor with the tables already written."""
        if self._ws is None:
            store = torch.empty(self.workspace_bytes + 256, dtype=torch.uint8, device=self.device)
            off = (-store.data_ptr()) % 256
            self._ws_store = store
            self._ws = store[off: off + self.workspace_bytes]
            plan_init(self.handle, self._ws, stream)
        return self._ws

    def close(self) -> None:
        if self.handle:
            plan_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
