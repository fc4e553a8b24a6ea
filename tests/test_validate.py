"""Host-side precondition checks of the binding (S4DPLR_VALIDATE=1): each
violated precondition -- Re(Lambda) >= 0, dt <= 0, a value that is not
finite -- raises S4DPLRPreconditionError naming the input, and valid inputs
pass.  The checker itself runs on CPU tensors (no GPU needed); the GPU tests
call the entry points with and without the flag."""
import os

import numpy as np
import pytest

from synth import make_generic_inputs

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "structured_state_space_dplr_amd", "libs4dplr.so")


@pytest.fixture(scope="module")
def s4():
    if not os.path.exists(LIB):
        from structured_state_space_dplr_amd.build import build
        build()
    import structured_state_space_dplr_amd as s4
    return s4


def _params(seed=3):
    import torch
    x = make_generic_inputs(H=3, N=8, L=64, batch=2, seed=seed)
    return {k: torch.from_numpy(np.ascontiguousarray(x[k])) for k in
            ("lam", "P", "B", "C", "dt", "D", "u")}


def test_valid_inputs_pass(s4):
    t = _params()
    s4.check_preconditions("forward", lam=t["lam"], dt=t["dt"], P=t["P"], B=t["B"], C=t["C"],
                           D=t["D"], u=t["u"], Q=None)


@pytest.mark.parametrize("case", ["re_positive", "re_zero", "dt_zero", "dt_negative",
                                  "nan_u", "inf_C", "nan_lam_im", "inf_D"])
def test_each_violation_raises(s4, case):
    t = _params()
    if case == "re_positive":
        t["lam"][1, 4, 0] = 0.25
        frag = "Re(lam)"
    elif case == "re_zero":
        t["lam"][2, 0, 0] = 0.0
        frag = "Re(lam)"
    elif case == "dt_zero":
        t["dt"][1] = 0.0
        frag = "dt must be > 0"
    elif case == "dt_negative":
        t["dt"][0] = -1e-3
        frag = "dt must be > 0"
    elif case == "nan_u":
        t["u"][1, 2, 17] = float("nan")
        frag = "u is not finite"
    elif case == "inf_C":
        t["C"][0, 3, 1] = float("inf")
        frag = "C is not finite"
    elif case == "nan_lam_im":
        t["lam"][0, 1, 1] = float("nan")
        frag = "lam is not finite"
    else:
        t["D"][2] = float("-inf")
        frag = "D is not finite"
    with pytest.raises(s4.S4DPLRPreconditionError) as ei:
        s4.check_preconditions("forward", lam=t["lam"], dt=t["dt"], P=t["P"], B=t["B"],
                               C=t["C"], D=t["D"], u=t["u"])
    assert frag in str(ei.value)
    assert ei.value.where == "forward"


def test_flag_read_from_environment(s4, monkeypatch):
    monkeypatch.delenv("S4DPLR_VALIDATE", raising=False)
    assert not s4.validation_enabled()
    monkeypatch.setenv("S4DPLR_VALIDATE", "1")
    assert s4.validation_enabled()
    monkeypatch.setenv("S4DPLR_VALIDATE", "0")
    assert not s4.validation_enabled()


# ---- through the entry points on the GPU ----------------------------------------

@pytest.mark.gpu
@pytest.mark.parametrize("case", ["re_positive", "dt_zero", "nan_u"])
def test_gpu_entry_points_with_and_without_flag(s4, case, monkeypatch):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"case: validation {case}", flush=True)
    t = {k: v.cuda() for k, v in _params().items()}
    if case == "re_positive":
        t["lam"][0, 0, 0] = 0.5
    elif case == "dt_zero":
        t["dt"][2] = 0.0
    else:
        t["u"][0, 0, 5] = float("nan")
    plan = s4.Plan(3, 8, 64, 2)
    ws = plan.workspace()
    K = torch.empty((3, 64), device="cuda")
    y = torch.empty((2, 3, 64), device="cuda")
    monkeypatch.setenv("S4DPLR_VALIDATE", "1")
    with pytest.raises(s4.S4DPLRPreconditionError):
        s4.forward(plan, t["lam"], t["P"], None, t["B"], t["C"], t["dt"], t["D"], t["u"], K, y, ws)
    if case != "nan_u":
        with pytest.raises(s4.S4DPLRPreconditionError):
            s4.kernel_gen(plan, t["lam"], t["P"], None, t["B"], t["C"], t["dt"], K, ws)
    # without the flag the call goes through (the kernels do not check)
    monkeypatch.delenv("S4DPLR_VALIDATE")
    s4.forward(plan, t["lam"], t["P"], None, t["B"], t["C"], t["dt"], t["D"], t["u"], K, y, ws)
    torch.cuda.synchronize()
    # and valid inputs pass with the flag set
    monkeypatch.setenv("S4DPLR_VALIDATE", "1")
    v = {k: x.cuda() for k, x in _params().items()}
    s4.forward(plan, v["lam"], v["P"], None, v["B"], v["C"], v["dt"], v["D"], v["u"], K, y, ws)
    torch.cuda.synchronize()
    plan.close()


@pytest.mark.gpu
def test_gpu_misaligned_buffer_is_rejected(s4):
    """A contiguous float32 view 4 bytes past an 8-byte boundary is refused by
    the C ABI (status 8, ERR_ALIGN) before anything is enqueued; the same
    values at an aligned address go through."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("case: misaligned u and y views", flush=True)
    t = {k: v.cuda() for k, v in _params().items()}
    plan = s4.Plan(3, 8, 64, 2)
    ws = plan.workspace()
    K = torch.empty((3, 64), device="cuda")
    y = torch.empty((2, 3, 64), device="cuda")
    store = torch.empty(t["u"].numel() + 1, device="cuda")
    u_odd = store[1:].view(2, 3, 64)
    u_odd.copy_(t["u"])
    assert u_odd.is_contiguous() and u_odd.data_ptr() % 8 == 4
    with pytest.raises(s4.S4DPLRError) as ei:
        s4.forward(plan, t["lam"], t["P"], None, t["B"], t["C"], t["dt"], t["D"], u_odd, K, y, ws)
    assert ei.value.status == 8
    ystore = torch.empty(y.numel() + 1, device="cuda")
    y_odd = ystore[1:].view(2, 3, 64)
    with pytest.raises(s4.S4DPLRError) as ei:
        s4.conv_apply(plan, t["u"], y_odd, ws)
    assert ei.value.status == 8
    s4.forward(plan, t["lam"], t["P"], None, t["B"], t["C"], t["dt"], t["D"], t["u"], K, y, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    plan.close()
