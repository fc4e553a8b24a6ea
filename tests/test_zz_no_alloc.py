"""GPU test of s4dplr_forward_noalloc (the forward pass on the library's
static device scratch, for callers that cannot allocate) through the C ABI:
two calls in a row, the second on a smaller plan, each compared with
s4dplr_forward on a caller workspace (same kernels: identical bits) and with
the fp64 oracle (max|err| / max|ref| <= 1e-4).  Plans whose forward scratch
exceeds the array are rejected before any launch."""
import numpy as np
import pytest

import oracle as o
from synth import make_generic_inputs, make_inputs

pytestmark = pytest.mark.gpu
TOL = 1e-4


@pytest.fixture(scope="module")
def s4():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import structured_state_space_dplr_amd as s4
    return s4


def _dev(a):
    import torch
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _rel(gpu, ref):
    return float(np.abs(gpu.astype(np.float64) - ref).max() / np.abs(ref).max())


def _both(s4, x, diagonal=False, rank=1):
    """(K, y) from the workspace entry point and from the no-allocation one."""
    import torch
    H, N = x["lam"].shape[:2]
    batch, _, L = x["u"].shape
    plan = s4.Plan(H, N, L, batch, diagonal=diagonal, rank=rank)
    t = {k: _dev(x[k]) for k in ("lam", "P", "Q", "B", "C", "dt", "D", "u")}
    P = None if diagonal else t["P"]
    out = []
    for noalloc in (False, True):
        K = torch.full((H, L), float("nan"), device="cuda")
        y = torch.full((batch, H, L), float("nan"), device="cuda")
        if noalloc:
            s4.forward_noalloc(plan, t["lam"], P, t["Q"], t["B"], t["C"], t["dt"], t["D"],
                               t["u"], K, y)
        else:
            s4.forward(plan, t["lam"], P, t["Q"], t["B"], t["C"], t["dt"], t["D"], t["u"], K, y,
                       plan.workspace())
        torch.cuda.synchronize()
        out.append((K.cpu().numpy(), y.cpu().numpy()))
    plan.close()
    return out


def test_two_calls_second_smaller(s4):
    cases = [("mid, then a smaller generic plan", make_inputs("mid"), False),
             ("", make_generic_inputs(H=3, N=8, L=512, batch=2, seed=5), False)]
    for label, x, diag in cases:
        if label:
            print(f"case: forward_noalloc {label}", flush=True)
        (Kw, yw), (Kn, yn) = _both(s4, x, diagonal=diag)
        assert np.array_equal(Kw, Kn) and np.array_equal(yw, yn)
        Kr, yr = o.forward(x["lam"], x["P"], x["Q"], x["B"], x["C"], x["dt"], x["D"], x["u"],
                           diagonal=diag)
        assert _rel(Kn, Kr) <= TOL and _rel(yn, yr) <= TOL


@pytest.mark.parametrize("L,diag", [(16384, False), (4096, True), (65536, False)])
def test_length_classes(s4, L, diag):
    # the row kernels (L = 4096, 16384) and the four-step path (65536), each
    # after a call of another shape has left its contents in the array
    print(f"case: forward_noalloc L={L} diagonal={diag}", flush=True)
    x = make_generic_inputs(H=4, N=16, L=L, batch=2, seed=L + 1, diagonal=diag)
    (Kw, yw), (Kn, yn) = _both(s4, x, diagonal=diag)
    assert np.array_equal(Kw, Kn) and np.array_equal(yw, yn)
    Kr, yr = o.forward(x["lam"], x["P"], x["Q"], x["B"], x["C"], x["dt"], x["D"], x["u"],
                       diagonal=diag)
    assert _rel(Kn, Kr) <= TOL and _rel(yn, yr) <= TOL


@pytest.mark.parametrize("L,rank", [(2048, 2), (32768, 3)])
def test_low_rank_plans(s4, L, rank):
    # rank r > 1 plans read the two-float frequency nodes, which the
    # no-allocation path computes on the device like every other table
    print(f"case: forward_noalloc L={L} rank={rank}", flush=True)
    x = make_generic_inputs(H=3, N=12, L=L, batch=2, seed=L + rank, distinct_q=True, rank=rank)
    (Kw, yw), (Kn, yn) = _both(s4, x, rank=rank)
    assert np.array_equal(Kw, Kn) and np.array_equal(yw, yn)
    Kr, yr = o.forward(x["lam"], x["P"], x["Q"], x["B"], x["C"], x["dt"], x["D"], x["u"])
    assert _rel(Kn, Kr) <= TOL and _rel(yn, yr) <= TOL


def test_too_large_plan_is_rejected(s4):
    import torch
    plan = s4.Plan(64, 64, 65536, 4)
    z = lambda *s: torch.zeros(s, device="cuda")
    c = z(64, 64, 2)
    with pytest.raises(s4.S4DPLRError) as ei:
        s4.forward_noalloc(plan, c, c, None, c, c, z(64), None, z(4, 64, 65536), None,
                           z(4, 64, 65536))
    assert ei.value.status == 7
    plan.close()
