"""GPU parity of the block around the layer (s4dplr_block_forward through the C
ABI: layer norm over channels, the layer, the GLU projection on the bf16
matrix cores with split operands, bias and residual) against the fp64 oracle's block_forward on the same
seeded inputs.  Gate: max|gpu - oracle| / max|oracle| <= 1e-4."""
import numpy as np
import pytest

import oracle as o
from synth import make_block_params, make_generic_inputs, make_inputs

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
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _rel(gpu, ref):
    return float(np.abs(gpu.astype(np.float64) - ref).max() / max(np.abs(ref).max(), 1e-300))


def run_block(s4, x, bp, diagonal=False, zoh=False, in_place=False):
    import torch
    H, N = x["lam"].shape[:2]
    batch, _, L = x["u"].shape
    plan = s4.Plan(H, N, L, batch, diagonal=diagonal, zoh=zoh, block=True)
    ws = plan.workspace()
    t = {k: _dev(x[k]) for k in ("lam", "P", "Q", "B", "C", "dt", "D", "u")}
    b = {k: _dev(v) for k, v in bp.items()}
    out = t["u"] if in_place else torch.empty_like(t["u"])
    s4.block_forward(plan, t["u"], b["gamma"], b["beta"], t["lam"], None if diagonal else t["P"],
                     t["Q"], t["B"], t["C"], t["dt"], t["D"], b["W"], b["bias"], out, ws)
    torch.cuda.synchronize()
    res = out.cpu().numpy()
    plan.close()
    return res


def oracle_block(x, bp, diagonal=False, zoh=False):
    return o.block_forward(x["u"], bp["gamma"], bp["beta"], x["lam"], x["P"], x["Q"], x["B"],
                           x["C"], x["dt"], x["D"], bp["W"], bp["bias"], diagonal=diagonal,
                           disc="zoh" if zoh else "bilinear")


@pytest.mark.parametrize("H,N,L,batch", [(3, 4, 16, 2), (64, 8, 128, 2), (100, 16, 256, 3),
                                         (33, 8, 64, 1), (256, 8, 32, 2),
                                         # full 128-channel x 256-step tiles (L is a
                                         # power of two, so only L < 256 leaves a tail)
                                         (128, 8, 512, 2), (384, 8, 256, 1), (512, 8, 256, 1)])
def test_block_shapes(s4, H, N, L, batch):
    print(f"case: block H={H} N={N} L={L} batch={batch}", flush=True)
    x = make_generic_inputs(H=H, N=N, L=L, batch=batch, seed=H + L)
    bp = make_block_params(H, seed=H)
    out = run_block(s4, x, bp)
    ref = oracle_block(x, bp)
    e = _rel(out, ref)
    print(f"  rel err {e:.2e}", flush=True)
    assert e <= TOL


def test_block_in_place_and_diagonal_zoh(s4):
    print("case: block in place, diagonal ZOH", flush=True)
    x = make_generic_inputs(H=48, N=16, L=512, batch=2, seed=5, diagonal=True)
    bp = make_block_params(48, seed=6)
    out = run_block(s4, x, bp, diagonal=True, zoh=True, in_place=True)
    ref = oracle_block(x, bp, diagonal=True, zoh=True)
    assert _rel(out, ref) <= TOL


def test_block_in_place_full_tiles(s4):
    # H a multiple of 128 and L >= 256: every projection tile takes the
    # full-tile path, whose epilogue reads all residuals before any store
    print("case: block in place, H=128 N=8 L=512 batch=2", flush=True)
    x = make_generic_inputs(H=128, N=8, L=512, batch=2, seed=11)
    bp = make_block_params(128, seed=12)
    out = run_block(s4, x, bp, in_place=True)
    ref = oracle_block(x, bp)
    e = _rel(out, ref)
    print(f"  rel err {e:.2e}", flush=True)
    assert e <= TOL


def test_block_mid_workload(s4):
    print("case: block on the mid workload (H=256 N=64 L=1024 batch=32)", flush=True)
    x = make_inputs("mid")
    bp = make_block_params(x["lam"].shape[0], seed=1)
    out = run_block(s4, x, bp)
    ref = oracle_block(x, bp)
    e = _rel(out, ref)
    print(f"  rel err {e:.2e}", flush=True)
    assert e <= TOL
