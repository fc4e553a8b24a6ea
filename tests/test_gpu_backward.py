"""GPU parity of the backward pass (s4dplr_conv_bwd, s4dplr_kernel_gen_bwd,
through the C ABI) against the fp64 oracle: the convolution gradients
against ``conv_backward_fft`` (pinned to the direct sums) and the parameter
gradients against reverse-mode differentiation of the dense aliased kernel
(pinned by central differences).  Gate: max|gpu - oracle| / max|oracle|
<= 1e-4 for every gradient tensor, the fp32-against-fp64 tolerance of the
forward pass."""
import numpy as np
import pytest

import oracle as o
from synth import WORKLOADS, make_generic_inputs, make_inputs

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


def gpu_conv_bwd(s4, u, K, D, dy, want=("du", "dK", "dD")):
    import torch
    batch, H, L = u.shape
    plan = s4.Plan(H, 1, L, batch)
    ws = plan.workspace()
    out = {
        "du": torch.empty((batch, H, L), device="cuda") if "du" in want else None,
        "dK": torch.empty((H, L), device="cuda") if "dK" in want else None,
        "dD": torch.empty((H,), device="cuda") if "dD" in want else None,
    }
    s4.conv_bwd(plan, _dev(u), _dev(K), _dev(D), _dev(dy), out["du"], out["dK"], out["dD"], ws)
    torch.cuda.synchronize()
    plan.close()
    return {k: (None if v is None else v.cpu().numpy()) for k, v in out.items()}


def gpu_kernel_gen_bwd(s4, x, dK, diagonal=False):
    import torch
    H, N = x["lam"].shape[:2]
    L = dK.shape[1]
    plan = s4.Plan(H, N, L, 1, diagonal=diagonal)
    ws = plan.workspace()
    t = {k: _dev(x[k]) for k in ("lam", "P", "Q", "B", "C", "dt")}
    if diagonal:
        t["P"] = t["Q"] = None
    z = lambda *s: torch.empty(s, device="cuda")
    g = {"lam": z(H, N, 2), "B": z(H, N, 2), "C": z(H, N, 2), "dt": z(H),
         "P": None if diagonal else z(H, N, 2),
         "Q": None if (diagonal or x["Q"] is None) else z(H, N, 2)}
    s4.kernel_gen_bwd(plan, t["lam"], t["P"], t["Q"], t["B"], t["C"], t["dt"], _dev(dK),
                      g["lam"], g["P"], g["Q"], g["B"], g["C"], g["dt"], ws)
    torch.cuda.synchronize()
    plan.close()
    return {k: (None if v is None else v.cpu().numpy()) for k, v in g.items()}


def check_param_grads(g, ref, label):
    errs = {}
    for k, v in ref.items():
        if v is None:
            continue
        errs[k] = _rel(g[k], v)
    print(f"  {label} " + " ".join(f"{k} {e:.2e}" for k, e in errs.items()), flush=True)
    assert all(e <= TOL for e in errs.values()), errs


# ---- convolution backward ---------------------------------------------------

@pytest.mark.parametrize("L", [2 ** k for k in range(1, 17)])
def test_conv_bwd_all_lengths(s4, L):
    print(f"case: conv_bwd L={L}", flush=True)
    rng = np.random.default_rng(L)
    batch, H = 5, 3              # 5 rows: a partial last group of batch rows
    u = rng.standard_normal((batch, H, L)).astype(np.float32)
    dy = rng.standard_normal((batch, H, L)).astype(np.float32)
    K = (rng.standard_normal((H, L)) * np.exp(-np.arange(L) / max(L / 4, 1))).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    g = gpu_conv_bwd(s4, u, K, D, dy)
    du, dK, dD = o.conv_backward_fft(u, K, D, dy)
    e = (_rel(g["du"], du), _rel(g["dK"], dK), _rel(g["dD"], dD))
    print(f"  rel err du {e[0]:.2e} dK {e[1]:.2e} dD {e[2]:.2e}", flush=True)
    assert max(e) <= TOL
    if L <= 64:
        d2 = o.conv_backward_direct(u, K, D, dy)
        assert _rel(g["du"], d2[0]) <= TOL and _rel(g["dK"], d2[1]) <= TOL


@pytest.mark.parametrize("L", [1024, 4096, 16384, 65536])
def test_conv_bwd_single_row(s4, L):
    # one channel, one batch row: a single row group in the correlation
    # kernels, the smallest grids of the four-step and row forms
    print(f"case: conv_bwd single row L={L}", flush=True)
    rng = np.random.default_rng(3 * L + 1)
    u = rng.standard_normal((1, 1, L)).astype(np.float32)
    dy = rng.standard_normal((1, 1, L)).astype(np.float32)
    K = (rng.standard_normal((1, L)) * np.exp(-np.arange(L) / (L / 4))).astype(np.float32)
    D = rng.standard_normal(1).astype(np.float32)
    g = gpu_conv_bwd(s4, u, K, D, dy)
    du, dK, dD = o.conv_backward_fft(u, K, D, dy)
    e = (_rel(g["du"], du), _rel(g["dK"], dK), _rel(g["dD"], dD))
    print(f"  rel err du {e[0]:.2e} dK {e[1]:.2e} dD {e[2]:.2e}", flush=True)
    assert max(e) <= TOL


def test_conv_bwd_optional_outputs_and_no_D(s4):
    rng = np.random.default_rng(7)
    u, dy = rng.standard_normal((2, 4, 256)), rng.standard_normal((2, 4, 256))
    K = rng.standard_normal((4, 256)) * 0.1
    ref = o.conv_backward_fft(u, K, np.zeros(4), dy)
    for want in [("du",), ("dK",), ("dD",), ("dK", "dD")]:
        g = gpu_conv_bwd(s4, u, K, None, dy, want=want)
        for i, k in enumerate(("du", "dK", "dD")):
            if k in want:
                assert _rel(g[k], ref[i]) <= TOL
            else:
                assert g[k] is None


def test_conv_bwd_large_batch(s4):
    print("case: conv_bwd mid shape", flush=True)
    x = make_inputs("mid")
    rng = np.random.default_rng(8)
    dy = rng.standard_normal(x["u"].shape).astype(np.float32)
    K, _ = o.forward(x["lam"], x["P"], x["Q"], x["B"], x["C"], x["dt"], x["D"], x["u"][:1])
    g = gpu_conv_bwd(s4, x["u"], K.astype(np.float32), x["D"], dy)
    du, dK, dD = o.conv_backward_fft(x["u"], K.astype(np.float32), x["D"], dy)
    e = (_rel(g["du"], du), _rel(g["dK"], dK), _rel(g["dD"], dD))
    print(f"  rel err du {e[0]:.2e} dK {e[1]:.2e} dD {e[2]:.2e}", flush=True)
    assert max(e) <= TOL


# ---- kernel generation backward -----------------------------------------------

@pytest.mark.parametrize("L", [2, 4, 16, 64, 256, 1024, 2048, 4096, 8192, 16384, 32768, 65536])
def test_kernel_gen_bwd_lengths(s4, L):
    # every length class of the Ghat transform (wave-resident, LDS Stockham
    # for 2048 <= L <= 16384, four-step above)
    H = 2 if L <= 2048 else 1
    print(f"case: kernel_gen_bwd generic H={H} N=8 L={L}", flush=True)
    x = make_generic_inputs(H=H, N=8, L=L, batch=1, seed=40 + L)
    dK = np.random.default_rng(L).standard_normal((H, L)).astype(np.float32)
    g = gpu_kernel_gen_bwd(s4, x, dK)
    ref = o.kernel_backward_dense(x["lam"], x["P"], x["Q"], x["B"], x["C"], x["dt"], dK)
    check_param_grads(g, ref, f"L={L}")


@pytest.mark.parametrize("L,init", [(4096, "generic"), (8192, "hippo"), (16384, "generic"),
                                    (16384, "hippo")])
def test_kernel_gen_bwd_64_poles_long(s4, L, init):
    # 64 poles (the workloads' pole count) at the lengths whose Ghat comes
    # from the block-level Stockham transform; HiPPO-LegS poles with the
    # long workload's step range, or generic per-channel DPLR parameters
    print(f"case: kernel_gen_bwd {init} H=2 N=64 L={L}", flush=True)
    if init == "hippo":
        x = make_inputs("long", H=2, batch=1, L=L)
    else:
        x = make_generic_inputs(H=2, N=64, L=L, batch=1, seed=80 + L)
    dK = np.random.default_rng(L + 3).standard_normal((2, L)).astype(np.float32)
    g = gpu_kernel_gen_bwd(s4, x, dK)
    ref = o.kernel_backward_dense(x["lam"], x["P"], x["Q"], x["B"], x["C"], x["dt"], dK)
    check_param_grads(g, ref, f"{init} N=64 L={L}")


@pytest.mark.parametrize("diagonal,distinct_q", [(True, False), (False, True)])
def test_kernel_gen_bwd_variants(s4, diagonal, distinct_q):
    print(f"case: kernel_gen_bwd diagonal={diagonal} distinct_q={distinct_q}", flush=True)
    x = make_generic_inputs(H=3, N=16, L=128, batch=1, seed=50, diagonal=diagonal,
                            distinct_q=distinct_q)
    dK = np.random.default_rng(51).standard_normal((3, 128)).astype(np.float32)
    g = gpu_kernel_gen_bwd(s4, x, dK, diagonal=diagonal)
    ref = o.kernel_backward_dense(x["lam"], x["P"], x["Q"], x["B"], x["C"], x["dt"], dK,
                                  diagonal=diagonal)
    check_param_grads(g, ref, "variant")


@pytest.mark.parametrize("N", [1, 3, 64, 100, 256])
def test_kernel_gen_bwd_pole_counts(s4, N):
    print(f"case: kernel_gen_bwd N={N}", flush=True)
    x = make_generic_inputs(H=2, N=N, L=64, batch=1, seed=60 + N)
    dK = np.random.default_rng(N).standard_normal((2, 64)).astype(np.float32)
    g = gpu_kernel_gen_bwd(s4, x, dK)
    ref = o.kernel_backward_dense(x["lam"], x["P"], x["Q"], x["B"], x["C"], x["dt"], dK)
    check_param_grads(g, ref, f"N={N}")


def _slice(x, hs):
    return {k: (v[hs] if isinstance(v, np.ndarray) and k != "u" else v) for k, v in x.items()}


@pytest.mark.parametrize("name,n_ch", [("tiny", 4), ("mid", 2), ("long", 1), ("s4d_lin", 1),
                                         ("waveform", 1)])
def test_layer_gradients_workload(s4, name, n_ch):
    # the whole chain on the GPU: forward, then conv_bwd -> dK -> kernel_gen_bwd,
    # against the oracle's chain on sampled channels
    import torch
    w = WORKLOADS[name]
    print(f"case: layer gradients {w.describe()}, {n_ch} channels checked", flush=True)
    x = make_inputs(name)
    rng = np.random.default_rng(70)
    dy = rng.standard_normal(x["u"].shape).astype(np.float32)
    plan = s4.Plan(w.H, w.N, w.L, w.batch, diagonal=w.diagonal)
    ws = plan.workspace()
    t = {k: _dev(x[k]) for k in ("lam", "P", "Q", "B", "C", "dt", "D", "u")}
    P = None if w.diagonal else t["P"]
    K = torch.empty((w.H, w.L), device="cuda")
    y = torch.empty_like(t["u"])
    s4.forward(plan, t["lam"], P, t["Q"], t["B"], t["C"], t["dt"], t["D"], t["u"], K, y, ws)
    du = torch.empty_like(t["u"])
    dK = torch.empty((w.H, w.L), device="cuda")
    dD = torch.empty((w.H,), device="cuda")
    s4.conv_bwd(plan, t["u"], K, t["D"], _dev(dy), du, dK, dD, ws)
    z = lambda *s: torch.empty(s, device="cuda")
    g = {"lam": z(w.H, w.N, 2), "B": z(w.H, w.N, 2), "C": z(w.H, w.N, 2), "dt": z(w.H),
         "P": None if w.diagonal else z(w.H, w.N, 2), "Q": None}
    s4.kernel_gen_bwd(plan, t["lam"], P, t["Q"], t["B"], t["C"], t["dt"], dK, g["lam"], g["P"],
                      None, g["B"], g["C"], g["dt"], ws)
    torch.cuda.synchronize()
    g = {k: (None if v is None else v.cpu().numpy()) for k, v in g.items()}
    K_np, du_np, dK_np, dD_np = (a.cpu().numpy() for a in (K, du, dK, dD))
    plan.close()
    Kr, _ = o.forward(x["lam"], x["P"], x["Q"], x["B"], x["C"], x["dt"], x["D"], x["u"][:1],
                      diagonal=w.diagonal)
    dur, dKr, dDr = o.conv_backward_fft(x["u"], Kr, x["D"], dy)
    e = (_rel(du_np, dur), _rel(dK_np, dKr), _rel(dD_np, dDr))
    print(f"  rel err du {e[0]:.2e} dK {e[1]:.2e} dD {e[2]:.2e}", flush=True)
    assert max(e) <= TOL
    hs = np.sort(np.random.default_rng(1).choice(w.H, size=min(n_ch, w.H), replace=False))
    xs = _slice(x, hs)
    ref = o.kernel_backward_dense(xs["lam"], xs["P"], xs["Q"], xs["B"], xs["C"], xs["dt"],
                                  dKr[hs], diagonal=w.diagonal)
    gs = {k: (None if v is None else v[hs]) for k, v in g.items()}
    check_param_grads(gs, ref, name)
