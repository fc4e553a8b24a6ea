"""GPU parity of the recurrent view (s4dplr_recurrent_prepare / _scan, through
the C ABI) against the fp64 oracle's dense recurrence on the same seeded
inputs.  Gate: max|gpu - oracle| / max|oracle| <= 1e-4 for the outputs y and
for the carried state, the fp32-against-fp64 tolerance used for the
convolution path."""
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
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _rel(gpu, ref):
    return float(np.abs(gpu.astype(np.complex128 if np.iscomplexobj(gpu) else np.float64) - ref).max()
                 / max(np.abs(ref).max(), 1e-300))


def _c(a):
    return a[..., 0].astype(np.float64) + 1j * a[..., 1]


def _pack(xc):
    return np.ascontiguousarray(np.stack([xc.real, xc.imag], -1), dtype=np.float32)


class Scanner:
    """One plan + workspace + prepared records; scan() advances the state."""

    def __init__(self, s4, x, diagonal=False, with_D=True, stream=None, x0=None):
        import torch
        self.s4, self.stream = s4, stream
        H, N = x["lam"].shape[:2]
        batch, _, T = x["u"].shape
        L = 2                    # any valid plan length: the scan takes T per call
        while L < min(T, 65536):
            L *= 2
        self.plan = s4.Plan(H, N, L, batch, diagonal=diagonal)
        self.ws = self.plan.workspace(stream)
        t = {k: _dev(x[k]) for k in ("lam", "P", "Q", "B", "C", "dt", "D")}
        self.D = t["D"] if with_D else None
        s4.recurrent_prepare(self.plan, t["lam"], None if diagonal else t["P"], t["Q"], t["B"],
                             t["C"], t["dt"], self.ws, stream)
        self._keep = t
        if x0 is None:
            self.state = torch.zeros((batch, H, N, 2), dtype=torch.float32, device="cuda")
        else:
            self.state = _dev(_pack(x0))

    def scan(self, u):
        import torch
        ud = _dev(u)
        y = torch.empty(ud.shape, dtype=torch.float32, device="cuda")
        self.s4.recurrent_scan(self.plan, self.D, ud, self.state, y, self.ws, self.stream)
        torch.cuda.synchronize()
        return y.cpu().numpy()

    def state_np(self):
        s = self.state.cpu().numpy()
        return s[..., 0].astype(np.float64) + 1j * s[..., 1]

    def close(self):
        self.plan.close()


def oracle_rec(x, diagonal=False, with_D=True, x0=None, hs=None):
    D = x["D"] if with_D else np.zeros_like(x["D"])
    sel = (lambda a: a) if hs is None else (lambda a: None if a is None else a[hs])
    u = x["u"] if hs is None else x["u"][:, hs]
    x0s = x0 if (x0 is None or hs is None) else x0[:, hs]
    return o.recurrent_forward(sel(x["lam"]), sel(x["P"]), sel(x["Q"]), sel(x["B"]),
                               sel(x["C"]), sel(x["dt"]), sel(D), u, x0=x0s, diagonal=diagonal)


def check(s4, x, diagonal=False, with_D=True, x0=None, label=""):
    sc = Scanner(s4, x, diagonal=diagonal, with_D=with_D, x0=x0)
    y = sc.scan(x["u"])
    st = sc.state_np()
    sc.close()
    yr, sr = oracle_rec(x, diagonal=diagonal, with_D=with_D, x0=x0)
    ey, es = _rel(y, yr), _rel(st, sr)
    print(f"  {label} rel err y {ey:.3e}  state {es:.3e}", flush=True)
    assert ey <= TOL and es <= TOL


# ---- generic parameters: every work split, ragged T ------------------------

@pytest.mark.parametrize("N,batch,H", [
    (1, 2, 3), (2, 4, 16), (3, 2, 3), (7, 1, 2), (16, 3, 4), (33, 2, 3), (64, 2, 3),
    (64, 64, 32), (100, 2, 2), (256, 2, 2), (256, 8, 64),
])
def test_generic_parity(s4, N, batch, H):
    T = 75                       # not a multiple of the 16-step chunk
    print(f"case: recurrent generic N={N} batch={batch} H={H} T={T}", flush=True)
    x = make_generic_inputs(H=H, N=N, L=T, batch=batch, seed=100 + N)
    check(s4, x, label=f"N={N}")


@pytest.mark.parametrize("T", [1, 2, 15, 16, 17, 33, 256])
def test_lengths(s4, T):
    print(f"case: recurrent lengths T={T}", flush=True)
    x = make_generic_inputs(H=4, N=64, L=T, batch=3, seed=T)
    check(s4, x, label=f"T={T}")


def test_diagonal(s4):
    print("case: recurrent diagonal", flush=True)
    x = make_generic_inputs(H=5, N=16, L=200, batch=3, seed=7, diagonal=True)
    check(s4, x, diagonal=True, label="diagonal")


def test_distinct_q_and_no_D(s4):
    print("case: recurrent distinct Q, D = 0", flush=True)
    x = make_generic_inputs(H=4, N=16, L=130, batch=2, seed=11, distinct_q=True)
    check(s4, x, with_D=False, label="distinct Q")


def test_from_nonzero_state(s4):
    print("case: recurrent from a nonzero state", flush=True)
    x = make_generic_inputs(H=3, N=32, L=50, batch=4, seed=12)
    rng = np.random.default_rng(13)
    x0 = rng.standard_normal((4, 3, 32)) + 1j * rng.standard_normal((4, 3, 32))
    x0 = _c(_pack(x0))          # the fp32 values the GPU receives
    check(s4, x, x0=x0, label="x0")


def test_chunked_from_nonzero_state(s4):
    # L = 512 with 12 sequences: chunks of 64 steps; T = 300 is five chunks,
    # the last one 44 steps, carried from a nonzero starting state
    print("case: recurrent chunked, nonzero state, T=300 (chunks of 64)", flush=True)
    x = make_generic_inputs(H=3, N=32, L=300, batch=4, seed=21)
    rng = np.random.default_rng(22)
    x0 = rng.standard_normal((4, 3, 32)) + 1j * rng.standard_normal((4, 3, 32))
    x0 = _c(_pack(x0))
    check(s4, x, x0=x0, label="chunked x0")


def test_call_longer_than_the_chunk_buffer(s4):
    # a plan with L = 128 holds two chunks of 64; a call of T = 300 steps
    # takes the step-by-step form
    import torch
    print("case: recurrent T=300 on a plan with L=128", flush=True)
    x = make_generic_inputs(H=3, N=16, L=300, batch=2, seed=23)
    plan = s4.Plan(3, 16, 128, 2)
    ws = plan.workspace()
    t = {k: _dev(x[k]) for k in ("lam", "P", "Q", "B", "C", "dt", "D", "u")}
    s4.recurrent_prepare(plan, t["lam"], t["P"], t["Q"], t["B"], t["C"], t["dt"], ws)
    state = torch.zeros((2, 3, 16, 2), dtype=torch.float32, device="cuda")
    y = torch.empty_like(t["u"])
    s4.recurrent_scan(plan, t["D"], t["u"], state, y, ws)
    torch.cuda.synchronize()
    yg = y.cpu().numpy()
    sg = state.cpu().numpy()
    plan.close()
    yr, sr = oracle_rec(x)
    ey, es = _rel(yg, yr), _rel(sg[..., 0] + 1j * sg[..., 1], sr)
    print(f"  rel err y {ey:.3e}  state {es:.3e}", flush=True)
    assert ey <= TOL and es <= TOL


# ---- streaming: consecutive calls continue one sequence ---------------------

def test_split_scan_continues_the_stream(s4):
    print("case: recurrent split scan 37 + 1 + 90", flush=True)
    x = make_generic_inputs(H=4, N=64, L=128, batch=3, seed=14)
    whole = Scanner(s4, x)
    y_all = whole.scan(x["u"])
    s_all = whole.state_np()
    whole.close()
    parts = Scanner(s4, x)
    ys = [parts.scan(x["u"][..., a:b]) for a, b in [(0, 37), (37, 38), (38, 128)]]
    s_parts = parts.state_np()
    parts.close()
    y_parts = np.concatenate(ys, -1)
    assert np.abs(y_parts - y_all).max() <= 1e-6 * np.abs(y_all).max()
    assert np.abs(s_parts - s_all).max() <= 1e-6 * np.abs(s_all).max()
    yr, sr = oracle_rec(x)
    assert _rel(y_parts, yr) <= TOL and _rel(s_parts, sr) <= TOL


def test_zero_steps_leaves_state(s4):
    import torch
    x = make_generic_inputs(H=2, N=8, L=16, batch=2, seed=15)
    sc = Scanner(s4, x)
    sc.scan(x["u"])
    before = sc.state.clone()
    sc.s4.recurrent_scan(sc.plan, sc.D, torch.empty((2, 2, 0), device="cuda"), sc.state,
                         torch.empty((2, 2, 0), device="cuda"), sc.ws)
    torch.cuda.synchronize()
    assert torch.equal(before, sc.state)
    sc.close()


def test_deterministic_and_non_default_stream(s4):
    import torch
    x = make_generic_inputs(H=8, N=64, L=300, batch=4, seed=16)
    a = Scanner(s4, x)
    ya = a.scan(x["u"])
    a.close()
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        b = Scanner(s4, x, stream=st)
        yb = b.scan(x["u"])
        b.close()
    assert np.array_equal(ya, yb)


# ---- the workloads at full size, sampled channels ---------------------------

@pytest.mark.parametrize("name,n_ch", [("tiny", 16), ("mid", 4), ("s4d_lin", 2), ("long", 1),
                                         ("waveform", 1)])
def test_workload_parity_sampled(s4, name, n_ch):
    w = WORKLOADS[name]
    print(f"case: recurrent workload {w.describe()}, {n_ch} channels checked", flush=True)
    x = make_inputs(name)
    sc = Scanner(s4, x, diagonal=w.diagonal)
    y = sc.scan(x["u"])
    st = sc.state_np()
    sc.close()
    hs = np.sort(np.random.default_rng(1).choice(w.H, size=min(n_ch, w.H), replace=False))
    yr, sr = oracle_rec(x, diagonal=w.diagonal, hs=hs)
    ey, es = _rel(y[:, hs], yr), _rel(st[:, hs], sr)
    print(f"  rel err y {ey:.3e}  state {es:.3e}", flush=True)
    assert ey <= TOL and es <= TOL


# ---- the two views agree on the GPU -----------------------------------------

def test_convolution_equals_recurrence_on_gpu(s4):
    # With A-bar^L negligible the aliased kernel equals the truncated one, so
    # the convolution path and the recurrent path compute the same map.
    import torch
    print("case: convolution vs recurrence, decayed HiPPO N=64 L=1024", flush=True)
    x = make_inputs("mid", batch=8, H=8)
    x["dt"] = np.linspace(0.1, 0.5, 8).astype(np.float32)
    for h in range(8):   # the decay condition, from the oracle's dense A-bar
        A = o.dense_state_matrix(_c(x["lam"][h]), _c(x["P"][h]), _c(x["P"][h]))
        Abar, _ = o.discretize_bilinear(A, _c(x["B"][h]), float(x["dt"][h]))
        assert np.abs(np.linalg.eigvals(Abar)).max() ** 1024 < 1e-9
    H, N, L, batch = 8, 64, 1024, 8
    plan = s4.Plan(H, N, L, batch)
    ws = plan.workspace()
    t = {k: _dev(x[k]) for k in ("lam", "P", "B", "C", "dt", "D", "u")}
    y_conv = torch.empty((batch, H, L), dtype=torch.float32, device="cuda")
    s4.forward(plan, t["lam"], t["P"], None, t["B"], t["C"], t["dt"], t["D"], t["u"], None,
               y_conv, ws)
    s4.recurrent_prepare(plan, t["lam"], t["P"], None, t["B"], t["C"], t["dt"], ws)
    state = torch.zeros((batch, H, N, 2), dtype=torch.float32, device="cuda")
    y_rec = torch.empty_like(y_conv)
    s4.recurrent_scan(plan, t["D"], t["u"], state, y_rec, ws)
    # the convolution spectrum is still in the workspace: apply it again
    y_conv2 = torch.empty_like(y_conv)
    s4.conv_apply(plan, t["u"], y_conv2, ws)
    torch.cuda.synchronize()
    yc, yr, yc2 = y_conv.cpu().numpy(), y_rec.cpu().numpy(), y_conv2.cpu().numpy()
    plan.close()
    e = float(np.abs(yc - yr).max() / np.abs(yc).max())
    print(f"  conv vs recurrence rel diff {e:.3e}", flush=True)
    assert e <= 2 * TOL
    assert np.array_equal(yc, yc2)
