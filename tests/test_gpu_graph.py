"""The forward pass captured in a HIP graph (torch.cuda.graph) and replayed:
the callers the no-allocation entry point is for, and the workspace entry
point with a workspace allocated before the capture.  Every replay, with
other eager work on the same plan and scratch in between, must reproduce the
eager result for the inputs it sees, bit for bit (the kernels are
deterministic and nothing in the path is a memset node)."""
import numpy as np
import pytest

from synth import make_generic_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def s4():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import structured_state_space_dplr_amd as s4
    return s4


def _tensors(x):
    import torch
    return {k: torch.from_numpy(np.ascontiguousarray(x[k])).cuda() for k in
            ("lam", "P", "B", "C", "dt", "D", "u")}


@pytest.mark.parametrize("noalloc", [True, False])
@pytest.mark.parametrize("H,N,L,batch", [(4, 16, 4096, 2), (2, 16, 32768, 1)])
def test_graph_replays(s4, noalloc, H, N, L, batch):
    import torch
    print(f"case: graph replay noalloc={noalloc} H={H} N={N} L={L} batch={batch}", flush=True)
    plan = s4.Plan(H, N, L, batch)
    ws = None if noalloc else plan.workspace()
    xs = [make_generic_inputs(H=H, N=N, L=L, batch=batch, seed=800 + i) for i in range(3)]

    def call(t, K, y, stream):
        if noalloc:
            s4.forward_noalloc(plan, t["lam"], t["P"], None, t["B"], t["C"], t["dt"], t["D"],
                               t["u"], K, y, stream)
        else:
            s4.forward(plan, t["lam"], t["P"], None, t["B"], t["C"], t["dt"], t["D"], t["u"], K,
                       y, ws, stream)

    # eager results for each input set
    ref = []
    for x in xs:
        t = _tensors(x)
        K = torch.empty((H, L), dtype=torch.float32, device="cuda")
        y = torch.empty((batch, H, L), dtype=torch.float32, device="cuda")
        call(t, K, y, torch.cuda.current_stream())
        torch.cuda.synchronize()
        ref.append((K.cpu().numpy(), y.cpu().numpy()))

    # static buffers for the graph, captured on the input set 0
    st = _tensors(xs[0])
    K = torch.empty((H, L), dtype=torch.float32, device="cuda")
    y = torch.empty((batch, H, L), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                     # warm-up outside the capture
        call(st, K, y, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(st, K, y, torch.cuda.current_stream())
    torch.cuda.synchronize()

    other = _tensors(xs[2])
    Ko = torch.empty_like(K)
    yo = torch.empty_like(y)
    for rep, i in enumerate([0, 1, 0, 1]):
        src = _tensors(xs[i])
        for k in st:
            st[k].copy_(src[k])
        K.fill_(float("nan"))
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(K.cpu().numpy(), ref[i][0]), f"replay {rep}: K differs"
        assert np.array_equal(y.cpu().numpy(), ref[i][1]), f"replay {rep}: y differs"
        # eager work on the same plan (and, without a workspace, the same
        # static scratch) between the replays
        call(other, Ko, yo, torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert np.array_equal(yo.cpu().numpy(), ref[2][1])
    del g
    plan.close()
