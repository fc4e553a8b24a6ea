"""One plan shared by two host threads, each with its own workspace and
stream: the plan is host-only and immutable after creation, so concurrent
forward calls with distinct workspaces must give exactly the results of the
same calls made one at a time (the kernels are deterministic, so bit for bit).
"""
import threading

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


def _workspace(s4, plan, stream):
    """A workspace of the plan's own (Plan.workspace caches a single one)."""
    import torch
    store = torch.empty(plan.workspace_bytes + 256, dtype=torch.uint8, device="cuda")
    off = (-store.data_ptr()) % 256
    ws = store[off: off + plan.workspace_bytes]
    s4.plan_init(plan.handle, ws, stream)
    return store, ws


def _buffers(x):
    """The inputs on the device and empty K, y for them."""
    import torch
    t = {k: torch.from_numpy(np.ascontiguousarray(x[k])).cuda() for k in
         ("lam", "P", "B", "C", "dt", "D", "u")}
    H, L = x["lam"].shape[0], x["u"].shape[2]
    K = torch.empty((H, L), dtype=torch.float32, device="cuda")
    y = torch.empty_like(t["u"])
    return t, K, y


@pytest.mark.parametrize("H,N,L,batch", [(8, 16, 4096, 2), (2, 16, 65536, 1)])
def test_one_plan_two_threads(s4, H, N, L, batch):
    import torch
    print(f"case: two threads, one plan, H={H} N={N} L={L} batch={batch}", flush=True)
    plan = s4.Plan(H, N, L, batch)
    xs = [make_generic_inputs(H=H, N=N, L=L, batch=batch, seed=500 + i) for i in range(2)]

    # reference: the two problems one after the other on the current stream
    ref = []
    for x in xs:
        _, ws = _workspace(s4, plan, None)
        t, K, y = _buffers(x)
        s4.forward(plan, t["lam"], t["P"], None, t["B"], t["C"], t["dt"], t["D"], t["u"], K, y,
                   ws, None)
        torch.cuda.synchronize()
        ref.append((K.cpu().numpy(), y.cpu().numpy()))

    errors = []

    def worker(i):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                store, ws = _workspace(s4, plan, stream)
                t, K, y = _buffers(xs[i])
                for rep in range(4):
                    y.fill_(float("nan"))
                    s4.forward(plan, t["lam"], t["P"], None, t["B"], t["C"], t["dt"], t["D"],
                               t["u"], K, y, ws, stream)
                    stream.synchronize()
                    if not (np.array_equal(K.cpu().numpy(), ref[i][0]) and
                            np.array_equal(y.cpu().numpy(), ref[i][1])):
                        errors.append(f"thread {i} call {rep}: results differ")
        except Exception as e:  # reported below, from the main thread
            errors.append(f"thread {i}: {e!r}")

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    assert not errors, errors
    plan.close()
