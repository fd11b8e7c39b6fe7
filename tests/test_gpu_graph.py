"""moe_plan + moe_forward captured in a HIP graph, on batches with both kinds
of GEMM launch (experts of many rows for the tiled kernel, experts of at most
32 rows for the streaming kernel): every replay must reproduce the eager
output bit for bit, with eager work on the caller's stream between the
replays (the path allocates nothing and clears nothing with memset nodes).
The eager output must also equal moe_forward_noalloc's, which runs the same
kernels in the library's static workspace."""

import numpy as np
import pytest
import torch

import top_reduce_amd as tr
from tests._gpu import say

pytestmark = pytest.mark.gpu


def _mixed_batch(T, E, H, I, seed):
    """Routing with 8 experts of many rows (tiled) and E - 8 of at most 32
    (streamed): slot 0 of row t goes to expert t % 8, slot 1 of the first
    rows to the small experts, -1 elsewhere."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    idx = np.full((T, 2), -1, dtype=np.int64)
    idx[:, 0] = np.arange(T) % 8
    n_small = (E - 8) * 15
    idx[:n_small, 1] = 8 + np.arange(n_small) % (E - 8)
    x = torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16)
    w = torch.rand((T, 2), generator=g, device="cuda")
    w1 = (torch.randn((E, 2 * I, H), generator=g, device="cuda") / H ** 0.5).to(torch.bfloat16)
    w2 = (torch.randn((E, H, I), generator=g, device="cuda") / I ** 0.5).to(torch.bfloat16)
    return torch.from_numpy(idx).cuda(), x, w, w1, w2


def _same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


# (T, E, H, I): two GEMM launches each kind; the three-launch tiled form
# (GEMM1 tile bound above two rounds on 256 CUs) with the streamed experts
@pytest.mark.parametrize("T,E,H,I", [(1536, 12, 512, 256), (4096, 12, 512, 2048)])
def test_forward_graph_replay(T, E, H, I):
    say(f"graph replay: T={T} E={E} H={H} I={I}")
    idx, x, w, w1, w2 = _mixed_batch(T, E, H, I, seed=T + I)
    counts = torch.bincount(idx[idx >= 0], minlength=E).cpu().numpy()
    assert (counts[:8] > 32).all() and (counts[8:] <= 32).all() and (counts[8:] > 0).all()
    stream = torch.cuda.current_stream()

    # eager
    p = tr.plan(idx, E=E, H=H, I=I)
    y_eager = tr.forward(p, x, w, w1, w2)
    torch.cuda.synchronize()

    # the same kernels in the static workspace
    y_static = torch.empty_like(y_eager)
    tr.forward_noalloc(idx, x, w, w1, w2, y=y_static, E=E)
    torch.cuda.synchronize()
    assert _same(y_eager, y_static), "moe_forward_noalloc differs from moe_forward"

    # plan + forward captured in a graph on another stream, replayed
    ws = torch.empty(tr.workspace_size(tr.make_desc(T, 2, E, H, I, torch.bfloat16, idx.dtype)),
                     dtype=torch.uint8, device="cuda")
    y = torch.empty_like(y_eager)
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        q = tr.plan(idx, E=E, H=H, I=I, ws=ws, stream=cap)
        tr.forward(q, x, w, w1, w2, y=y, stream=cap)
    torch.cuda.synchronize()
    for rep in range(4):
        y.zero_()
        graph.replay()
        # eager work on the caller's stream between replays
        y2 = tr.forward(tr.plan(idx, E=E, H=H, I=I), x, w, w1, w2)
        torch.cuda.synchronize()
        assert _same(y, y_eager), f"graph replay {rep} differs from the eager forward"
        assert _same(y2, y_eager), f"eager forward after replay {rep} differs"


# decode batches: the route scan's single-block kernel, the decode GEMM and
# GEMM2 with the reduce folded in, replayed with eager decode steps between
@pytest.mark.parametrize("T", [1, 2])
def test_decode_graph_replay(T):
    import gen
    from tests._gpu import upload
    say(f"decode graph replay: c3 T={T}")
    wl = gen.make_workload("c3", T=T, with_weights=True)
    d = upload(wl)
    p = tr.plan(d["idx"], E=wl.E, H=wl.H, I=wl.I)
    y_eager = tr.forward(p, d["x"], d["w"], d["w1"], d["w2"])
    torch.cuda.synchronize()
    y = torch.empty_like(y_eager)
    stream = torch.cuda.current_stream()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        q = tr.plan(d["idx"], E=wl.E, H=wl.H, I=wl.I, stream=cap)
        tr.forward(q, d["x"], d["w"], d["w1"], d["w2"], y=y, stream=cap)
    torch.cuda.synchronize()
    for rep in range(6):
        y.zero_()
        graph.replay()
        y2 = tr.forward(tr.plan(d["idx"], E=wl.E, H=wl.H, I=wl.I), d["x"], d["w"], d["w1"], d["w2"])
        torch.cuda.synchronize()
        assert _same(y, y_eager), f"graph replay {rep} differs from the eager forward"
        assert _same(y2, y_eager), f"eager forward after replay {rep} differs"


def _replay_matches(capture_step, eager_step, y, reps=4):
    """Capture capture_step() (writing y) on a side stream, replay it reps
    times with eager_step() between, each replay bit-equal to the eager
    output."""
    y_eager = eager_step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        capture_step(cap)
    torch.cuda.synchronize()
    for rep in range(reps):
        y.zero_()
        graph.replay()
        y2 = eager_step()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_eager.view(torch.int16)), f"replay {rep}"
        assert torch.equal(y2.view(torch.int16), y_eager.view(torch.int16)), f"eager after {rep}"


def test_fp32_graph_replay():
    """The fp32 path (c1): GEMM1 gathering x, fp32 MFMA GEMMs, full reduce."""
    import gen
    from tests._gpu import upload
    say("fp32 graph replay: c1")
    wl = gen.make_workload("c1", with_weights=True)
    d = upload(wl)
    y = torch.empty((wl.T, wl.H), dtype=torch.float32, device="cuda")

    def eager():
        p = tr.plan(d["idx"], E=wl.E, H=wl.H, I=wl.I, dtype=torch.float32)
        return tr.forward(p, d["x"], d["w"], d["w1"], d["w2"])

    def capture(s):
        q = tr.plan(d["idx"], E=wl.E, H=wl.H, I=wl.I, dtype=torch.float32, stream=s)
        tr.forward(q, d["x"], d["w"], d["w1"], d["w2"], y=y, stream=s)

    _replay_matches(capture, eager, y)


def test_padded_plan_graph_replay():
    """A DP-padded plan (block counts read on the device, padding rows'
    stale ids never read) and its forward, c4's buffer."""
    import gen
    from tests._gpu import upload
    say("padded plan graph replay: c4")
    wl = gen.make_workload("c4", with_weights=True)
    d = upload(wl)
    bc = torch.tensor(gen.C4_WORKER_COUNTS, dtype=torch.int32, device="cuda")
    y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")

    def eager():
        p = tr.plan(d["idx"], E=wl.E, H=wl.H, I=wl.I, block_rows=gen.C4_WORKER_ROWS,
                    block_counts=bc)
        return tr.forward(p, d["x"], d["w"], d["w1"], d["w2"])

    def capture(s):
        q = tr.plan(d["idx"], E=wl.E, H=wl.H, I=wl.I, block_rows=gen.C4_WORKER_ROWS,
                    block_counts=bc, stream=s)
        tr.forward(q, d["x"], d["w"], d["w1"], d["w2"], y=y, stream=s)

    _replay_matches(capture, eager, y)
