"""mi_sgemm captured in a HIP graph and replayed, against eager calls.

The library enqueues kernels only (no memset, no allocation once a stream's
split-K workspace exists), and the split-K / stream-K kernels reset their
own counters, so a captured call can be replayed. Each replay runs after
eager work on the same buffers (new operand values copied in, C reset) and
a synchronisation, and must reproduce the eager result for those operands
bit for bit (every kernel sums in a fixed order).
"""
import pytest

import fp32_gemm_nn_amd as mg
from synthetic import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

# Plain tile kernel, split-K over workgroups (64 x 64), stream-K (128 x 128),
# and the skinny band kernel with its cross-workgroup reduction.
CASES = [W.C2, W.C1, W.c3(1536), W.C5B]


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mg.load_library()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
def test_graph_replays_match_eager(case):
    print(f"[gpu] graph {case.name} config {mg.config_names()[mg.mi_sgemm_select_config(case.transA, case.transB, case.M, case.N, case.K)]}", flush=True)
    inp0 = W.make_inputs(case)
    inp1 = W.make_inputs(case.with_(seed=case.seed + 100))
    A0, B0 = torch.from_numpy(inp0.A).cuda(), torch.from_numpy(inp0.B).cuda()
    A1, B1 = torch.from_numpy(inp1.A).cuda(), torch.from_numpy(inp1.B).cuda()
    C_in = torch.from_numpy(inp0.C.copy()).cuda()
    stream = torch.cuda.Stream()
    h = stream.cuda_stream

    def call(A, B, C):
        mg.sgemm(case.transA, case.transB, case.alpha, A, B, case.beta, C, stream=h)

    # Eager results on the capture stream; the first call also creates the
    # stream's workspace, outside the capture.
    want = []
    for A, B in ((A0, B0), (A1, B1)):
        C = C_in.clone()
        with torch.cuda.stream(stream):
            call(A, B, C)
        stream.synchronize()
        want.append(C)

    A, B, C = A0.clone(), B0.clone(), C_in.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        call(A, B, C)
    torch.cuda.synchronize()

    for rep in range(6):
        k = rep % 2
        # Eager work between replays: new operands into the captured buffers, C reset.
        A.copy_(A1 if k else A0)
        B.copy_(B1 if k else B0)
        C.copy_(C_in)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(C, want[k]), f"replay {rep} differs from the eager result"
    # The captured kernels hold the stream's workspace: releasing it is
    # refused while it is pinned, and the graph still replays correctly.
    name = mg.config_names()[mg.mi_sgemm_select_config(case.transA, case.transB, case.M, case.N, case.K)]
    uses_ws = "split" in name or "streamk" in name
    assert mg.mi_sgemm_release_workspace(h) == (2 if uses_ws else 0), name
    C.copy_(C_in)
    A.copy_(A0)
    B.copy_(B0)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(C, want[0]), "replay after the refused release differs"
    del graph


def test_capture_without_workspace_runs_unsplit():
    """Captured on a stream with no workspace yet, a split-K call runs unsplit
    (no allocation during capture); on integer inputs every summation order
    gives the same bits, so replays must equal the eager split result."""
    case = W.C1.with_(name="int_c1_graph", fill="int_rand")
    inp = W.make_inputs(case)
    A, B = torch.from_numpy(inp.A).cuda(), torch.from_numpy(inp.B).cuda()
    want = torch.from_numpy(inp.C.copy()).cuda()
    mg.sgemm(case.transA, case.transB, case.alpha, A, B, case.beta, want)     # eager, split
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    C = torch.full_like(want, float("nan"))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        mg.sgemm(case.transA, case.transB, case.alpha, A, B, case.beta, C, stream=stream.cuda_stream)
    torch.cuda.synchronize()
    for rep in range(3):
        C.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(C, want), f"replay {rep}"
    del graph
