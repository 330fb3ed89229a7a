"""mi_sgemm_noalloc against mi_sgemm, through the C ABI.

The entry point for callers that cannot allocate keeps split-K partial blocks
and tile counters in the device's static scratch instead of a per-stream
workspace. Its capacity equals a workspace's, so it makes the same split
plans, and its results must be the same bits as mi_sgemm's (and within the
oracle's tolerance). Each pair of calls runs a product, then a smaller one of
the same kernel family, on the one shared scratch: the second must not see
the first's partials or counters.
"""
import sys

import numpy as np
import pytest

import fp32_gemm_nn_amd as mg
import oracle
from synthetic import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 1e-3


def note(msg):
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mg.load_library()
    yield
    torch.cuda.synchronize()


def _run(entry, case, inp, stream):
    A = torch.from_numpy(inp.A).cuda()
    B = torch.from_numpy(inp.B).cuda()
    C = torch.from_numpy(inp.C.copy()).cuda()
    torch.cuda.synchronize()
    rc = entry(case.transA, case.transB, case.M, case.N, case.K, case.alpha, A.data_ptr(), case.lda_,
               B.data_ptr(), case.ldb_, case.beta, C.data_ptr(), case.ldc_, stream)
    assert rc == 0, mg.mi_sgemm_status_string(rc)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def _oracle(case, inp):
    C = inp.C.copy()
    assert oracle.sgemm(case.transA, case.transB, case.M, case.N, case.K, case.alpha, inp.A, case.lda_,
                        inp.B, case.ldb_, case.beta, C, case.ldc_) == 0
    return C


# (first, second): the second product is smaller and uses the same kernel
# family, whose split plan is named in the id.
PAIRS = [
    ("band", W.C5B, W.Case("band_small", "N", "N", 9, 1024, 2048, 1.0, 1.0, seed=81)),
    ("splitk64", W.C1, W.Case("splitk_small", "N", "N", 300, 500, 600, 1.5, 0.5, seed=82)),
    ("streamk16", W.c3(1536), W.Case("streamk16_small", "N", "N", 1280, 1280, 1280, 1.0, 0.0, seed=83)),
    ("streamk16_2wg", W.c3(2560), W.Case("streamk16_2wg_small", "N", "N", 2304, 3328, 2048, 1.0, 1.0, seed=86)),
    ("streamk256x128", W.Case("nt_3328", "N", "T", 3328, 3328, 2048, 1.0, 0.0, seed=84),
     W.Case("nt_2304", "N", "T", 2304, 2304, 1024, 1.0, 1.0, seed=85)),
]


@pytest.mark.parametrize("first,second", [(p[1], p[2]) for p in PAIRS], ids=[p[0] for p in PAIRS])
def test_noalloc_matches_mi_sgemm(first, second):
    names = mg.config_names()
    stream = torch.cuda.current_stream().cuda_stream
    for case in (first, second):
        cfg = names[mg.mi_sgemm_select_config(case.transA, case.transB, case.M, case.N, case.K)]
        assert "split" in cfg or "streamk" in cfg, (case.name, cfg)
    outs = []
    for case in (first, second):
        note(f"noalloc {case.name} {case.transA}{case.transB} {case.M}x{case.N}x{case.K}")
        inp = W.make_inputs(case)
        got = _run(mg.mi_sgemm_noalloc, case, inp, stream)
        ref = _run(mg.mi_sgemm, case, inp, stream)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"{case.name}: differs from mi_sgemm"
        want = _oracle(case, inp)
        err = float(np.abs(got.astype(np.float64) - want).max())
        assert err <= TOL, f"{case.name}: max abs error {err}"
        outs.append(got)


def test_noalloc_integer_inputs_bit_exact_back_to_back():
    """Ten calls in a row on one stream without synchronising, alternating a
    large and a smaller split product on integer inputs: each is exact."""
    stream = torch.cuda.current_stream()
    cases = [W.Case("int_big", "N", "N", 1000, 1300, 700, 1.0, -1.0, seed=86, fill="int_rand"),
             W.Case("int_small", "N", "N", 200, 300, 900, 2.0, 0.0, seed=87, fill="int_rand")]
    inputs = [W.make_inputs(c) for c in cases]
    wants = [_oracle(c, i) for c, i in zip(cases, inputs)]
    dev = [(torch.from_numpy(i.A).cuda(), torch.from_numpy(i.B).cuda()) for i in inputs]
    outs = []
    for rep in range(10):
        c = cases[rep % 2]
        A, B = dev[rep % 2]
        C = torch.from_numpy(inputs[rep % 2].C.copy()).cuda()
        rc = mg.mi_sgemm_noalloc(c.transA, c.transB, c.M, c.N, c.K, c.alpha, A.data_ptr(), c.lda_, B.data_ptr(),
                                 c.ldb_, c.beta, C.data_ptr(), c.ldc_, stream.cuda_stream)
        assert rc == 0, mg.mi_sgemm_status_string(rc)
        outs.append(C)
    torch.cuda.synchronize()
    for rep, C in enumerate(outs):
        assert np.array_equal(C.cpu().numpy(), wants[rep % 2]), f"call {rep} ({cases[rep % 2].name})"


def test_noalloc_argument_errors_and_quick_returns():
    stream = torch.cuda.current_stream().cuda_stream
    assert mg.mi_sgemm_noalloc("X", "N", 4, 4, 4, 1.0, 0, 4, 0, 4, 0.0, 0, 4, stream) == -1
    assert mg.mi_sgemm_noalloc("N", "N", 4, 4, 4, 1.0, 0, 4, 0, 4, 0.0, 0, 3, stream) == -13
    assert mg.mi_sgemm_noalloc("N", "N", 0, 4, 4, 1.0, 0, 4, 0, 4, 0.0, 0, 4, stream) == 0


@pytest.mark.parametrize("case", [W.C5B.with_(name="graph_band", beta=0.0), W.C1.with_(name="graph_splitk"),
                                  W.c3(1536).with_(name="graph_streamk", beta=0.0)], ids=lambda c: c.name)
def test_noalloc_captured_in_a_graph(case):
    """The use the entry point is for: a call captured into a HIP graph with
    no allocation, replayed four times with eager work on the same buffers
    between the replays (new operands copied in, C reset), each replay equal
    bit for bit to an eager mi_sgemm on those operands."""
    note(f"noalloc graph {case.name}")
    stream = torch.cuda.Stream()
    h = stream.cuda_stream
    inp0 = W.make_inputs(case)
    inp1 = W.make_inputs(case.with_(seed=case.seed + 100))
    A0, B0 = torch.from_numpy(inp0.A).cuda(), torch.from_numpy(inp0.B).cuda()
    A1, B1 = torch.from_numpy(inp1.A).cuda(), torch.from_numpy(inp1.B).cuda()
    C_in = torch.from_numpy(inp0.C.copy()).cuda()
    torch.cuda.synchronize()

    def args(A, B, C):
        return (case.transA, case.transB, case.M, case.N, case.K, case.alpha, A.data_ptr(), case.lda_,
                B.data_ptr(), case.ldb_, case.beta, C.data_ptr(), case.ldc_, h)

    want = []
    for A, B in ((A0, B0), (A1, B1)):
        C = C_in.clone()
        torch.cuda.synchronize()
        assert mg.mi_sgemm(*args(A, B, C)) == 0
        stream.synchronize()
        want.append(C)
    A, B, C = A0.clone(), B0.clone(), C_in.clone()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        rc = mg.mi_sgemm_noalloc(*args(A, B, C))
    assert rc == 0, mg.mi_sgemm_status_string(rc)
    torch.cuda.synchronize()
    for rep in range(4):
        k = rep % 2
        A.copy_(A1 if k else A0)
        B.copy_(B1 if k else B0)
        C.copy_(C_in)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(C, want[k]), f"replay {rep} differs from the eager result"
    del graph
