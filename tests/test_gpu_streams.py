"""Split products on streams that the caller creates and destroys.

The split-K workspace is kept per (device, stream handle). A stream that is
synchronised and destroyed without mi_sgemm_release_workspace leaves its
workspace behind, and a new stream may be handed the same handle and reuse
it: every split product leaves the counters at zero and overwrites each
partial block before it is read, so the inherited workspace is as good as a
fresh one once the old stream's work has finished. Whether or not the
runtime reuses a handle here, every product on every stream must equal the
same product on torch's stream, bit for bit (integer inputs).
"""
import ctypes
import sys

import pytest

import fp32_gemm_nn_amd as mg
from synthetic import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def note(msg):
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module")
def hip():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mg.load_library()
    # The HIP runtime the library itself is linked against (the one already
    # loaded in this process), looked up through the library's handle.
    lib = mg._lib
    lib.hipStreamCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    lib.hipStreamSynchronize.argtypes = [ctypes.c_void_p]
    return lib


def _product(case, seed, stream):
    inp = W.make_inputs(case.with_(seed=seed))
    A, B = torch.from_numpy(inp.A).cuda(), torch.from_numpy(inp.B).cuda()
    C0 = torch.from_numpy(inp.C.copy()).cuda()
    want, got = C0.clone(), C0.clone()
    torch.cuda.synchronize()
    mg.sgemm(case.transA, case.transB, case.alpha, A, B, case.beta, want)
    torch.cuda.synchronize()
    mg.sgemm(case.transA, case.transB, case.alpha, A, B, case.beta, got, stream=stream)
    return want, got


@pytest.mark.parametrize("case", [W.C1.with_(name="int_c1", fill="int_rand"),
                                  W.c3(1536).with_(name="int_1536", fill="int_rand"),
                                  W.C5B.with_(name="int_c5b", fill="int_rand")], ids=lambda c: c.name)
def test_destroyed_streams_without_release(hip, case):
    handles = []
    for rep in range(6):
        s = ctypes.c_void_p()
        assert hip.hipStreamCreate(ctypes.byref(s)) == 0
        note(f"streams {case.name} rep {rep} handle {s.value:#x}")
        want, got = _product(case, 40 + rep, s.value)
        assert hip.hipStreamSynchronize(s) == 0
        assert torch.equal(got, want), f"rep {rep}"
        handles.append(s.value)
        if rep == 5:
            assert mg.mi_sgemm_release_workspace(s.value) == 0
        assert hip.hipStreamDestroy(s) == 0      # without release (except the last)
    note(f"{len(set(handles))} distinct handles over {len(handles)} streams")

