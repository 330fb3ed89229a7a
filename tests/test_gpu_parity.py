"""HIP SGEMM vs the CPU oracle, element by element, through the C ABI.

Integer-valued inputs must match bit for bit (every partial sum is an exact
FP32 integer, so any summation order gives the same result). Uniform [-1, 1)
inputs must satisfy max |GPU - oracle| <= 1e-3 for K <= 4096.
"""
import sys

import numpy as np
import pytest

import fp32_gemm_nn_amd as mg
import oracle
from synthetic import Drand48, uniform_matrix
from synthetic import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 1e-3
OPS = [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]
EDGE = [1, 2, 3, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]


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


class DevMat:
    """A stored matrix in a device buffer: rows x ld, padding and guard rows
    filled with `fill`, optionally starting `offset` floats into the buffer."""

    def __init__(self, host, ld=None, fill=float("nan"), guard_rows=1, offset=0):
        rows, cols = host.shape
        self.rows, self.cols = rows, cols
        self.ld = ld if ld is not None else max(cols, 1)
        self.offset = offset
        total = offset + (rows + guard_rows) * self.ld + 4
        self.buf = torch.full((total,), fill, dtype=torch.float32, device="cuda")
        if rows and cols:
            self.view().copy_(torch.from_numpy(np.ascontiguousarray(host)).cuda())
        self.fill = fill

    def view(self):
        return self.buf[self.offset:self.offset + self.rows * self.ld].view(self.rows, self.ld)[:, :self.cols]

    @property
    def ptr(self):
        return self.buf.data_ptr() + 4 * self.offset

    def host(self):
        return self.view().cpu().numpy()

    def outside_untouched(self):
        """Everything except the logical rows x cols still holds `fill`."""
        full = self.buf.cpu().numpy()
        mask = np.ones(full.shape, bool)
        if self.rows and self.cols:
            idx = (self.offset + np.arange(self.rows)[:, None] * self.ld + np.arange(self.cols)[None, :]).ravel()
            mask[idx] = False
        rest = full[mask]
        return np.all(np.isnan(rest)) if np.isnan(self.fill) else np.all(rest == self.fill)


def run_gpu(case, inp, config=None, lda=None, ldb=None, ldc=None, offset=0, c_fill=-3.0, ab_fill=float("nan")):
    lda = lda or case.lda_
    ldb = ldb or case.ldb_
    ldc = ldc or case.ldc_
    A = DevMat(inp.A, lda, fill=ab_fill, offset=offset)
    B = DevMat(inp.B, ldb, fill=ab_fill, offset=offset)
    C = DevMat(inp.C, ldc, fill=c_fill, offset=offset)
    args = (case.transA, case.transB, case.M, case.N, case.K, case.alpha, A.ptr, lda, B.ptr, ldb,
            case.beta, C.ptr, ldc, torch.cuda.current_stream().cuda_stream)
    rc = mg.mi_sgemm(*args) if config is None else mg.mi_sgemm_with_config(config, *args)
    assert rc == 0, mg.mi_sgemm_status_string(rc)
    torch.cuda.synchronize()
    assert C.outside_untouched(), "C padding or guard band was written"
    return C.host()


def run_oracle(case, inp):
    C = inp.C.copy()
    rc = oracle.sgemm(case.transA, case.transB, case.M, case.N, case.K, case.alpha, inp.A, case.lda_,
                      inp.B, case.ldb_, case.beta, C, case.ldc_)
    assert rc == 0
    return C


def compare(case, got, want, exact):
    if exact:
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{case.name}: {len(bad)} mismatches, first at {bad[0]}: {got[tuple(bad[0])]} vs {want[tuple(bad[0])]}"
        return
    assert np.all(np.isfinite(got))
    d = got.astype(np.float64) - want.astype(np.float64)
    maxabs = float(np.abs(d).max()) if d.size else 0.0
    note(f"{case.name}: max|err| {maxabs:.3e}  mean err {float(d.mean()) if d.size else 0:.2e}")
    assert maxabs <= TOL, f"{case.name}: max abs error {maxabs}"


def is_exact(case):
    return case.fill != "uniform"


# --- the workload configurations -----------------------------------------------------

CONFIG_CASES = [W.C1, W.C2, W.C2_INT, W.C4, *W.C5A, W.C5B, *W.SHARD8]


@pytest.mark.parametrize("case", CONFIG_CASES, ids=lambda c: c.name)
def test_workload_configs(case):
    note(f"config {case.name} {case.transA}{case.transB} {case.M}x{case.N}x{case.K}")
    inp = W.make_inputs(case)
    compare(case, run_gpu(case, inp), run_oracle(case, inp), is_exact(case))


@pytest.mark.parametrize("n", W.C3_SIZES)
def test_square_sweep(n):
    case = W.c3(n)
    note(f"sweep {case.name}")
    inp = W.make_inputs(case)
    compare(case, run_gpu(case, inp), run_oracle(case, inp), False)


INT_CASES = [
    W.C1.with_(name="int_c1", fill="int_trunc"),
    W.C2.with_(name="int_floor_1024", fill="int_floor"),
    W.C2.with_(name="int_nt_1024", transB="T", fill="int_rand", beta=-1.0),
    W.C4.with_(name="int_4096", fill="int_trunc"),
    W.C5B.with_(name="int_skinny", fill="int_rand"),
    *[c.with_(name="int_" + c.name, fill="int_rand", alpha=2.0, beta=-1.0) for c in W.C5A],
    *[W.c3(n).with_(name=f"int_sweep_{n}", fill="int_rand", alpha=0.5, beta=-2.0) for n in (256, 768, 1280, 2304)],
    # The 256 x 256 tiles for the transposed op pairs (direct-to-LDS for TN and TT).
    *[W.Case(f"int_{ta}{tb}_4096x4096x512".lower(), ta, tb, 4096, 4096, 512, 1.0, -1.0, seed=77, fill="int_rand")
      for ta, tb in (("N", "T"), ("T", "N"), ("T", "T"))],
    # The 192 x 192 tile for every op pair (256 tiles), and on a grid whose edge
    # tiles cross M and N (clamped loads) with a k tail.
    *[W.Case(f"int_{ta}{tb}_3072x3072x512".lower(), ta, tb, 3072, 3072, 512, 1.0, -1.0, seed=78, fill="int_rand")
      for ta in "NT" for tb in "NT"],
    *[W.Case(f"int_{ta}{tb}_3000x2900x{k}".lower(), ta, tb, 3000, 2900, k, 2.0, -1.0, seed=79, fill="int_rand")
      for ta, tb, k in (("N", "N", 700), ("T", "T", 701))],
    # k tails of every length mod 4 on the chosen kernels (zero-filled clamped
    # loads of the last k-tile): split-K, k-groups, stream-K.
    W.Case("int_nn_1000x1300x703", "N", "N", 1000, 1300, 703, 1.0, 1.0, seed=80, fill="int_rand"),
    *[W.Case(f"int_{ta}{tb}_1024x1024x1001".lower(), ta, tb, 1024, 1024, 1001, 1.0, -1.0, seed=81, fill="int_rand")
      for ta, tb in (("T", "N"), ("N", "T"))],
    W.Case("int_tn_1568x1124x949", "T", "N", 1568, 1124, 949, 1.0, 0.0, seed=82, fill="int_rand"),
    W.Case("int_nn_2500x2500x2502", "N", "N", 2500, 2500, 2502, 0.5, 1.0, seed=83, fill="int_rand"),
    # Two k-groups of eight waves on one round of 128 x 128 tiles (ragged M).
    W.Case("int_tn_2016x2048x2048", "T", "N", 2016, 2048, 2048, 1.0, -1.0, seed=85, fill="int_rand"),
    W.Case("int_nt_1920x2048x2100", "N", "T", 1920, 2048, 2100, 1.0, 0.0, seed=86, fill="int_rand"),
    # Two 16 x 16 stream-K workgroups per CU (520 tiles of 128 x 128, k tail).
    W.Case("int_nn_3328x2560x1000", "N", "N", 3328, 2560, 1000, 1.0, -1.0, seed=84, fill="int_rand"),
]


@pytest.mark.parametrize("case", INT_CASES, ids=lambda c: c.name)
def test_integer_inputs_bit_exact(case):
    note(f"int {case.name}")
    inp = W.make_inputs(case)
    compare(case, run_gpu(case, inp), run_oracle(case, inp), True)


@pytest.mark.parametrize("ta,tb", OPS)
@pytest.mark.parametrize("M", [1, 5, 16, 17, 31, 32])
def test_skinny_rows_every_op(ta, tb, M):
    case = W.Case(f"skinny_{ta}{tb}_M{M}", ta, tb, M, 1000, 1037, 2.0, -1.0, seed=40 + M, fill="int_rand")
    note(case.name)
    inp = W.make_inputs(case)
    compare(case, run_gpu(case, inp), run_oracle(case, inp), True)
    ucase = case.with_(name=case.name + "_uniform", fill="uniform", alpha=1.0, beta=1.0, K=4096)
    inp = W.make_inputs(ucase)
    compare(ucase, run_gpu(ucase, inp), run_oracle(ucase, inp), False)


BAND = mg.config_names().index("skinny_mfma16_band128_splitk")


@pytest.mark.parametrize("ta,tb", OPS)
@pytest.mark.parametrize("M,N,K", [(16, 4096, 4096), (7, 1000, 3001), (32, 130, 17), (17, 4096, 2048),
                                   (1, 65, 100000), (24, 640, 640),
                                   # unguarded B streaming with rows of A beyond M (one and two row blocks)
                                   (1, 1024, 4096), (5, 512, 2048), (12, 512, 1024), (28, 384, 512),
                                   (31, 256, 4096)])
def test_band_split_k(ta, tb, M, N, K):
    """Split-K band kernel: integer inputs bit-exact, whatever the split."""
    case = W.Case(f"band_{ta}{tb}_{M}x{N}x{K}", ta, tb, M, N, K, 1.0, -1.0, seed=50 + M, fill="int_rand")
    note(case.name)
    inp = W.make_inputs(case)
    compare(case, run_gpu(case, inp, config=BAND), run_oracle(case, inp), True)


def test_band_reduction_is_deterministic():
    """Twenty back-to-back calls of the split reduction give identical bits."""
    case = W.C5B.with_(beta=0.0)
    inp = W.make_inputs(case)
    A = torch.from_numpy(inp.A).cuda()
    B = torch.from_numpy(inp.B).cuda()
    outs = [torch.empty(case.M, case.N, device="cuda") for _ in range(20)]
    for C in outs:
        mg.sgemm("N", "N", 1.0, A, B, 0.0, C, config=BAND)
    torch.cuda.synchronize()
    ref = outs[0].cpu().numpy()
    compare(case, ref, run_oracle(case, inp), False)
    for C in outs[1:]:
        assert np.array_equal(C.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_band_workspace_reuse_alternating_inputs():
    """Back-to-back split calls on one stream with different data each time:
    a partial left from the previous call must never reach the result."""
    cases = [W.Case(f"alt{i}", "N", "N", 16, 4096, 4096, 1.0, 0.0, seed=60 + i, fill="int_rand") for i in range(2)]
    inputs = [W.make_inputs(c) for c in cases]
    wants = [run_oracle(c, i) for c, i in zip(cases, inputs)]
    dev = [(torch.from_numpy(i.A).cuda(), torch.from_numpy(i.B).cuda()) for i in inputs]
    outs = []
    for rep in range(10):
        A, B = dev[rep % 2]
        C = torch.empty(16, 4096, device="cuda")
        mg.sgemm("N", "N", 1.0, A, B, 0.0, C, config=BAND)
        outs.append(C)
    torch.cuda.synchronize()
    for rep, C in enumerate(outs):
        compare(cases[rep % 2], C.cpu().numpy(), wants[rep % 2], True)


def test_band_concurrent_streams():
    """Two streams run split reductions at once; each has its own workspace."""
    case = W.C5B.with_(beta=0.0)
    inp = W.make_inputs(case)
    want = run_oracle(case, inp)
    A = torch.from_numpy(inp.A).cuda()
    B = torch.from_numpy(inp.B).cuda()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for rep in range(6):
        for st in (s1, s2):
            C = torch.empty(case.M, case.N, device="cuda")
            C.record_stream(st)
            mg.sgemm("N", "N", 1.0, A, B, 0.0, C, stream=st.cuda_stream, config=BAND)
            outs.append(C)
    torch.cuda.synchronize()
    for C in outs:
        compare(case, C.cpu().numpy(), want, False)
    ref = outs[0].cpu().numpy().view(np.uint32)
    assert all(np.array_equal(C.cpu().numpy().view(np.uint32), ref) for C in outs)


# --- split-K and stream-K tile kernels -----------------------------------------------------

_NAMES = mg.config_names()
STREAMK = [_NAMES.index(n) for n in ("mfma32_128x128x32_w4x2_streamk_1wg", "mfma32_128x128x32_w4x2_streamk_2wg",
                                     "mfma32_256x128x32_w4x2_streamk", "mfma32_128x256x32_w2x4_streamk",
                                     "mfma16_128x128x32_w4x2_streamk_1wg")]
SPLIT_TILE = [i for i, n in enumerate(_NAMES) if n.startswith("mfma") and n.endswith("_splitk")]


@pytest.mark.parametrize("config", STREAMK + SPLIT_TILE)
@pytest.mark.parametrize("ta,tb", OPS)
@pytest.mark.parametrize("M,N,K", [(256, 256, 4096),    # 4 tiles, each cut across dozens of workgroups
                                   (1000, 1300, 700),   # ragged edges, tiles cut mid-k
                                   (129, 1000, 3001),   # ragged k tail inside a cut tile
                                   (2304, 2304, 96),    # many tiles, three k-tiles each
                                   (5000, 4100, 96)])   # > 2 waves of tiles: whole-tile waves after the shares
def test_split_and_stream_k_integer(config, ta, tb, M, N, K):
    """Tiles whose k-range is cut between workgroups: integer inputs, so the
    result is bit-exact whatever the cut and the partial-sum order."""
    case = W.Case(f"sk_{ta}{tb}_{M}x{N}x{K}_cfg{config}", ta, tb, M, N, K, 1.0, -1.0, seed=70 + K % 7,
                  fill="int_rand")
    note(case.name)
    inp = W.make_inputs(case)
    compare(case, run_gpu(case, inp, config=config), run_oracle(case, inp), True)


@pytest.mark.parametrize("config", STREAMK)
def test_stream_k_deterministic_and_concurrent(config):
    """Stream-K on uniform data: within tolerance of the oracle, and twenty
    calls over two concurrent streams (each with its own workspace) give
    identical bits."""
    case = W.Case(f"sk_det_cfg{config}", "N", "N", 1000, 1300, 700, 1.0, 0.0, seed=71)
    note(case.name)
    inp = W.make_inputs(case)
    A = torch.from_numpy(inp.A).cuda()
    B = torch.from_numpy(inp.B).cuda()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for rep in range(10):
        for st in (s1, s2):
            with torch.cuda.stream(st):      # the NaN fill runs on st, before the product
                C = torch.full((case.M, case.N), float("nan"), device="cuda")
            mg.sgemm("N", "N", 1.0, A, B, 0.0, C, stream=st.cuda_stream, config=config)
            outs.append(C)
    torch.cuda.synchronize()
    ref = outs[0].cpu().numpy()
    compare(case, ref, run_oracle(case, inp), False)
    assert all(np.array_equal(C.cpu().numpy().view(np.uint32), ref.view(np.uint32)) for C in outs)


@pytest.mark.parametrize("which", ["band", "streamk"])
def test_release_workspace_then_split_again(which):
    """mi_sgemm_release_workspace waits for the stream and frees its workspace;
    the next split call on that stream allocates a fresh one and is correct."""
    if which == "band":
        case, config = W.C5B.with_(beta=0.0), BAND
    else:
        case, config = W.C1, STREAMK[0]
    inp = W.make_inputs(case)
    want = run_oracle(case, inp)
    A = torch.from_numpy(inp.A).cuda()
    B = torch.from_numpy(inp.B).cuda()
    st = torch.cuda.Stream()
    for rep in range(3):
        with torch.cuda.stream(st):
            C = torch.full((case.M, case.N), float("nan"), device="cuda")
        mg.sgemm(case.transA, case.transB, case.alpha, A, B, 0.0, C, stream=st.cuda_stream, config=config)
        assert mg.mi_sgemm_release_workspace(st.cuda_stream) == 0
        compare(case, C.cpu().numpy(), want, False)
    assert mg.mi_sgemm_release_workspace(torch.cuda.Stream().cuda_stream) == 0   # none kept: no-op


# --- every kernel configuration on ragged shapes ------------------------------------------

def _edge_triples(count, seed):
    rng = np.random.default_rng(seed)
    trip = [(e, e, e) for e in EDGE]
    trip += [tuple(int(v) for v in rng.choice(EDGE, 3)) for _ in range(count)]
    return trip


NCONFIG = mg.mi_sgemm_config_count()


@pytest.mark.parametrize("ta,tb", OPS)
@pytest.mark.parametrize("config", range(NCONFIG))
def test_edge_shapes_every_config(ta, tb, config):
    scal = [(1.0, 0.0), (-1.0, 1.0), (2.0, -1.0), (0.5, 0.5), (1.0, 1.0)]
    for t, (M, N, K) in enumerate(_edge_triples(30, 100 + config)):
        alpha, beta = scal[t % len(scal)]
        case = W.Case(f"edge_{ta}{tb}_{M}x{N}x{K}_cfg{config}", ta, tb, M, N, K, alpha, beta,
                      seed=1000 + t, fill="int_rand")
        note(case.name)
        inp = W.make_inputs(case)
        if beta == 0.0:
            inp.C[:] = np.nan                       # beta == 0: C must not be read
        compare(case, run_gpu(case, inp, config=config), run_oracle(case, inp), True)


TILE_CONFIGS = [i for i, n in enumerate(mg.config_names()) if n.startswith("mfma")]


def _padded_ld(rows_cols, pad=4):
    """A leading dimension divisible by 4 with at least `pad` floats of row padding."""
    return (rows_cols[1] + 3) // 4 * 4 + pad


@pytest.mark.parametrize("layout", ["aligned", "odd_ld", "offset"])
@pytest.mark.parametrize("config", TILE_CONFIGS)
@pytest.mark.parametrize("ta,tb", OPS)
def test_clamped_edge_tiles(config, ta, tb, layout):
    """Tiles that cross M or N keep the straight-line k-loop with clamped
    loads. With 16-byte-aligned operands and leading dimensions divisible by 4
    (aligned): rows past M re-read the last row, column chunks past the edge
    re-read the last aligned chunk, which may hold the NaN row padding. With
    odd leading dimensions or pointers one float off 16 bytes: the 4-byte
    instantiation clamps every element into the matrix. Only outputs beyond M
    or N see the extra values; every stored output must equal the oracle's bit
    for bit (integer inputs), with and without a k tail. The k tail (K mod 32
    of 4, 3, 1 and 6 here) is loaded the same way with the elements past K
    zeroed: a 16-byte chunk that straddles K reads NaN row padding beyond it."""
    for t, (M, N, K) in enumerate([(100, 76, 96), (5, 200, 128), (130, 3, 64), (100, 76, 100), (257, 129, 36),
                                   (100, 76, 99), (70, 130, 37), (66, 200, 102)]):
        case = W.Case(f"clamp_{layout}_{ta}{tb}_{M}x{N}x{K}_cfg{config}", ta, tb, M, N, K, 1.0 if t % 2 else 2.0,
                      0.0 if t % 2 else -1.0, seed=500 + t, fill="int_rand")
        note(case.name)
        inp = W.make_inputs(case)
        if layout == "odd_ld":
            lda, ldb, ldc = (_padded_ld(x.shape) + 1 for x in (inp.A, inp.B, inp.C))
        else:
            lda, ldb, ldc = (_padded_ld(x.shape) for x in (inp.A, inp.B, inp.C))
        want = run_oracle(case, inp)
        got = run_gpu(case, inp, config=config, lda=lda, ldb=ldb, ldc=ldc, offset=1 if layout == "offset" else 0)
        compare(case, got, want, True)


@pytest.mark.parametrize("ta,tb,M,N,K,layout,aligned_pick", [
    ("N", "N", 4096, 4096, 2048, "offset", "mfma32_256x256x32_w4x2"),
    ("T", "T", 4096, 4096, 1024, "odd_ld", "mfma32_256x256x32_w4x2_dl"),
    ("N", "N", 4000, 4000, 4000, "offset", "mfma32_128x256x16_w2x2"),
    ("T", "N", 4000, 4000, 2000, "odd_ld", "mfma32_128x256x16_w2x2"),
    ("N", "T", 2304, 2304, 1024, "offset", "mfma32_128x128x32_w4x2_streamk_2wg"),
    ("T", "T", 2304, 2304, 1024, "odd_ld", "mfma32_128x128x32_w4x2_streamk_2wg"),
    ("N", "N", 2048, 4096, 1024, "offset", "mfma16_128x128x32_w4x2"),
    ("T", "N", 2048, 4096, 1024, "odd_ld", "mfma16_128x128x32_w4x2"),
    ("T", "T", 2048, 4096, 1024, "offset", "mfma16_128x128x32_w4x2"),
    ("N", "T", 2048, 4096, 1024, "offset", "mfma16_128x128x32_w4x2"),
    ("N", "N", 2000, 2000, 2001, "odd_ld", "mfma16_128x128x32_w4x2"),
    ("N", "N", 3072, 3072, 1024, "offset", "mfma16_192x192x32_w4x3"),
    ("N", "N", 3328, 2560, 1000, "odd_ld", "mfma16_128x128x32_w4x2_streamk_2wg"),
    ("T", "N", 2048, 2048, 2048, "offset", "mfma16_128x128x32_w4x2_kg2"),
    ("T", "T", 3000, 2900, 700, "odd_ld", "mfma16_192x192x32_w4x3"),
])
def test_unaligned_operands_on_substituted_tiles(ta, tb, M, N, K, layout, aligned_pick):
    """Shapes whose pick for 16-byte-loadable operands is a tile without a
    4-byte straight-line form for that op pair (the 256 x 256, 192 x 192 and
    128 x 256 x 16 tiles, the two-workgroup stream-K tiles, the 16 x 16
    128 x 128 w4x2 tile except NT): with unaligned operands mi_sgemm runs a
    substitute with 4-byte straight-line rounds. Bit-exact on integer inputs."""
    assert mg.config_names()[mg.mi_sgemm_select_config(ta, tb, M, N, K)] == aligned_pick
    case = W.Case(f"unaligned_{layout}_{ta}{tb}_{M}x{N}x{K}", ta, tb, M, N, K, 1.0, -1.0, seed=61, fill="int_rand")
    note(case.name)
    inp = W.make_inputs(case)
    if layout == "odd_ld":
        lda, ldb, ldc = (x.shape[1] + 1 for x in (inp.A, inp.B, inp.C))
        got = run_gpu(case, inp, lda=lda, ldb=ldb, ldc=ldc)
    else:
        got = run_gpu(case, inp, offset=1)
    compare(case, got, run_oracle(case, inp), True)


@pytest.mark.parametrize("config", range(NCONFIG))
@pytest.mark.parametrize("ta,tb", OPS)
def test_every_config_uniform_medium(config, ta, tb):
    case = W.Case(f"medium_{ta}{tb}_cfg{config}", ta, tb, 333, 517, 429, 1.5, 0.5, seed=77)
    note(case.name)
    inp = W.make_inputs(case)
    compare(case, run_gpu(case, inp, config=config), run_oracle(case, inp), False)


# --- the vector-ALU technique ladder at the workload shapes ---------------------------------

LADDER = [i for i, n in enumerate(mg.config_names()) if n.startswith("valu_")]
LADDER_CASES = [W.C1, W.C2_INT, *[c.with_(name="int_" + c.name, fill="int_rand", alpha=2.0, beta=-1.0)
                                  for c in W.C5A]]


@pytest.mark.parametrize("case", LADDER_CASES, ids=lambda c: c.name)
@pytest.mark.parametrize("config", LADDER)
def test_ladder_workloads(config, case):
    note(f"ladder cfg{config} {case.name}")
    inp = W.make_inputs(case)
    compare(case, run_gpu(case, inp, config=config), run_oracle(case, inp), is_exact(case))


# --- layouts: leading-dimension padding, alignment, poisoned padding ------------------------

@pytest.mark.parametrize("ta,tb", OPS)
@pytest.mark.parametrize("pad,offset", [(0, 1), (3, 0), (4, 0), (5, 3), (64, 2)])
def test_padding_and_alignment(ta, tb, pad, offset):
    case = W.Case(f"ld_{ta}{tb}_p{pad}_o{offset}", ta, tb, 200, 150, 131, 1.0, 1.0, seed=9, fill="int_rand")
    note(case.name)
    inp = W.make_inputs(case)
    got = run_gpu(case, inp, lda=case.lda_ + pad, ldb=case.ldb_ + pad, ldc=case.ldc_ + pad, offset=offset)
    compare(case, got, run_oracle(case, inp), True)


def test_large_tile_path_with_padding():
    case = W.Case("ld_large", "N", "N", 2048, 2048, 256, 1.0, 0.0, seed=10, fill="int_rand")
    inp = W.make_inputs(case)
    got = run_gpu(case, inp, lda=260, ldb=2052, ldc=2056)
    compare(case, got, run_oracle(case, inp), True)


# --- IEEE special values ------------------------------------------------------------------

@pytest.mark.parametrize("config", range(NCONFIG))
@pytest.mark.parametrize("ta,tb", OPS)
def test_special_values_propagate(config, ta, tb):
    """+Inf in one entry of op(A) and NaN in one entry of op(B): the outputs
    they reach are +-Inf or NaN exactly where IEEE arithmetic puts them (the
    integer fill has zeros, so Inf * 0 = NaN occurs), and every other output
    is bit-exact."""
    M, N, K = 150, 230, 97
    i0, k0, k1, j1 = 77, 40, 61, 129
    case = W.Case(f"special_{ta}{tb}_cfg{config}", ta, tb, M, N, K, 1.0, -1.0, seed=90, fill="int_rand")
    note(case.name)
    inp = W.make_inputs(case)
    if ta == "N":
        inp.A[i0, k0] = np.inf
    else:
        inp.A[k0, i0] = np.inf
    if tb == "N":
        inp.B[k1, j1] = np.nan
    else:
        inp.B[j1, k1] = np.nan
    got = run_gpu(case, inp, config=config)
    want = run_oracle(case, inp)
    assert np.isnan(want[:, j1]).all() and np.isinf(want[i0]).any()
    assert np.array_equal(np.isnan(got), np.isnan(want)), f"{case.name}: NaN positions differ"
    inf = np.isinf(want)
    assert np.array_equal(np.isinf(got), inf), f"{case.name}: Inf positions differ"
    assert np.array_equal(np.signbit(got[inf]), np.signbit(want[inf])), f"{case.name}: Inf signs differ"
    fin = np.isfinite(want)
    assert np.array_equal(got[fin], want[fin]), f"{case.name}: finite outputs differ"


# --- BLAS semantics of the scalars and empty sizes ------------------------------------------

def test_beta_zero_ignores_nan_c():
    case = W.Case("beta0_nan", "N", "N", 300, 260, 70, 1.0, 0.0, seed=12)
    inp = W.make_inputs(case)
    inp.C[:] = np.nan
    got = run_gpu(case, inp)
    inp.C[:] = 0.0
    compare(case, got, run_oracle(case, inp), False)


@pytest.mark.parametrize("beta", [0.0, 0.5, -2.0])
def test_alpha_zero_scales_c_without_reading_ab(beta):
    case = W.Case("alpha0", "N", "T", 130, 70, 50, 0.0, beta, seed=13)
    inp = W.make_inputs(case)
    inp.C[:] = uniform_matrix(Drand48(14), 130, 70)
    inp.A[:] = np.nan
    inp.B[:] = np.nan
    got = run_gpu(case, inp)
    want = run_oracle(case, inp)
    assert np.array_equal(got, want)


def test_k_zero_scales_c():
    case = W.Case("k0", "N", "N", 100, 90, 0, 1.0, -0.5, seed=15)
    inp = W.make_inputs(case)
    inp.C[:] = uniform_matrix(Drand48(16), 100, 90)
    got = run_gpu(case, inp)
    assert np.array_equal(got, run_oracle(case, inp))


def test_alpha_zero_beta_one_leaves_c():
    case = W.Case("noop", "N", "N", 64, 64, 64, 0.0, 1.0, seed=17)
    inp = W.make_inputs(case)
    inp.C[:] = np.nan
    got = run_gpu(case, inp)
    assert np.all(np.isnan(got))


@pytest.mark.parametrize("M,N", [(0, 5), (5, 0), (0, 0)])
def test_empty_output(M, N):
    C = torch.full((16,), 7.0, device="cuda")
    rc = mg.mi_sgemm("N", "N", M, N, 3, 1.0, 0, 3, 0, max(N, 1), 0.0, C.data_ptr(), max(N, 1),
                     torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0 and bool(torch.all(C == 7.0))


# --- determinism ------------------------------------------------------------------------------

@pytest.mark.parametrize("case", [W.C4, W.C5A[3], W.C5B, W.C1], ids=lambda c: c.name)
def test_run_to_run_bitwise(case):
    inp = W.make_inputs(case)
    a = run_gpu(case, inp)
    b = run_gpu(case, inp)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# --- the torch-tensor wrapper ---------------------------------------------------------------

def test_tensor_wrapper_matches_oracle():
    case = W.Case("wrapper", "T", "N", 257, 129, 65, 1.5, 0.5, seed=18)
    inp = W.make_inputs(case)
    A = torch.from_numpy(inp.A).cuda()
    B = torch.from_numpy(inp.B).cuda()
    C = torch.from_numpy(inp.C.copy()).cuda()
    mg.sgemm("T", "N", 1.5, A, B, 0.5, C)
    torch.cuda.synchronize()
    compare(case, C.cpu().numpy(), run_oracle(case, inp), False)
    with pytest.raises(ValueError):
        mg.sgemm("N", "N", 1.0, A, B, 0.0, C)         # shapes do not chain
