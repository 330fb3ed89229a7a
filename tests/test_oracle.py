"""Pins for the CPU oracle against facts fixed outside the oracle itself.

The oracle computes C <- alpha*op(A)*op(B) + beta*C with an FP64 sum in
ascending k and one rounding to FP32. Each test below pins it to something
independent of its own code: exact rational arithmetic (brute force), exact
integer products from numpy, closed forms, transpose identities and a float64
library product.
"""
import os
import subprocess
import sys
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synthetic import Drand48, padded, uniform_matrix
from synthetic import workloads as W

OPS = [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]


# --- helpers ---------------------------------------------------------------------

def stored(rows, cols, trans):
    """Shape of the stored matrix for op(X) of logical size rows x cols."""
    return (rows, cols) if trans == "N" else (cols, rows)


def run(ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc):
    rc = oracle.sgemm(ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc)
    assert rc == 0
    return C


def round_to_f32(fr: Fraction) -> np.float32:
    """Correctly rounded (nearest, ties to even) float32 of an exact rational."""
    if fr == 0:
        return np.float32(0.0)
    x = np.float32(float(fr))
    cands = [np.nextafter(x, np.float32(-np.inf)), x, np.nextafter(x, np.float32(np.inf))]
    best, bestd = None, None
    for c in cands:
        d = abs(Fraction(float(c)) - fr)
        if best is None or d < bestd or (d == bestd and (int(c.view(np.uint32)) & 1) == 0):
            best, bestd = c, d
    return best


def ordered(a):
    i = np.asarray(a, dtype=np.float32).view(np.int32).astype(np.int64)
    return np.where(i < 0, -(2**31) - i, i)


def ulp_diff(a, b):
    return np.abs(ordered(a) - ordered(b))


def frac_matrix(x):
    return np.array([[Fraction(float(v)) for v in row] for row in x], dtype=object).reshape(x.shape)


# --- P1: brute force in exact rational arithmetic --------------------------------

@pytest.mark.parametrize("ta,tb", OPS)
def test_bruteforce_rational(ta, tb):
    bruteforce(ta, tb, trials=30)


def bruteforce(ta, tb, trials):
    rng = np.random.default_rng(1000 + 7 * OPS.index((ta, tb)))
    scalars = [0.0, 1.0, -1.0, 0.5, 1.5, 2.0, -0.75]
    exact_hits = total = 0
    for trial in range(trials):
        M, N, K = (int(v) for v in rng.integers(1, 13 if trial % 3 else 18, 3))
        alpha = float(rng.choice(scalars))
        beta = float(rng.choice(scalars))
        ar, ac = stored(M, K, ta)
        br, bc = stored(K, N, tb)
        # Mixed magnitudes so that rounding matters.
        a = (rng.standard_normal((ar, ac)) * 2.0 ** rng.integers(-6, 7, (ar, ac))).astype(np.float32)
        b = (rng.standard_normal((br, bc)) * 2.0 ** rng.integers(-6, 7, (br, bc))).astype(np.float32)
        c = (rng.standard_normal((M, N)) * 4).astype(np.float32)
        lda, ldb, ldc = ac + int(rng.integers(0, 3)), bc + int(rng.integers(0, 3)), N + int(rng.integers(0, 3))
        # Padding is NaN: any read of it shows up as NaN in C.
        Ab = padded(a, lda, fill=np.nan, extra_rows=1)
        Bb = padded(b, ldb, fill=np.nan, extra_rows=1)
        c_in = c.copy()
        if beta == 0.0:
            c_in[:] = np.nan                       # must not be read
        if alpha == 0.0:
            Ab[:] = np.nan                         # must not be read
            Bb[:] = np.nan
        Cb = padded(c_in, ldc, fill=-7.0, extra_rows=1)
        run(ta, tb, M, N, K, alpha, Ab, lda, Bb, ldb, beta, Cb, ldc)
        # Padding and guard row of C untouched.
        assert np.all(Cb[:M, N:] == -7.0) and np.all(Cb[M:] == -7.0)
        got = Cb[:M, :N]

        fa = frac_matrix(a)
        fb = frac_matrix(b)
        opa = fa if ta == "N" else fa.T
        opb = fb if tb == "N" else fb.T
        for i in range(M):
            for j in range(N):
                s = sum((opa[i, k] * opb[k, j] for k in range(K)), Fraction(0))
                ex = (Fraction(alpha) * s if alpha != 0.0 else Fraction(0)) + \
                     (Fraction(beta) * Fraction(float(c[i, j])) if beta != 0.0 else Fraction(0))
                want = round_to_f32(ex)
                assert ulp_diff(got[i, j], want) <= 1, (trial, i, j, got[i, j], want)
                exact_hits += int(got[i, j] == want)
                total += 1
    # FP64 accumulation then one rounding: correctly rounded except for rare
    # double-rounding cases.
    assert exact_hits >= 0.999 * total, (exact_hits, total)


# --- P2: exact integer products ---------------------------------------------------

def _exact_int_product(case, inp):
    """alpha*op(A)op(B) + beta*C in float64: exact for these integer inputs."""
    a = inp.A.astype(np.float64)
    b = inp.B.astype(np.float64)
    opa = a if case.transA == "N" else a.T
    opb = b if case.transB == "N" else b.T
    out = case.alpha * (opa @ opb)
    if case.beta != 0.0:
        out = out + case.beta * inp.C.astype(np.float64)
    assert np.abs(out).max() < 2**24            # every value exact in float32
    return out.astype(np.float32)


def _oracle_case(case, inp):
    C = inp.C.copy()
    return run(case.transA, case.transB, case.M, case.N, case.K, case.alpha, inp.A, case.lda_,
               inp.B, case.ldb_, case.beta, C, case.ldc_)


@pytest.mark.parametrize("case", [
    W.C2_INT,
    W.C2.with_(name="int_floor_1024", fill="int_floor"),
    W.C1.with_(name="int_c1", fill="int_trunc"),
    W.C1.with_(name="int_rand_c1", fill="int_rand", alpha=2.0, beta=-1.0),
    W.C5B.with_(name="int_skinny", fill="int_rand", K=1024),
] + [W.C5A[i].with_(name=f"int_op{i}", M=300, N=400, K=250, fill="int_rand", alpha=2.0, beta=-1.0)
     for i in range(4)], ids=lambda c: c.name)
def test_integer_inputs_exact(case):
    inp = W.make_inputs(case)
    got = _oracle_case(case, inp)
    want = _exact_int_product(case, inp)
    assert np.array_equal(got, want)


def test_integer_vs_int64_matmul():
    g = Drand48(11)
    a = np.floor(g.drand48(90 * 70) * 9).reshape(90, 70).astype(np.int64) - 4
    b = np.floor(g.drand48(70 * 110) * 9).reshape(70, 110).astype(np.int64) - 4
    want = a @ b
    got = oracle.matmul("N", "N", 1.0, a.astype(np.float32), b.astype(np.float32))
    assert np.array_equal(got.astype(np.int64), want)


# --- P3: closed forms ----------------------------------------------------------------

@pytest.mark.parametrize("ta", ["N", "T"])
def test_identity(ta):
    B = uniform_matrix(Drand48(21), 64, 48)
    I = np.eye(64, dtype=np.float32)
    got = oracle.matmul(ta, "N", 1.0, I, B)
    assert np.array_equal(got, B)


def test_permutation_rows_and_columns():
    # A = P (a non-symmetric permutation): C = P B permutes rows of B. A swapped
    # index or a transposed operand would apply P^T instead.
    rng = np.random.default_rng(3)
    perm = rng.permutation(40)
    P = np.zeros((40, 40), np.float32)
    P[np.arange(40), perm] = 1.0
    B = uniform_matrix(Drand48(22), 40, 33)
    assert np.array_equal(oracle.matmul("N", "N", 1.0, P, B), B[perm])
    assert np.array_equal(oracle.matmul("T", "N", 1.0, P, B), B[np.argsort(perm)])
    Q = np.eye(33, dtype=np.float32)[rng.permutation(33)]
    # B Q permutes columns.
    qcols = np.argmax(Q, axis=0)
    assert np.array_equal(oracle.matmul("N", "N", 1.0, B, Q), B[:, qcols])


def test_ramp_closed_form():
    M, N, K = 17, 23, 301
    A = np.ones((M, K), np.float32)
    k = np.arange(K)[:, None]
    j = np.arange(N)[None, :]
    B = (k - j).astype(np.float32)                      # B(k,j) = k - j
    got = oracle.matmul("N", "N", 1.0, A, B)
    want = K * (K - 1) // 2 - K * np.arange(N)          # sum_k (k - j)
    assert np.array_equal(got, np.broadcast_to(want.astype(np.float32), (M, N)))


def test_zero_A_gives_beta_c():
    C = uniform_matrix(Drand48(23), 20, 30)
    got = oracle.matmul("N", "N", 1.0, np.zeros((20, 9), np.float32), uniform_matrix(Drand48(24), 9, 30), 0.5, C)
    assert np.array_equal(got, C * np.float32(0.5))


def test_k_zero_and_alpha_zero_scale_c():
    C = uniform_matrix(Drand48(25), 12, 13)
    Cb = C.copy()
    run("N", "N", 12, 13, 0, 1.0, None, 1, None, 13, -2.0, Cb, 13)
    assert np.array_equal(Cb, C * np.float32(-2.0))
    nanA = np.full((12, 5), np.nan, np.float32)
    nanB = np.full((5, 13), np.nan, np.float32)
    Cb = C.copy()
    run("N", "N", 12, 13, 5, 0.0, nanA, 5, nanB, 13, 1.5, Cb, 13)   # A, B not read
    assert np.array_equal(Cb, (C.astype(np.float64) * 1.5).astype(np.float32))
    Cb = np.full((12, 13), np.nan, np.float32)
    run("N", "N", 12, 13, 5, 0.0, nanA, 5, nanB, 13, 0.0, Cb, 13)   # beta = 0: zeros
    assert np.all(Cb == 0.0)


def test_beta_zero_does_not_read_c():
    A = uniform_matrix(Drand48(26), 8, 7)
    B = uniform_matrix(Drand48(27), 7, 9)
    ref = oracle.matmul("N", "N", 1.0, A, B)
    Cn = np.full((8, 9), np.nan, np.float32)
    run("N", "N", 8, 9, 7, 1.0, A, 7, B, 9, 0.0, Cn, 9)
    assert np.array_equal(Cn, ref)


def test_empty_shapes_are_no_ops():
    C = np.full((4, 4), 3.0, np.float32)
    assert oracle.sgemm("N", "N", 0, 4, 4, 1.0, None, 4, None, 4, 0.0, C, 4) == 0
    assert oracle.sgemm("N", "N", 4, 0, 4, 1.0, None, 4, None, 1, 0.0, C, 4) == 0
    assert np.all(C == 3.0)


def test_fp64_accumulation():
    # 2^24 + 1 is not a float: an FP32 running sum loses the 1; FP64 keeps it.
    A = np.ones((1, 3), np.float32)
    B = np.array([[2.0**24], [1.0], [-(2.0**24)]], np.float32)
    assert oracle.matmul("N", "N", 1.0, A, B)[0, 0] == 1.0
    B2 = np.array([[1.0], [2.0**24], [-(2.0**24)]], np.float32)
    assert oracle.matmul("N", "N", 1.0, A, B2)[0, 0] == 1.0


def test_single_final_rounding():
    # s = 1 + 2^-24 (exact in FP64), beta*c = 2^-25: the exact result
    # 1 + 3*2^-25 rounds to 1 + 2^-23. Rounding s to float first (a tie, to
    # even: 1.0) and then adding would give 1.0.
    A = np.array([[1.0, 2.0**-12]], np.float32)
    B = np.array([[1.0], [2.0**-12]], np.float32)
    C = np.array([[2.0**-25]], np.float32)
    got = oracle.matmul("N", "N", 1.0, A, B, 1.0, C)[0, 0]
    assert got == np.float32(1.0 + 2.0**-23)


# --- P4: transpose identities ------------------------------------------------------

def _rand_case(seed, M, N, K):
    g = Drand48(seed)
    return uniform_matrix(g, M, K), uniform_matrix(g, K, N), uniform_matrix(g, M, N)


def test_transpose_of_product_bit_exact():
    M, N, K = 37, 53, 29
    A, B, C = _rand_case(31, M, N, K)
    ref = oracle.matmul("N", "N", 1.5, A, B, 0.5, C)
    # (AB)^T = B^T A^T: call with transA = transB = 'T' on the stored B and A.
    got = oracle.matmul("T", "T", 1.5, B, A, 0.5, C.T.copy())
    assert np.array_equal(got.T, ref)


@pytest.mark.parametrize("ta,tb", OPS)
def test_explicit_transposed_copies(ta, tb):
    M, N, K = 41, 19, 66
    A, B, C = _rand_case(32, M, N, K)
    ref = oracle.matmul("N", "N", -1.25, A, B, 2.0, C)
    As = A if ta == "N" else A.T.copy()
    Bs = B if tb == "N" else B.T.copy()
    assert np.array_equal(oracle.matmul(ta, tb, -1.25, As, Bs, 2.0, C), ref)


def test_lowercase_and_conjugate_trans_letters():
    A, B, C = _rand_case(33, 9, 10, 11)
    ref = oracle.matmul("T", "N", 1.0, A.T.copy(), B)
    for t in ("t", "C", "c"):
        assert np.array_equal(oracle.matmul(t, "n", 1.0, A.T.copy(), B), ref)


# --- P5: float64 library cross-check at a real size ----------------------------------

def test_against_float64_library_product():
    case = W.C1
    inp = W.make_inputs(case)
    got = _oracle_case(case, inp)
    want = (inp.A.astype(np.float64) @ inp.B.astype(np.float64)).astype(np.float32)
    d = ulp_diff(got, want)
    close = np.abs(got.astype(np.float64) - want.astype(np.float64)) <= 1e-9
    assert np.all((d <= 1) | close), int(d.max())


def test_against_float64_library_product_all_ops_alpha_beta():
    for i, base in enumerate(W.C5A):
        case = base.with_(M=129, N=67, K=300, alpha=1.5, beta=-0.5)
        inp = W.make_inputs(case)
        got = _oracle_case(case, inp)
        a = inp.A.astype(np.float64)
        b = inp.B.astype(np.float64)
        opa = a if case.transA == "N" else a.T
        opb = b if case.transB == "N" else b.T
        want = (1.5 * (opa @ opb) - 0.5 * inp.C.astype(np.float64)).astype(np.float32)
        d = ulp_diff(got, want)
        close = np.abs(got.astype(np.float64) - want.astype(np.float64)) <= 1e-9
        assert np.all((d <= 1) | close), (case.name, int(d.max()))


# --- sampled entries and thread independence ----------------------------------------

def test_entries_match_full_product():
    case = W.C5A[2].with_(M=150, N=170, K=90, beta=0.75)
    inp = W.make_inputs(case)
    full = _oracle_case(case, inp)
    rng = np.random.default_rng(5)
    r = rng.integers(0, case.M, 300)
    c = rng.integers(0, case.N, 300)
    got = oracle.sgemm_entries(case.transA, case.transB, case.M, case.N, case.K, case.alpha,
                               inp.A, case.lda_, inp.B, case.ldb_, case.beta, inp.C[r, c], r, c)
    assert np.array_equal(got, full[r, c])


def test_thread_count_does_not_change_result(tmp_path):
    code = (
        "import sys, hashlib, numpy as np; sys.path.insert(0, %r);"
        "import oracle; from synthetic import workloads as W;"
        "c = W.C5A[1].with_(M=200, N=190, K=170); i = W.make_inputs(c); C = i.C.copy();"
        "oracle.sgemm(c.transA, c.transB, c.M, c.N, c.K, c.alpha, i.A, c.lda_, i.B, c.ldb_, c.beta, C, c.ldc_);"
        "print(hashlib.sha256(C.tobytes()).hexdigest(), oracle.num_threads())"
    ) % os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    outs = []
    for threads in ("1", "3", "8"):
        env = dict(os.environ, OMP_NUM_THREADS=threads)
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, check=True)
        h, n = r.stdout.split()
        assert n == threads
        outs.append(h)
    assert len(set(outs)) == 1


# --- argument checking ------------------------------------------------------------------

def test_argument_errors():
    A = np.zeros((4, 4), np.float32)
    C = np.zeros((4, 4), np.float32)
    s = oracle.sgemm
    assert s("X", "N", 4, 4, 4, 1.0, A, 4, A, 4, 0.0, C, 4) == -1
    assert s("N", "Q", 4, 4, 4, 1.0, A, 4, A, 4, 0.0, C, 4) == -2
    assert s("N", "N", -1, 4, 4, 1.0, A, 4, A, 4, 0.0, C, 4) == -3
    assert s("N", "N", 4, -1, 4, 1.0, A, 4, A, 4, 0.0, C, 4) == -4
    assert s("N", "N", 4, 4, -1, 1.0, A, 4, A, 4, 0.0, C, 4) == -5
    assert s("N", "N", 4, 4, 4, 1.0, None, 4, A, 4, 0.0, C, 4) == -7
    assert s("N", "N", 4, 4, 5, 1.0, A, 4, A, 4, 0.0, C, 4) == -8
    assert s("T", "N", 5, 4, 4, 1.0, A, 4, A, 4, 0.0, C, 5) == -8
    assert s("N", "N", 4, 4, 4, 1.0, A, 4, None, 4, 0.0, C, 4) == -9
    assert s("N", "N", 4, 5, 4, 1.0, A, 4, A, 4, 0.0, C, 5) == -10
    assert s("N", "T", 4, 4, 5, 1.0, A, 5, A, 4, 0.0, C, 4) == -10
    assert s("N", "N", 4, 4, 4, 1.0, A, 4, A, 4, 0.0, None, 4) == -12
    assert s("N", "N", 4, 4, 4, 1.0, A, 4, A, 4, 0.0, C, 3) == -13
