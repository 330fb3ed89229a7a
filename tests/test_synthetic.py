"""The seeded input generator: POSIX drand48 stream and the fills."""
import ctypes

import numpy as np
import pytest

from synthetic import Drand48, int_pattern_matrix, padded, uniform_matrix
from synthetic import workloads as W


def _libc_drand48(seed, count):
    libc = ctypes.CDLL("libc.so.6")
    libc.drand48.restype = ctypes.c_double
    libc.srand48(ctypes.c_long(seed))
    return np.array([libc.drand48() for _ in range(count)])


@pytest.mark.parametrize("seed", [0, 1, 2, 5, 12345, 2**31 - 1, 2**32 + 3])
def test_stream_matches_libc(seed):
    """The vectorised jump-ahead reproduces glibc's drand48 draw for draw."""
    ref = _libc_drand48(seed, 3000)
    g = Drand48(seed)
    got = np.concatenate([g.drand48(1), g.drand48(999), g.drand48(2000)])
    assert np.array_equal(got, ref)


def test_posix_first_values():
    # srand48(1) sets X0 = 0x1330E; one step of X <- 0x5DEECE66D*X + 0xB mod 2^48.
    x1 = (0x5DEECE66D * 0x1330E + 0xB) % 2**48
    assert Drand48(1).drand48(1)[0] == x1 / 2**48


def test_uniform_grid_and_range():
    g = Drand48(7)
    a = uniform_matrix(g, 300, 257)
    assert a.dtype == np.float32 and a.shape == (300, 257)
    assert a.min() >= -1.0 and a.max() <= 1.0 - 2.0**-23
    scaled = (a.astype(np.float64) + 1.0) * 2.0**23
    assert np.array_equal(scaled, np.round(scaled))          # on the 2^-23 grid
    assert abs(float(a.mean())) < 0.01                         # centred
    assert 0.32 < float(a.var()) < 0.345                       # var of U[-1,1) = 1/3


def test_uniform_is_quantised_drand48():
    u = Drand48(3).drand48(1000)
    a = uniform_matrix(Drand48(3), 10, 100).ravel()
    expect = (np.floor(u * 2**24) * 2.0**-23 - 1.0).astype(np.float32)
    assert np.array_equal(a, expect)


def test_seed_determinism_and_order():
    c = W.C5B
    x, y = W.make_inputs(c), W.make_inputs(c)
    assert np.array_equal(x.A, y.A) and np.array_equal(x.B, y.B) and np.array_equal(x.C, y.C)
    g = Drand48(c.seed)
    a = uniform_matrix(g, *c.a_shape)
    b = uniform_matrix(g, *c.b_shape)
    cc = uniform_matrix(g, c.M, c.N)
    assert np.array_equal(a, x.A) and np.array_equal(b, x.B) and np.array_equal(cc, x.C)


def test_int_pattern_values():
    t = int_pattern_matrix(6, 7)
    f = int_pattern_matrix(6, 7, floored=True)
    assert t[0, 1] == 1 and t[1, 0] == -1 and t[0, 5] == 2 and t[5, 0] == -2 and t[3, 3] == 0
    assert f[1, 0] == 2 and f[5, 0] == 1 and f[0, 5] == 2
    assert set(np.unique(t)) <= {-2.0, -1.0, 0.0, 1.0, 2.0}
    assert set(np.unique(f)) <= {0.0, 1.0, 2.0}


def test_padded_layout():
    m = np.arange(6, dtype=np.float32).reshape(2, 3)
    p = padded(m, 5, fill=np.nan, extra_rows=1)
    assert p.shape == (3, 5) and np.array_equal(p[:2, :3], m) and np.isnan(p[:2, 3:]).all()


def test_workload_metrics():
    assert W.C4.flops == 2 * 4096**3
    # 1024^3, beta = 0: 4(MK + KN + MN) bytes = 12,582,912 B, the minimum the
    # itan.pw page's bound analysis (section 2.1) prints for this shape.
    assert W.C2.algorithmic_bytes == 12_582_912
    assert W.C5B.algorithmic_bytes == 4 * (16 * 4096 + 4096 * 4096 + 2 * 16 * 4096)
    names = [c.name for c in W.all_cases()]
    assert len(names) == len(set(names)) == 3 + 16 + 1 + 4 + 1
