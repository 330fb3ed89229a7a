"""The C-ABI library on the host: exports, argument checks, shape-class choice.

Nothing here launches a kernel: every call below either fails validation or
takes a quick return, both of which happen before any HIP call.
"""
import ctypes
import os
import re

import pytest

import fp32_gemm_nn_amd as mg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h")]


def declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \*]*?\b(mi_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


def test_header_declares_entry_points():
    names = declared_functions()
    assert "mi_sgemm" in names and "mi_sgemm_status_string" in names
    assert len(names) >= 6


@pytest.mark.parametrize("name", declared_functions())
def test_every_declared_symbol_is_exported(name):
    lib = ctypes.CDLL(mg.library_path)
    assert hasattr(lib, name)


def test_library_exports_nothing_undeclared():
    out = os.popen(f"nm -D --defined-only {mg.library_path}").read()
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    ours = {s for s in exported if s.startswith("mi_")}
    assert ours == set(declared_functions())


GOOD = dict(transA="N", transB="N", M=4, N=4, K=4, alpha=1.0, A=0x1000, lda=4, B=0x2000, ldb=4,
            beta=0.0, C=0x3000, ldc=4)


def call(**kw):
    a = dict(GOOD)
    a.update(kw)
    return mg.mi_sgemm(a["transA"], a["transB"], a["M"], a["N"], a["K"], a["alpha"], a["A"], a["lda"],
                       a["B"], a["ldb"], a["beta"], a["C"], a["ldc"], 0)


@pytest.mark.parametrize("kw,code", [
    (dict(transA="X"), -1), (dict(transB="q"), -2),
    (dict(M=-1), -3), (dict(N=-2), -4), (dict(K=-3), -5),
    (dict(A=0), -7), (dict(lda=3), -8), (dict(transA="T", M=5, lda=4, ldc=4), -8),
    (dict(B=0), -9), (dict(ldb=3), -10), (dict(transB="t", K=6, lda=6), -10),
    (dict(C=0), -12), (dict(ldc=3), -13),
    # First bad argument wins, in parameter order.
    (dict(transA="X", M=-1, ldc=0), -1), (dict(M=-1, ldc=0), -3), (dict(lda=0, ldc=0), -8),
])
def test_argument_errors(kw, code):
    assert call(**kw) == code
    assert mg.mi_sgemm_status_string(code) not in ("", "unknown status")


def test_quick_returns_do_not_launch():
    # M == 0 or N == 0: success, pointers never touched (null is fine).
    assert call(M=0, A=0, B=0, C=0) == 0
    assert call(N=0, A=0, B=0, C=0, ldb=1, ldc=1) == 0
    # alpha == 0 or K == 0 with beta == 1: C unchanged, nothing enqueued; A, B may be null.
    assert call(alpha=0.0, beta=1.0, A=0, B=0) == 0
    assert call(K=0, beta=1.0, A=0, B=0, lda=1) == 0


def test_null_ab_allowed_when_not_read_but_c_required():
    assert call(alpha=0.0, beta=1.0, A=0, B=0, C=0) == -12


def test_too_large_leading_dimension():
    assert call(lda=2**30) == mg.MisgemmError(-21).status
    assert "too large" in mg.mi_sgemm_status_string(-21)


def test_config_table():
    n = mg.mi_sgemm_config_count()
    assert n >= 2
    names = mg.config_names()
    assert len(set(names)) == n and all(names)
    assert mg.mi_sgemm_config_name(n) is None and mg.mi_sgemm_config_name(-1) is None


def test_with_config_rejects_unknown_id():
    a = dict(GOOD)
    args = [a[k] for k in ("transA", "transB", "M", "N", "K", "alpha", "A", "lda", "B", "ldb", "beta", "C", "ldc")]
    n = mg.mi_sgemm_config_count()
    assert mg.mi_sgemm_with_config(n, *args, 0) == -20
    assert mg.mi_sgemm_with_config(-1, *args, 0) == -20
    # Argument errors still come first.
    args[2] = -1
    assert mg.mi_sgemm_with_config(n, *args, 0) == -3


def test_selection_fuzz():
    """Seeded random shapes: the pick is always a valid matrix-core
    configuration (never a vector-ALU ladder rung), the band kernel exactly
    when M <= 32 and N >= 128, and the direct-to-LDS 256 x 256 tile only with
    A transposed."""
    import random

    names = mg.config_names()
    rng = random.Random(5)
    for _ in range(5000):
        M = rng.choice([rng.randint(1, 64), rng.randint(1, 5000), rng.randint(1, 20000)])
        N = rng.choice([rng.randint(1, 256), rng.randint(1, 5000), rng.randint(1, 20000)])
        K = rng.choice([rng.randint(0, 64), rng.randint(1, 5000), rng.randint(1, 20000)])
        ta, tb = rng.choice("NnTtCc"), rng.choice("NnTtCc")
        c = mg.mi_sgemm_select_config(ta, tb, M, N, K)
        assert 0 <= c < len(names), (ta, tb, M, N, K, c)
        name = names[c]
        assert not name.startswith("valu_"), (ta, tb, M, N, K, name)
        assert ("band" in name) == (M <= 32 and N >= 128), (ta, tb, M, N, K, name)
        if name.endswith("_dl"):
            assert ta in "TtCc" and name == "mfma32_256x256x32_w4x2_dl", (ta, tb, M, N, K, name)
        # With A transposed the 256 x 256 tile takes its direct-to-LDS form
        # (the register-staged one spills for TT and is slower for TN).
        if ta in "TtCc":
            assert name != "mfma32_256x256x32_w4x2", (ta, tb, M, N, K, name)
        # The 16 x 16 two-workgroup stream-K tile only with neither operand
        # transposed (its TT form spills).
        if name == "mfma16_128x128x32_w4x2_streamk_2wg":
            assert ta in "Nn" and tb in "Nn", (ta, tb, M, N, K, name)


def test_shape_class_selection():
    names = mg.config_names()
    sel = lambda *s: names[mg.mi_sgemm_select_config(*s)]
    # 4096^2 output: 256 tiles of 256 x 256, one per CU.
    assert sel("N", "N", 4096, 4096, 4096) == "mfma32_256x256x32_w4x2"
    assert sel("N", "T", 4096, 4096, 4096) == "mfma32_256x256x32_w4x2"
    # A transposed: the 256 x 256 tile with direct-to-LDS loads.
    assert sel("T", "N", 4096, 4096, 4096) == "mfma32_256x256x32_w4x2_dl"
    assert sel("T", "N", 8192, 8192, 2048) == "mfma32_256x256x32_w4x2_dl"
    assert sel("T", "T", 4096, 4096, 4096) == "mfma32_256x256x32_w4x2_dl"
    assert sel("T", "T", 4096, 4096, 1024) == "mfma32_256x256x32_w4x2_dl"
    assert sel("T", "T", 2048, 4096, 2048) == "mfma32_256x128x32_w4x2"
    # A 256 x 256 grid that does not divide M and N: its edge tiles run guarded,
    # so a tile whose edges clamp their loads wins.
    assert sel("N", "N", 4000, 4000, 4000) == "mfma32_128x256x16_w2x2"
    assert sel("T", "T", 4000, 4000, 4000) == "mfma32_256x128x32_w4x2"
    assert sel("N", "N", 3800, 4000, 4000) == "mfma32_128x256x16_w2x2"
    # 128 x 128 and 64 x 64 tiles run as 16 x 16 MFMA blocks, for every op pair;
    # one round of 128 x 128 tiles with K >= 2048 as two k-groups of eight waves.
    assert sel("T", "N", 2048, 2048, 2048) == "mfma16_128x128x32_w4x2_kg2"
    assert sel("T", "N", 2048, 2048, 4096) == "mfma16_128x128x32_w4x2_kg2"
    assert sel("N", "N", 2048, 2048, 2048) == "mfma16_128x128x32_w4x2_kg2"
    assert sel("N", "N", 2048, 2048, 1024) == "mfma16_128x128x32_w4x2"
    # 2048 x 4096 x 1024: short K on a grid that fills the chip once: 128 x 128
    # (two workgroups per CU), for every op pair.
    assert sel("N", "N", 2048, 4096, 1024) == "mfma16_128x128x32_w4x2"
    assert sel("T", "N", 2048, 4096, 1024) == "mfma16_128x128x32_w4x2"
    assert sel("N", "N", 2048, 4096, 2048) == "mfma32_128x256x32_w2x4"
    assert sel("T", "T", 2048, 4096, 1024) == "mfma16_128x128x32_w4x2"
    assert sel("N", "T", 2048, 4096, 1024) == "mfma16_128x128x32_w4x2"
    # 1024^2 output: 64 tiles of 128 x 128 only, so smaller tiles with four k-groups.
    # Four k-groups of two waves where the grid fills at least 224 CUs, A is not
    # transposed and K has no tail; of four waves otherwise.
    assert sel("N", "N", 1024, 1024, 1024) == "mfma16_64x64x32_w2x1_kg4"
    assert sel("N", "T", 1024, 1024, 1024) == "mfma16_64x64x32_w2x1_kg4"
    assert sel("T", "N", 1024, 1024, 1024) == "mfma16_64x64x32_w2x2_kg4"
    assert sel("N", "N", 1024, 1024, 1000) == "mfma16_64x64x32_w2x2_kg4"
    assert sel("N", "N", 1024, 896, 1024) == "mfma16_64x64x32_w2x1_kg4"
    assert sel("N", "N", 1024, 832, 1024) == "mfma16_64x64x32_w2x2_kg4"
    assert sel("N", "N", 1000, 1300, 700) == "mfma16_64x64x32_w2x2_splitk"
    # 257..511 tiles of 64 x 64 filling 75-85% of two slots per CU, with enough
    # k-work and B not transposed: stream-K over 128 x 128 tiles; fuller grids,
    # short k or transposed B: two k-groups.
    assert sel("N", "N", 1280, 1280, 1280) == "mfma16_128x128x32_w4x2_streamk_1wg"
    assert sel("T", "N", 1280, 1280, 2560) == "mfma16_128x128x32_w4x2_streamk_1wg"
    assert sel("N", "N", 1536, 1024, 1024) == "mfma16_128x128x32_w4x2_streamk_1wg"
    assert sel("T", "T", 1280, 1280, 1280) == "mfma16_64x64x32_w2x2_kg2"
    assert sel("N", "T", 1280, 1280, 1280) == "mfma16_64x64x32_w2x2_kg2"
    assert sel("N", "N", 1280, 1280, 640) == "mfma16_64x64x32_w2x2_kg2"
    assert sel("N", "N", 1408, 1408, 1408) == "mfma16_64x64x32_w2x2_kg2"
    # ... but split-K where the 64 x 64 timing model splits k (384 tiles, K <= 1024).
    assert sel("T", "T", 2048, 768, 1024) == "mfma16_64x64x32_w2x2_splitk"
    assert sel("N", "N", 1536, 1024, 512) == "mfma16_64x64x32_w2x2_splitk"
    assert sel("N", "N", 1792, 1024, 1024) == "mfma16_64x64x32_w2x2_kg2"
    assert sel("N", "N", 512, 512, 512) == "mfma16_64x64x32_w2x2_splitk"
    # Up to 256 tiles of 64 x 64: split-K where the 64 x 64 timing model puts
    # it ahead of four k-groups (short grids, long K).
    assert sel("N", "N", 768, 768, 768) == "mfma16_64x64x32_w2x2_splitk"
    assert sel("T", "T", 832, 832, 832) == "mfma16_64x64x32_w2x2_splitk"
    assert sel("N", "N", 2048, 256, 2048) == "mfma16_64x64x32_w2x2_splitk"
    assert sel("N", "N", 960, 960, 960) == "mfma16_64x64x32_w2x1_kg4"
    # 361 tiles fill under 75% of two slots per CU: split-K.
    assert sel("N", "N", 1216, 1216, 1216) == "mfma16_64x64x32_w2x2_splitk"
    # 144..255 tiles of 128 x 128 with enough k-work: stream-K, one workgroup per CU.
    assert sel("N", "N", 1792, 1792, 1792) == "mfma16_128x128x32_w4x2_streamk_1wg"
    assert sel("N", "N", 1536, 1536, 1536) == "mfma16_128x128x32_w4x2_streamk_1wg"
    # ... but not with little k-work per workgroup.
    assert sel("N", "N", 1536, 1536, 256) == "mfma16_64x64x32_w2x2"
    # Square sizes: whichever tile spreads most evenly over the 256 CUs.
    # Stream-K over 256 x 128 tiles where no data-parallel tile spreads evenly.
    skw = "mfma32_256x128x32_w4x2_streamk"
    sk16 = "mfma16_128x128x32_w4x2_streamk_1wg"
    q192 = "mfma16_192x192x32_w4x3"
    # From 400 tiles of 128 x 128, NN takes two 16 x 16 stream-K workgroups per CU.
    sk16b = "mfma16_128x128x32_w4x2_streamk_2wg"
    for n, want in [(2048, "mfma16_128x128x32_w4x2_kg2"), (2304, sk16), (2560, sk16b), (2816, "mfma32_256x128x32_w4x2"),
                    (3072, q192), (3328, sk16b), (3584, sk16b), (3840, sk16b), (4096, "mfma32_256x256x32_w4x2"),
                    (6144, q192), (8192, "mfma32_256x256x32_w4x2")]:
        assert sel("N", "N", n, n, n) == want, n
    # The 192 x 192 tile where its grid fills at least 88% of a whole number of
    # waves (3072^2: 256 tiles; 3000 x 2900: 256, 92% of them outputs), every op
    # pair, also at short K; not on 209 tiles (82%), nor on 484 (4096^2).
    for ta in "NT":
        for tb in "NT":
            assert sel(ta, tb, 3072, 3072, 3072) == q192
            assert sel(ta, tb, 3000, 2900, 700) == q192
    assert sel("N", "N", 3072, 3072, 512) == q192
    assert sel("N", "N", 1536, 6144, 4096) == q192
    assert sel("T", "T", 2112, 3636, 3684) == sk16
    # Stream-K over big tiles for NT; over 128 x 128 tiles of 16 x 16 blocks for
    # TN, and for TT from K = 2048; 128 x 128 (two per CU) where big tiles do not pay.
    assert sel("N", "T", 3328, 3328, 3328) == "mfma32_256x128x32_w4x2_streamk"
    assert sel("T", "N", 3328, 3328, 3328) == "mfma16_128x128x32_w4x2_streamk_1wg"
    assert sel("T", "T", 2560, 2560, 2560) == "mfma16_128x128x32_w4x2_streamk_1wg"
    assert sel("T", "N", 3584, 4096, 1024) == "mfma16_128x128x32_w4x2_streamk_1wg"
    # K <= 256 over at least 128 tiles of 64 x 64: the plain 64 x 64 tile,
    # unless 128 x 128 tiles spread over the CUs as evenly.
    assert sel("T", "T", 1024, 2048, 256) == "mfma16_64x64x32_w2x2"
    assert sel("N", "N", 2048, 4096, 256) == "mfma16_128x128x32_w4x2"
    assert sel("T", "T", 1792, 1792, 256) == "mfma16_128x128x32_w4x2"
    # Where the stream-K rules apply, split-K over 64 x 64 tiles when the timing
    # models put it first.
    assert sel("N", "T", 1548, 920, 2236) == "mfma16_64x64x32_w2x2_splitk"
    assert sel("T", "T", 792, 1612, 2196) == "mfma16_64x64x32_w2x2_splitk"
    assert sel("T", "N", 1792, 1280, 4096) == "mfma16_128x128x32_w4x2_streamk_1wg"
    assert sel("N", "N", 2560, 2560, 256) == "mfma16_64x64x32_w2x2"
    # No stream-K below K = 1024 on big grids.
    assert sel("T", "T", 3584, 2560, 512) == "mfma16_64x64x32_w2x2"
    assert "streamk" not in sel("N", "T", 2304, 3072, 512)
    # 128..229 tiles of 128 x 128 with enough k-work, or 72..127 with K >= 2048:
    # stream-K; from 230 tiles the data-parallel 128 x 128 tile.
    assert sel("T", "N", 1792, 1280, 4096) == "mfma16_128x128x32_w4x2_streamk_1wg"
    assert sel("T", "N", 1536, 768, 4096) == "mfma16_128x128x32_w4x2_streamk_1wg"
    assert sel("N", "N", 512, 4096, 4096) == "mfma16_128x128x32_w4x2_streamk_1wg"
    assert sel("N", "T", 3584, 1152, 1024) == "mfma16_128x128x32_w4x2"
    assert sel("N", "N", 1024, 2048, 1024) == "mfma16_64x64x32_w2x2"
    # ... and 461..511 tiles of 64 x 64 (two k-group workgroups fill 90% of the
    # slots): two k-groups; exactly 512 keeps stream-K.
    assert sel("N", "N", 1844, 1056, 2032) == "mfma16_64x64x32_w2x2_kg2"
    assert sel("N", "T", 828, 2392, 3588) == "mfma16_64x64x32_w2x2_kg2"
    # The edges of that band, with long K: 460 tiles of 64 x 64 (1280 x 1472)
    # fill under 90% of two slots per CU and take stream-K (72..127 tiles of
    # 128 x 128 with K >= 2048); 462 (1344 x 1408; 461 is prime, and no grid of
    # 461 such tiles stays under 230 tiles of 128 x 128) and 511 (448 x 4672)
    # take two k-groups; exactly 512 (1024 x 2048) keeps stream-K.
    assert sel("N", "N", 1280, 1472, 4096) == "mfma16_128x128x32_w4x2_streamk_1wg"
    assert sel("N", "N", 1344, 1408, 4096) == "mfma16_64x64x32_w2x2_kg2"
    assert sel("N", "N", 448, 4672, 4096) == "mfma16_64x64x32_w2x2_kg2"
    assert sel("N", "N", 1024, 2048, 4096) == "mfma16_128x128x32_w4x2_streamk_1wg"
    # With short K (K < 1024) the short-k rule comes first: 512 tiles take the
    # plain 64 x 64 tile, 460 and 462 still two k-groups.
    assert sel("N", "N", 1024, 2048, 512) == "mfma16_64x64x32_w2x2"
    assert sel("N", "N", 1344, 1408, 512) == "mfma16_64x64x32_w2x2_kg2"
    assert sel("N", "N", 1280, 1472, 512) == "mfma16_64x64x32_w2x2_kg2"
    # ... and short k on up to 229 such tiles: the plain 64 x 64 tile, or
    # 128 x 128 where its grid spreads nearly as evenly.
    assert sel("N", "N", 1280, 2560, 512) == "mfma16_128x128x32_w4x2"
    assert sel("N", "N", 1972, 1644, 788) == "mfma16_128x128x32_w4x2"
    assert sel("T", "T", 2560, 2560, 512) == "mfma16_64x64x32_w2x2"
    assert sel("N", "T", 1072, 2768, 764) == "mfma16_64x64x32_w2x2"
    assert sel("N", "N", 1536, 2048, 512) == "mfma16_64x64x32_w2x2"
    assert sel("N", "T", 2304, 2304, 1024) == "mfma32_128x128x32_w4x2_streamk_2wg"
    # N > M: NN takes the 16 x 16 stream-K tile (two per CU from 400 tiles); transposed B keeps the
    # 128 x 256 stream-K tile.
    assert sel("N", "N", 2304, 3328, 2048) == "mfma16_128x128x32_w4x2_streamk_2wg"
    assert sel("N", "N", 2304, 2304, 2048) == "mfma16_128x128x32_w4x2_streamk_1wg"
    assert sel("N", "T", 2304, 3328, 2048) == "mfma32_128x256x32_w2x4_streamk"
    # M <= 32: the skinny, bandwidth-bound kernel.
    assert "skinny" in sel("N", "N", 16, 4096, 4096)
    assert "skinny" in sel("T", "T", 32, 128, 7)
    # ... but not below one 128-column band.
    assert "skinny" not in sel("T", "T", 32, 100, 7)
    assert "skinny" not in sel("N", "N", 32, 64, 64)
    assert "skinny" not in sel("N", "N", 33, 4096, 4096)
    assert mg.mi_sgemm_select_config("Z", "N", 1, 1, 1) == -1
    assert mg.mi_sgemm_select_config("N", "N", 1, 1, -1) == -5


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(mg, "_lib", None)
    monkeypatch.setattr(mg, "library_path", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="not built"):
        mg.mi_sgemm_config_count()


def test_one_hip_runtime_when_library_is_loaded_first():
    """Using the library before torch must not load a second HIP runtime: the
    binding loads torch's copy first, and libmisgemm.so binds to that one."""
    import subprocess
    import sys
    code = ("import fp32_gemm_nn_amd as mg\n"
            "mg.config_names()\n"
            "import torch\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "libs = {l.split()[-1] for l in maps if 'libamdhip64' in l or 'libhsa-runtime64' in l}\n"
            "print(len([l for l in libs if 'libamdhip64' in l]), len([l for l in libs if 'libhsa-runtime64' in l]))\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split() == ["1", "1"], out.stdout


def test_wrapper_overlap_check():
    """The tensor wrapper's test that keeps C from aliasing A or B: exact on
    rows, so C may live in the padding columns of A; checked against a
    brute-force set intersection of element addresses."""
    torch = pytest.importorskip("torch")
    import itertools

    import numpy as np

    buf = torch.zeros(1000)
    a = buf[:400].view(20, 20)
    assert mg._overlaps(a, a)
    assert mg._overlaps(a, buf[399:400].view(1, 1))            # last element shared
    assert not mg._overlaps(a, buf[400:800].view(20, 20))      # adjacent, disjoint
    strided = a[:, :5]                                          # rows of 5 at stride 20
    assert mg._overlaps(strided, buf[383:388].view(1, 5))
    assert not mg._overlaps(strided, buf[385:390].view(1, 5))   # past the last row
    assert not mg._overlaps(strided, a[:, 5:20])                # the padding columns
    assert not mg._overlaps(strided, a[:, 5:20][:, :0])         # empty

    def addrs(t):
        return {t.data_ptr() + 4 * (i * t.stride(0) + j) for i in range(t.shape[0]) for j in range(t.shape[1])}

    rng = np.random.default_rng(7)
    views = []
    for _ in range(60):
        r, c = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        ld = c + int(rng.integers(0, 4))
        off = int(rng.integers(0, 60))
        views.append(buf[off:off + r * ld].view(r, ld)[:, :c])
    for x, y in itertools.combinations(views, 2):
        assert mg._overlaps(x, y) == bool(addrs(x) & addrs(y))


def test_wrapper_leading_dimension():
    """The tensor wrapper's leading dimension: the row stride for tensors with
    distinct rows, the row length for a single row, and ValueError (before any
    launch) for rows that overlap or are broadcast, whose elements no leading
    dimension can address."""
    torch = pytest.importorskip("torch")

    buf = torch.zeros(100)
    assert mg._ld(buf[:12].view(3, 4)) == 4                       # packed
    assert mg._ld(buf[:60].view(6, 10)[:, :7]) == 10              # padded rows
    assert mg._ld(buf[:4].view(1, 4)) == 4                        # one row
    assert mg._ld(buf[:1].view(1, 1)) == 1
    assert mg._ld(buf[10:13].view(1, 3)) == 3
    assert mg._ld(buf[:5].view(5, 1)) == 1                        # one column, stride 1
    assert mg._ld(torch.zeros(3, 0)) >= 1
    assert mg._ld(torch.zeros(4).expand(1, 4)) == 4                # one broadcast row is still one row
    with pytest.raises(ValueError, match="row stride"):
        mg._ld(torch.zeros(4).expand(3, 4))                       # stride (0, 1): 4 floats of storage
    with pytest.raises(ValueError, match="row stride"):
        mg._ld(buf.as_strided((3, 4), (2, 1)))                    # overlapping rows
    with pytest.raises(ValueError, match="row stride"):
        mg._ld(torch.zeros(1).expand(3, 1))                       # stride 0, one column
    with pytest.raises(ValueError, match="contiguous"):
        mg._ld(buf[:12].view(3, 4).t())                           # transposed view: pass op 'T'
    with pytest.raises(ValueError):
        mg._ld(buf[:8])                                           # not 2-D
    # The overlap check rejects the same tensors instead of dividing by a zero stride.
    with pytest.raises(ValueError, match="row stride"):
        mg._overlaps(torch.zeros(4).expand(3, 4), buf[:12].view(3, 4))
    with pytest.raises(ValueError, match="row stride"):
        mg._overlaps(buf[:12].view(3, 4), buf.as_strided((3, 4), (2, 1)))


def test_wrapper_rejects_broadcast_before_launch():
    """sgemm() on CPU tensors with a broadcast C fails on the device check or
    on the leading dimension, never reaching the library."""
    torch = pytest.importorskip("torch")

    A = torch.zeros(3, 4)
    B = torch.zeros(4, 4)
    C = torch.zeros(4).expand(3, 4)
    with pytest.raises(ValueError):
        mg.sgemm("N", "N", 1.0, A, B, 0.0, C)
