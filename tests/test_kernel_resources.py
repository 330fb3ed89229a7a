"""Register spills of the built kernels, read from the library's code objects.

Each kernel's private (scratch) segment size is part of the AMDGPU code-object
metadata that hipcc embeds in libmisgemm.so (read by fp32_gemm_nn_amd.codeobj:
the gfx950 code object of each offload bundle, its NT_AMDGPU_METADATA note),
whose amdhsa.kernels list gives .private_segment_fixed_size per kernel. A kernel
that spills registers has a non-zero size there (the youngju.dev CUDA primer,
section よくある落とし穴とチェックリスト, item 4, 過度なレジスタ使用: spilled
registers go to slow local memory).

No instantiation the shape-class selection can reach may spill, for any op
pair, aligned or not. Two forced-only instantiations are allowed to: the
register-staged 256 x 256 tile with both operands transposed (with A
transposed the selection takes the direct-to-LDS form) and the 16 x 16
two-workgroup stream-K tile with both transposed (selected for NN only);
test_abi's selection fuzz checks that neither is chosen.
"""
import os

import pytest

import fp32_gemm_nn_amd as mg
from fp32_gemm_nn_amd import codeobj

msgpack = pytest.importorskip("msgpack")

# Mangled-name fragment of the forced-only instantiation that spills:
# TileCfg<256,256,32,4,2,1,0,false,false,false,false> with TA = TB = true.
FORCED_ONLY_SPILLING = {
    "TileCfgILi256ELi256ELi32ELi4ELi2ELi1ELi0ELb0ELb0ELb0ELb0EEELb1ELb1ELb0E": "256x256 register-staged, TT",
    # TileCfg<128,128,32,4,2,1,4,false,true,false,true> (16 x 16 stream-K, two
    # workgroups per CU) with TA = TB = true: selected only for NN.
    "TileCfgILi128ELi128ELi32ELi4ELi2ELi1ELi4ELb0ELb1ELb0ELb1EEELb1ELb1ELb0E": "16x16 stream-K 2 WG/CU, TT",
}


@pytest.fixture(scope="module")
def kernels():
    if not os.path.exists(mg.library_path):
        pytest.skip("library not built")
    ks = codeobj.kernel_metadata(mg.library_path)
    assert ks, "no gfx950 kernels found in the library's code objects"
    return ks


def test_metadata_covers_every_kernel_family(kernels):
    names = [k[".name"] for k in kernels]
    assert len(names) > 200
    for family in ("sgemm_mfma32", "sgemm_skinny_band", "sgemm_skinny16", "scale_c", "zero_ints", "clock_probe"):
        assert any(family in n for n in names), family
    # 4-byte (SCALAR) instantiations exist for the clamping tiles (87: every
    # clamping tile and op pair whose form fits its register budget).
    assert sum(n.endswith("ELb1EEEvNS_8GemmArgsE") for n in names if "sgemm_mfma32" in n) >= 80


def test_no_selectable_kernel_spills(kernels):
    spilling = {k[".name"]: k[".private_segment_fixed_size"] for k in kernels if k[".private_segment_fixed_size"]}
    unexpected = {n: s for n, s in spilling.items() if not any(frag in n for frag in FORCED_ONLY_SPILLING)}
    assert not unexpected, f"kernels with scratch (bytes per lane): {unexpected}"


def test_no_selectable_kernel_spills_vgprs(kernels):
    """The metadata's own spill count agrees: no VGPR spilled outside the
    forced-only instantiation."""
    spilling = {k[".name"]: k.get(".vgpr_spill_count", 0) for k in kernels if k.get(".vgpr_spill_count", 0)}
    unexpected = {n: s for n, s in spilling.items() if not any(frag in n for frag in FORCED_ONLY_SPILLING)}
    assert not unexpected, f"kernels with spilled VGPRs: {unexpected}"
