"""Register spills of the built kernels, read from the library's code objects.

Each kernel's private (scratch) segment size is part of the AMDGPU code-object
metadata that hipcc embeds in libmisgemm.so: the .hip_fatbin section holds one
clang offload bundle per translation unit, the gfx950 entry of each bundle is
an ELF code object, and its NT_AMDGPU_METADATA note is a msgpack map whose
amdhsa.kernels list gives .private_segment_fixed_size per kernel. A kernel
that spills registers has a non-zero size there (the youngju.dev CUDA primer,
section よくある落とし穴とチェックリスト, item 4, 過度なレジスタ使用: spilled
registers go to slow local memory).

No instantiation the shape-class selection can reach may spill, for any op
pair, aligned or not. Two forced-only instantiations are allowed to: the
register-staged 256 x 256 tile with both operands transposed (TT takes the
direct-to-LDS form) and the direct-to-LDS 256 x 256 tile with only A
transposed (direct-to-LDS is chosen only for TT); test_abi's selection fuzz
checks that neither is ever chosen.
"""
import os
import struct

import pytest

import fp32_gemm_nn_amd as mg

msgpack = pytest.importorskip("msgpack")

BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
NT_AMDGPU_METADATA = 32
SHT_NOTE = 7

# Mangled-name fragments of the two forced-only instantiations that spill:
# TileCfg<256,256,32,4,2,1,0,false,false,false,false> with TA = TB = true, and
# TileCfg<256,256,32,4,2,1,0,false,false,true,false> (direct-to-LDS) with
# TA = true, TB = false.
FORCED_ONLY_SPILLING = {
    "TileCfgILi256ELi256ELi32ELi4ELi2ELi1ELi0ELb0ELb0ELb0ELb0EEELb1ELb1ELb0E": "256x256 register-staged, TT",
    "TileCfgILi256ELi256ELi32ELi4ELi2ELi1ELi0ELb0ELb0ELb1ELb0EEELb1ELb0ELb0E": "256x256 direct-to-LDS, TN",
}


def _sections(elf):
    shoff = struct.unpack_from("<Q", elf, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", elf, 0x3A)
    hdrs = [struct.unpack_from("<IIQQQQ", elf, shoff + i * shentsize) for i in range(shnum)]
    strtab = hdrs[shstrndx][4]
    out = {}
    for name, typ, _flags, _addr, off, size in hdrs:
        end = elf.index(b"\0", strtab + name)
        out.setdefault(elf[strtab + name:end].decode(), []).append((typ, off, size))
    return out


def _bundle_entries(blob):
    pos = 0
    while True:
        start = blob.find(BUNDLE_MAGIC, pos)
        if start < 0:
            return
        count = struct.unpack_from("<Q", blob, start + len(BUNDLE_MAGIC))[0]
        p = start + len(BUNDLE_MAGIC) + 8
        for _ in range(count):
            off, size, tsize = struct.unpack_from("<QQQ", blob, p)
            p += 24
            triple = blob[p:p + tsize].decode()
            p += tsize
            yield triple, blob[start + off:start + off + size]
        pos = start + len(BUNDLE_MAGIC)


def _kernels(code_object):
    for entries in _sections(code_object).values():
        for typ, off, size in entries:
            if typ != SHT_NOTE:
                continue
            q = off
            while q + 12 <= off + size:
                namesz, descsz, ntype = struct.unpack_from("<III", code_object, q)
                q += 12
                name = code_object[q:q + namesz]
                q += (namesz + 3) & ~3
                desc = code_object[q:q + descsz]
                q += (descsz + 3) & ~3
                if ntype == NT_AMDGPU_METADATA and name.startswith(b"AMDGPU"):
                    yield from msgpack.unpackb(desc, raw=False)["amdhsa.kernels"]


def library_kernels():
    with open(mg.library_path, "rb") as f:
        so = f.read()
    (typ, off, size), = _sections(so)[".hip_fatbin"]
    blob = so[off:off + size]
    kernels = []
    for triple, co in _bundle_entries(blob):
        if triple.endswith("gfx950") or "gfx950" in triple.split("-")[-1]:
            kernels.extend(_kernels(co))
    return kernels


@pytest.fixture(scope="module")
def kernels():
    if not os.path.exists(mg.library_path):
        pytest.skip("library not built")
    ks = library_kernels()
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
    """The metadata's own spill count agrees: no VGPR spilled outside the two
    forced-only instantiations."""
    spilling = {k[".name"]: k.get(".vgpr_spill_count", 0) for k in kernels if k.get(".vgpr_spill_count", 0)}
    unexpected = {n: s for n, s in spilling.items() if not any(frag in n for frag in FORCED_ONLY_SPILLING)}
    assert not unexpected, f"kernels with spilled VGPRs: {unexpected}"
