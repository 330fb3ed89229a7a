"""Read the gfx950 code objects embedded in libmisgemm.so.

hipcc places one clang offload bundle per translation unit in the library's
.hip_fatbin section; the bundle entry whose target triple names gfx950 is an
AMDGPU ELF code object. From it this module reads each kernel's machine code
(its symbol's bytes in .text) and the code-object metadata note
(NT_AMDGPU_METADATA, a msgpack map whose amdhsa.kernels list gives per-kernel
register counts and private segment sizes).

Host-side tooling only (measurement records and tests): nothing here runs on
the GPU or takes part in a product call.
"""
import hashlib
import re
import struct

BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
SHT_SYMTAB = 2
SHT_NOTE = 7
STT_FUNC = 2
NT_AMDGPU_METADATA = 32


def _sections(elf):
    """{name: [(type, offset, size, addr), ...]} of a 64-bit little-endian ELF."""
    shoff = struct.unpack_from("<Q", elf, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", elf, 0x3A)
    hdrs = [struct.unpack_from("<IIQQQQ", elf, shoff + i * shentsize) for i in range(shnum)]
    strtab = hdrs[shstrndx][4]
    out = {}
    for name, typ, _flags, addr, off, size in hdrs:
        end = elf.index(b"\0", strtab + name)
        out.setdefault(elf[strtab + name:end].decode(), []).append((typ, off, size, addr))
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


def gfx950_code_objects(library_path):
    """The gfx950 ELF code objects of the library, one per translation unit."""
    with open(library_path, "rb") as f:
        so = f.read()
    (_typ, off, size, _addr), = _sections(so)[".hip_fatbin"]
    blob = so[off:off + size]
    return [co for triple, co in _bundle_entries(blob) if "gfx950" in triple]


def kernel_code(library_path):
    """{mangled kernel name: machine code bytes} over every code object."""
    out = {}
    for co in gfx950_code_objects(library_path):
        secs = _sections(co)
        (_t, text_off, _s, text_addr), = secs[".text"]
        (_t, sym_off, sym_size, _a), = secs[".symtab"]
        (_t, str_off, _s, _a), = secs[".strtab"]
        for i in range(sym_size // 24):
            st_name, st_info, _other, _shndx, value, size = struct.unpack_from("<IBBHQQ", co, sym_off + 24 * i)
            if (st_info & 0xF) != STT_FUNC or size == 0:
                continue
            name = co[str_off + st_name:co.index(b"\0", str_off + st_name)].decode()
            start = text_off + (value - text_addr)
            out[name] = co[start:start + size]
    return out


def kernel_code_sha256(library_path, symbol):
    """sha256 of one kernel's machine code, or None when the library has no
    kernel of that mangled name."""
    code = kernel_code(library_path).get(symbol)
    return hashlib.sha256(code).hexdigest() if code is not None else None


def kernel_metadata(library_path):
    """The amdhsa.kernels metadata maps of every gfx950 kernel (needs msgpack)."""
    import msgpack

    kernels = []
    for co in gfx950_code_objects(library_path):
        for entries in _sections(co).values():
            for typ, off, size, _addr in entries:
                if typ != SHT_NOTE:
                    continue
                q = off
                while q + 12 <= off + size:
                    namesz, descsz, ntype = struct.unpack_from("<III", co, q)
                    q += 12
                    name = co[q:q + namesz]
                    q += (namesz + 3) & ~3
                    desc = co[q:q + descsz]
                    q += (descsz + 3) & ~3
                    if ntype == NT_AMDGPU_METADATA and name.startswith(b"AMDGPU"):
                        kernels.extend(msgpack.unpackb(desc, raw=False)["amdhsa.kernels"])
    return kernels


def find_symbol(library_path, pattern):
    """The one mangled kernel name matching the regular expression."""
    names = [n for n in kernel_code(library_path) if re.search(pattern, n)]
    if len(names) != 1:
        raise LookupError(f"{len(names)} kernels match {pattern!r}")
    return names[0]
