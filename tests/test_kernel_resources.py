"""Resource use of every kernel in the built library, read from the gfx950
code objects' own metadata (no GPU needed).

No kernel may use scratch (private) memory.  The compiler can put a kernel's
register arrays or closure state in scratch without any spill warning, for a
change as small as how a loop's unit index is selected; that turned the
decode kernels twice as slow once.  Nor may any kernel spill VGPRs.  SGPR
spills are allowed (the prefill and mixed kernels have a few): with no
scratch they go to lanes of spare VGPRs, a register move each."""

import os
import re
import struct
import subprocess
import tempfile

import pytest

READELF = "/opt/rocm/llvm/bin/llvm-readelf"
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def code_objects(blob):
    """The gfx950 code objects of every offload bundle in ``blob``: the
    bundle header is the magic, an entry count, then per entry its offset
    (from the bundle's start), size and target triple."""
    pos = 0
    while (i := blob.find(BUNDLE_MAGIC, pos)) >= 0:
        (n,) = struct.unpack_from("<Q", blob, i + len(BUNDLE_MAGIC))
        p = i + len(BUNDLE_MAGIC) + 8
        for _ in range(n):
            off, size, tl = struct.unpack_from("<QQQ", blob, p)
            triple = blob[p + 24:p + 24 + tl].decode()
            p += 24 + tl
            if "amdgcn" in triple and size > 0:
                assert triple.endswith("gfx950"), triple
                yield blob[i + off:i + off + size]
        pos = i + 1


def kernel_metadata(elf_bytes):
    """Per kernel: name, private segment size and spill counts, from the
    code object's AMDGPU metadata note."""
    with tempfile.NamedTemporaryFile(suffix=".co") as f:
        f.write(elf_bytes)
        f.flush()
        text = subprocess.run([READELF, "--notes", f.name], capture_output=True, text=True, check=True).stdout
    kernels = []
    for chunk in re.split(r"\n  - \.agpr_count:|\n  - \.args:", text)[1:]:
        fields = dict(re.findall(r"^    \.(name|private_segment_fixed_size|vgpr_spill_count|sgpr_spill_count):\s+(\S+)",
                                 chunk, flags=re.M))
        if "name" in fields:
            kernels.append(fields)
    return kernels


@pytest.fixture(scope="module")
def kernels():
    from paged_kv_cache_140_amd import _lib

    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libpa.so is not built")
    if not os.path.exists(READELF):
        pytest.skip("llvm-readelf is not installed")
    blob = open(_lib.LIB_PATH, "rb").read()
    found = [k for co in code_objects(blob) for k in kernel_metadata(co)]
    assert found, "no gfx950 kernels found in libpa.so"
    return found


def test_every_hot_path_kernel_is_present(kernels):
    names = " ".join(k["name"] for k in kernels)
    for part in ("decode_kernel", "decode_merge_kernel", "prefill_chunk_kernel", "prefill_merge_kernel",
                 "mixed_kernel", "append_kernel", "copy_blocks_kernel"):
        assert part in names, part


def test_no_kernel_uses_scratch_or_spills_vgprs(kernels):
    bad = [(k["name"], k.get("private_segment_fixed_size"), k.get("vgpr_spill_count"))
           for k in kernels
           if int(k.get("private_segment_fixed_size", 0)) or int(k.get("vgpr_spill_count", 0))]
    assert not bad, bad


def test_direct_lds_loads_take_m0_from_the_compiler():
    """The prefill's direct-to-LDS loads are inline assembly whose LDS
    address is an M0 operand ("{m0}" constraint), so the compiler writes M0
    itself before each of them and knows that the statement uses it.  A
    backstop on the built code: every global_load_lds_dwordx4 comes from that
    statement (right after its s_nop 0), and M0 is written in the code."""
    from paged_kv_cache_140_amd import _lib

    objdump = "/opt/rocm/llvm/bin/llvm-objdump"
    if not os.path.exists(_lib.LIB_PATH) or not os.path.exists(objdump):
        pytest.skip("libpa.so or llvm-objdump missing")
    blob = open(_lib.LIB_PATH, "rb").read()
    loads, m0_writes, stray = 0, 0, []
    for co in code_objects(blob):
        with tempfile.NamedTemporaryFile(suffix=".co") as f:
            f.write(co)
            f.flush()
            text = subprocess.run([objdump, "-d", "--mcpu=gfx950", f.name], capture_output=True, text=True,
                                  check=True).stdout
        ins = [re.sub(r"\s*//.*", "", line.strip()) for line in text.splitlines()]
        ins = [i for i in ins if i and not i.endswith(">:") and not i.startswith("Disassembly")]
        for k, line in enumerate(ins):
            if re.match(r"s_\w+ m0,", line):
                m0_writes += 1
            if line.startswith("global_load_lds_dwordx4"):
                loads += 1
                if not ins[k - 1].startswith("s_nop 0"):
                    stray.append(line)
    assert loads > 0, "no direct-to-LDS loads found"
    assert m0_writes > 0, "direct-to-LDS loads but no M0 write"
    assert not stray, stray[:10]
