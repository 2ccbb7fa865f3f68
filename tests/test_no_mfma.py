"""The decode path is bandwidth-bound and runs on the vector ALUs: the built
library's gfx950 code holds no matrix-core (MFMA) instruction.

Decode streams 4 D bytes of K/V per token and KV head against 4 g D flops, g =
2..7 flops per byte, below the fp32 vector ridge of MI355X; one query row per
entry is not a dense contraction, so matrix cores have nothing to do.  This
reads the code object of the library built here (the clang offload bundle in
its .hip_fatbin section) and disassembles it with the ROCm llvm-objdump."""
import os
import struct
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "paged_kv_decode_pkv_amd", "libpkv.so")
OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _gfx950_code_object(blob: bytes) -> bytes:
    """The gfx950 entry of the library's (uncompressed) clang offload bundle:
    magic, entry count, then per entry {offset, size, triple length, triple}."""
    base = blob.find(MAGIC)
    assert base >= 0, "no offload bundle in the library"
    (count,) = struct.unpack_from("<Q", blob, base + len(MAGIC))
    pos = base + len(MAGIC) + 8
    for _ in range(count):
        off, size, tlen = struct.unpack_from("<QQQ", blob, pos)
        pos += 24
        triple = blob[pos:pos + tlen].decode()
        pos += tlen
        if triple.endswith("gfx950"):
            return blob[base + off:base + off + size]
    raise AssertionError("no gfx950 code object in the bundle")


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
@pytest.mark.skipif(not os.path.exists(OBJDUMP), reason="ROCm llvm-objdump missing")
def test_no_mfma_in_decode_library(tmp_path):
    co = tmp_path / "pkv_gfx950.co"
    co.write_bytes(_gfx950_code_object(open(LIB, "rb").read()))
    asm = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", str(co)], capture_output=True,
                         text=True, check=True).stdout
    assert "v_dot2" in asm, "disassembly holds none of the kernels' bf16 dot products"
    assert "global_load_lds_dwordx4" in asm
    assert "v_mfma" not in asm and "v_smfmac" not in asm
