"""Which kernels of the built library use the matrix cores (CPU only).

Decode streams 4 D bytes of K/V per token and KV head against 4 g D flops, g =
2..7 flops per byte, below the fp32 vector ridge of MI355X; one query row per
entry is not a dense contraction, so the decode kernels (and the append, the
plan and the fused norm/rotary step) hold no matrix-core (MFMA) instruction.
The paged prefill, several rows against the same keys, is a dense contraction
and does use them.  This reads every gfx950 code object of the library built
here (one clang offload bundle per source file, in its .hip_fatbin section),
disassembles them with the ROCm llvm-objdump and sorts the MFMA instructions
by the kernel they sit in."""
import os
import re
import struct
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "paged_kv_decode_pkv_amd", "libpkv.so")
OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _gfx950_code_objects(blob: bytes):
    """The gfx950 entries of every (uncompressed) clang offload bundle in the
    library: magic, entry count, then per entry {offset, size, triple length,
    triple}."""
    found = []
    base = blob.find(MAGIC)
    while base >= 0:
        (count,) = struct.unpack_from("<Q", blob, base + len(MAGIC))
        pos = base + len(MAGIC) + 8
        for _ in range(count):
            off, size, tlen = struct.unpack_from("<QQQ", blob, pos)
            pos += 24
            triple = blob[pos:pos + tlen].decode()
            pos += tlen
            if triple.endswith("gfx950"):
                found.append(blob[base + off:base + off + size])
        base = blob.find(MAGIC, base + len(MAGIC))
    assert found, "no gfx950 code object in the library"
    return found


def _mfma_by_kernel(asm: str) -> dict:
    counts, current = {}, None
    for line in asm.splitlines():
        m = re.match(r"^[0-9a-f]+ <(.+)>:$", line)
        if m:
            current = m.group(1)
            counts.setdefault(current, 0)
        elif current is not None and ("v_mfma" in line or "v_smfmac" in line):
            counts[current] += 1
    return counts


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
@pytest.mark.skipif(not os.path.exists(OBJDUMP), reason="ROCm llvm-objdump missing")
def test_matrix_cores_only_in_prefill(tmp_path):
    counts, asm_all = {}, ""
    for i, code in enumerate(_gfx950_code_objects(open(LIB, "rb").read())):
        co = tmp_path / f"pkv_gfx950_{i}.co"
        co.write_bytes(code)
        asm = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", str(co)], capture_output=True,
                             text=True, check=True).stdout
        asm_all += asm
        for k, v in _mfma_by_kernel(asm).items():
            counts[k] = counts.get(k, 0) + v
    assert "v_dot2" in asm_all and "global_load_lds_dwordx4" in asm_all
    names = list(counts)
    for kernel in ("run_kernel", "plan_kernel", "append_kernel", "norm_rope_kernel"):
        assert any(kernel in n for n in names), f"{kernel} not found"
    with_mfma = {n: c for n, c in counts.items() if c}
    assert with_mfma and all("prefill_kernel" in n or "prefill_list_kernel" in n
                             for n in with_mfma), with_mfma


def _scratch_by_kernel(asm: str) -> dict:
    counts, current = {}, None
    for line in asm.splitlines():
        m = re.match(r"^[0-9a-f]+ <(.+)>:$", line)
        if m:
            current = m.group(1)
            counts.setdefault(current, 0)
        elif current is not None and "scratch_" in line:
            counts[current] += 1
    return counts


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
@pytest.mark.skipif(not os.path.exists(OBJDUMP), reason="ROCm llvm-objdump missing")
def test_decode_kernels_use_no_scratch(tmp_path):
    # The decode waits for its own direct-to-LDS copies by counting them; a
    # scratch access in its loop would make the compiler wait for every
    # outstanding copy (about a third of the streaming rate lost), so the
    # decode kernels of head_dim 64 and of head_dim 128 with up to 4 query
    # heads per KV head (every shape the workloads run) keep all their state in
    # registers.
    counts = {}
    for i, code in enumerate(_gfx950_code_objects(open(LIB, "rb").read())):
        co = tmp_path / f"pkv_gfx950_{i}.co"
        co.write_bytes(code)
        asm = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", str(co)], capture_output=True,
                             text=True, check=True).stdout
        for k, v in _scratch_by_kernel(asm).items():
            counts[k] = counts.get(k, 0) + v
    shapes = re.compile(r"run_kernelILi(64ELi[1-8]|128ELi[1-4])ELi")
    checked = {n: c for n, c in counts.items() if shapes.search(n)}
    assert len(checked) >= 12, sorted(counts)
    assert not any(checked.values()), {n: c for n, c in checked.items() if c}
