"""Host logic of bench.py: the kernel-code digest that ties counter summaries to the kernels.

bench.py reports `roofline.traffic` from a committed counter summary only when the summary
was taken on the kernels the library holds now.  These tests check the ELF walk behind that
digest and the accept/refuse rule, without a GPU.
"""
import os
import re
import struct
import sys

import pytest

sys.path.insert(0, os.path.join(os.path.dirname(__file__), ".."))
import bench  # noqa: E402

LIB = os.path.join(bench.ROOT, "attention_gqa_decode_amd", "libattn_gqa.so")


def test_elf_sections_of_the_python_binary():
    # any x86-64 ELF has these sections; offsets and sizes must lie inside the file
    blob = open(os.path.realpath(sys.executable), "rb").read()
    assert blob[:4] == b"\x7fELF" and blob[4] == 2  # 64-bit
    secs = bench._elf_sections(blob)
    assert ".text" in secs and ".shstrtab" in secs
    off, size = secs[".text"]
    assert 0 < off and off + size <= len(blob) and size > 0


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_code_digest_is_stable_and_covers_every_kernel_object():
    d = bench.kernel_code_digest()
    assert re.fullmatch(r"[0-9a-f]{16}", d)
    assert bench.kernel_code_digest() == d
    # one bundle per source file; the kernel sources each add machine code
    blob = open(LIB, "rb").read()
    so, ss = bench._elf_sections(blob)[".hip_fatbin"]
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    texts, off = [], blob.find(magic, so, so + ss)
    while off >= 0:
        n, = struct.unpack_from("<Q", blob, off + len(magic))
        pos = off + len(magic) + 8
        for _ in range(n):
            e_off, _, t_len = struct.unpack_from("<QQQ", blob, pos)
            triple = blob[pos + 24:pos + 24 + t_len].decode()
            pos += 24 + t_len
            if triple.endswith("gfx950"):
                texts.append(bench._elf_sections(blob, off + e_off).get(".text", (0, 0))[1])
        off = blob.find(magic, pos, so + ss)
    assert len(texts) == 4  # api, decode, prefill, probe
    assert sum(t > 0 for t in texts) == 3  # the C ABI file holds no kernel


def _summary(root, name, digest, nbytes):
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    with open(os.path.join(root, "profiles", f"{name}_counters.md"), "w") as f:
        f.write(f"# counters\n\nkernel_code_digest: {digest}\nhbm_bytes_per_launch: {nbytes:.6e}\n")


def test_traffic_is_read_only_for_matching_kernels(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_code_digest", lambda: "0123456789abcdef")
    _summary(str(tmp_path), "decode_a", "0123456789abcdef", 2.0567e9)
    _summary(str(tmp_path), "decode_b", "fedcba9876543210", 1.0e9)
    assert bench.committed_traffic("decode_a", 2.05e9) == pytest.approx(2.0567e9)
    assert bench.committed_traffic("decode_b", 1.0e9) is None  # taken on other kernels
    assert bench.committed_traffic("decode_c", 1.0e9) is None  # no summary
    monkeypatch.setattr(bench, "kernel_code_digest", lambda: None)  # library not built
    assert bench.committed_traffic("decode_a", 2.05e9) is None
