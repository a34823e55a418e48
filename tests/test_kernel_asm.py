"""Checks on the gfx950 assembly of the kernels (CPU only: hipcc cross-compiles).

* Every workgroup barrier that follows an LDS write or LDS atomic has an LDS
  wait (s_waitcnt lgkmcnt(0)) between the two.  A barrier only orders what has
  completed: without the wait, another wave may read LDS before the write lands.
  hipcc has emitted such a barrier without the wait on a loop back edge of the
  persistent scoring kernel (the block's next work item went to LDS just before
  it), and waves then repeated the previous item.  The scan walks the assembly
  in text order, which is how the compiler lays out each kernel's blocks.
* No packed fp32 VALU instruction appears in device code: the build keeps the
  packed-fp32-ops target feature off.
"""
import os
import re
import shutil
import subprocess

import pytest

from top_sparse_attention_02_amd import build as B

LDS_WRITE = re.compile(r"^ds_(write|store|add|sub|max|min|or|and|xor|inc|dec|cmpst|wrxchg)")
KERNEL = re.compile(r"^(_Z\S+):\s*(;.*)?$")


@pytest.fixture(scope="module")
def asm_text(tmp_path_factory):
    cc = B.hipcc()
    if not (os.path.isabs(cc) and os.path.exists(cc)) and shutil.which(cc) is None:
        pytest.skip("hipcc not found")
    d = tmp_path_factory.mktemp("asm")
    flags = [f for f in B.HIPCC_FLAGS if f != "-fPIC"]
    texts = []
    for name in sorted(f for f in os.listdir(B.CSRC) if f.endswith(".hip")):
        out = d / (name + ".s")
        r = subprocess.run([cc, *flags, "--cuda-device-only", "-S", os.path.join(B.CSRC, name), "-o", str(out)],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        texts.append(out.read_text())
    return "\n".join(texts)


def barriers_without_lds_wait(text):
    bad, kernel, pending = [], None, None
    for n, raw in enumerate(text.splitlines(), 1):
        s = raw.strip()
        m = KERNEL.match(s)
        if m:
            kernel, pending = m.group(1), None
            continue
        if LDS_WRITE.match(s):
            pending = n
        elif s.startswith("s_waitcnt") and ("lgkmcnt(0)" in s or re.fullmatch(r"s_waitcnt\s+0", s)):
            pending = None
        elif s.startswith("s_barrier"):
            if pending is not None:
                bad.append((kernel, pending, n))
            pending = None
        elif s.startswith("s_endpgm"):
            pending = None
    return bad


def test_scan_flags_a_missing_wait():
    # the scan itself: a write then a barrier is flagged, a wait in between clears it
    k = "_Zfoo:\n"
    assert barriers_without_lds_wait(k + "ds_write_b32 v1, v2\ns_barrier\n") == [("_Zfoo", 2, 3)]
    assert barriers_without_lds_wait(k + "ds_add_u32 v1, v2\ns_waitcnt lgkmcnt(0)\ns_barrier\n") == []
    assert barriers_without_lds_wait(k + "ds_write_b32 v1, v2\ns_waitcnt vmcnt(0) lgkmcnt(0)\ns_barrier\n") == []
    assert barriers_without_lds_wait(k + "ds_read_b32 v1, v2\ns_barrier\n") == []


def test_every_barrier_after_an_lds_write_waits_for_it(asm_text):
    bad = barriers_without_lds_wait(asm_text)
    assert not bad, "barriers without an LDS wait: " + ", ".join(f"{k} (write line {w}, barrier {b})"
                                                                 for k, w, b in bad[:5])


def test_no_packed_fp32_instructions(asm_text):
    found = re.findall(r"^\s*(v_pk_(?:add|mul|fma|mov)_f32)\b", asm_text, re.M)
    assert not found, sorted(set(found))


def test_no_scalar_memory_writes(asm_text):
    # every store and atomic of the kernels goes through the vector memory path:
    # nothing writes through the scalar data cache (no scalar stores or atomics,
    # and no write-back or discard of that cache)
    found = re.findall(r"^\s*(s_(?:buffer_|scratch_)?(?:store|atomic)\w*|s_dcache_(?:wb|discard)\w*)\b", asm_text, re.M)
    assert not found, sorted(set(found))
