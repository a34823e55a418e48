"""Checks on the gfx950 assembly of the kernels (CPU only: hipcc cross-compiles).

* Every workgroup barrier that follows an LDS write or LDS atomic has an LDS
  wait (s_waitcnt lgkmcnt(0)) between the two.  A barrier only orders what has
  completed: without the wait, another wave may read LDS before the write lands.
  hipcc has emitted such a barrier without the wait on a loop back edge of the
  persistent scoring kernel (the block's next work item went to LDS just before
  it), and waves then repeated the previous item.  The scan follows each
  kernel's control flow (basic blocks, branch and fall-through edges) from its
  entry.
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


LABEL = re.compile(r"^(\.?[A-Za-z_$][\w.$]*):")
BRANCH = re.compile(r"^s_(c?branch\w*)\s+(\S+)")


def _kernels(text):
    """(name, [(line number, instruction)]) per kernel, comments and directives dropped
    (labels kept)."""
    out, name, body = [], None, []
    for n, raw in enumerate(text.splitlines(), 1):
        s = raw.split(";", 1)[0].strip()
        m = KERNEL.match(raw.strip())
        if m:
            if name:
                out.append((name, body))
            name, body = m.group(1), []
            continue
        if name is None or not s or (s.startswith(".") and not LABEL.match(s)):
            continue
        body.append((n, s))
        if s.startswith("s_endpgm"):
            out.append((name, body))
            name, body = None, []
    if name:
        out.append((name, body))
    return out


def barriers_without_lds_wait(text):
    """Barriers that a path can reach with an LDS write not yet waited for.

    Per kernel, basic blocks are cut at labels and after branches; an LDS write
    leaves the block's state pending until an s_waitcnt with lgkmcnt(0) (or a
    full wait), and the pending state flows along fall-through edges and branch
    edges (s_branch: target only; s_cbranch_*: target and fall-through) to a
    fixed point.  A barrier met while pending is reported with the write that
    left it pending (its line in the assembly)."""
    bad = []
    for name, body in _kernels(text):
        blocks, labels, cur = [], {}, []
        for n, s in body:
            m = LABEL.match(s)
            if m:
                if cur:
                    blocks.append(cur)
                cur = []
                labels[m.group(1)] = len(blocks)
                continue
            cur.append((n, s))
            if BRANCH.match(s) or s.startswith("s_endpgm"):
                blocks.append(cur)
                cur = []
        if cur:
            blocks.append(cur)
        # a label that ends up on an empty block points to the next block
        succ = []
        for i, blk in enumerate(blocks):
            last = blk[-1][1] if blk else ""
            m = BRANCH.match(last)
            nxt = [i + 1] if i + 1 < len(blocks) else []
            if last.startswith("s_endpgm"):
                succ.append([])
            elif m and m.group(1) == "branch":
                succ.append([labels[m.group(2)]] if m.group(2) in labels else [])
            elif m:
                succ.append(([labels[m.group(2)]] if m.group(2) in labels else []) + nxt)
            else:
                succ.append(nxt)
        state_in = [None] * len(blocks)  # None: not reached yet; else the pending write's line or 0
        state_in[0] = 0 if blocks else None
        work = [0] if blocks else []
        found = {}
        while work:
            i = work.pop()
            pending = state_in[i]
            for n, s in blocks[i]:
                if LDS_WRITE.match(s):
                    pending = n
                elif s.startswith("s_waitcnt") and ("lgkmcnt(0)" in s or re.fullmatch(r"s_waitcnt\s+0", s)):
                    pending = 0
                elif s.startswith("s_barrier"):
                    if pending:
                        found[(pending, n)] = True
                    pending = 0
            for j in succ[i]:
                if j >= len(blocks):
                    continue
                old = state_in[j]
                new = pending if old is None else (old or pending)
                if old is None or (new and not old):
                    state_in[j] = new
                    work.append(j)
        bad += [(name, w, b) for (w, b) in sorted(found)]
    return bad


def test_scan_flags_a_missing_wait():
    # the scan itself: a write then a barrier is flagged, a wait in between clears it
    k = "_Zfoo:\n"
    assert barriers_without_lds_wait(k + "ds_write_b32 v1, v2\ns_barrier\n") == [("_Zfoo", 2, 3)]
    assert barriers_without_lds_wait(k + "ds_add_u32 v1, v2\ns_waitcnt lgkmcnt(0)\ns_barrier\n") == []
    assert barriers_without_lds_wait(k + "ds_write_b32 v1, v2\ns_waitcnt vmcnt(0) lgkmcnt(0)\ns_barrier\n") == []
    assert barriers_without_lds_wait(k + "ds_read_b32 v1, v2\ns_barrier\n") == []


def test_scan_follows_branches():
    k = "_Zfoo:\n"
    # a write whose block jumps away does not reach a barrier laid out after it ...
    text = k + "ds_write_b32 v1, v2\ns_branch .LBB0_2\n.LBB0_1:\ns_barrier\n.LBB0_2:\ns_endpgm\n"
    assert barriers_without_lds_wait(text) == []
    # ... but a branch to the barrier's block carries it there (a back edge, as the
    # compiler laid out the scoring loop), and so does the fall-through of a
    # conditional branch
    text = k + ".LBB0_1:\ns_barrier\nds_write_b32 v1, v2\ns_cbranch_scc1 .LBB0_1\ns_endpgm\n"
    assert barriers_without_lds_wait(text) == [("_Zfoo", 4, 3)]
    text = k + "ds_write_b32 v1, v2\ns_cbranch_scc1 .LBB0_2\ns_barrier\n.LBB0_2:\ns_endpgm\n"
    assert barriers_without_lds_wait(text) == [("_Zfoo", 2, 4)]


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
