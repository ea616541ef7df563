"""Wait states in front of every inline-asm global->LDS copy, checked in the gfx950 assembly.

The compiler inserts hazard waits for the instructions it generates but not around inline
asm. Two GFX9 rules apply to a `buffer_load_dwordx4 ... lds` copy: a buffer instruction must
issue at least 5 wait states after a vector instruction (here v_readfirstlane) wrote one of
its descriptor's SGPRs, and an LDS copy at least 1 after a scalar write of M0 (the compiler's
own LDS-copy builtins get an `s_nop 0` after the M0 write for the second rule). A copy that
misses the first can read a stale descriptor word (a paged-cache variant of the decode that
staged V through such copies, with descriptors built from block-table loads, read V rows from
the wrong tile until the asm carried the wait).

This compiles every kernel source that issues such copies to device assembly (no GPU needed) and
walks back from each copy: within its basic block the last vector write of a descriptor SGPR
must lie at least 5 wait states back, the last scalar write of M0 at least 1; a block start
reached before that many wait states counts as a failure (a predecessor could end in a write).
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

from grouped_query_attention_02_amd import build as B


def _sources_with_copies():
    """Kernel sources whose inline asm issues LDS copies."""
    return sorted(f for f in os.listdir(B.CSRC)
                  if f.endswith(".hip") and "offen lds" in open(os.path.join(B.CSRC, f)).read())


SOURCES = _sources_with_copies()
SGPR_WAITS, M0_WAITS = 5, 1

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists(B.HIPCC),
                                reason="hipcc not installed")


def _asm(src, out):
    cmd = [B.HIPCC, *[f for f in B.CFLAGS if f != "-fPIC"], "--cuda-device-only", "-S",
           "-o", out, os.path.join(B.CSRC, src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out


def _sgprs(tok):
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"s(\d+)", tok)
    return {int(m.group(1))} if m else set()


def _stream(path):
    """Instructions and block starts (None) in program order."""
    out = []
    for raw in open(path):
        line = raw.split(";")[0].strip()
        if not line or line.startswith((".", "//")):
            continue
        if line.endswith(":"):
            out.append(None)
            continue
        out.append(line)
    return out


def _waits_before(ins, i, is_hit):
    """Wait states between instruction i and the nearest earlier one matching is_hit; None
    when a block start or the stream start comes first."""
    ws = 0
    for j in range(i - 1, -1, -1):
        p = ins[j]
        if p is None:
            return None, ws
        if is_hit(p):
            return ws, ws
        op = p.split()[0]
        ws += int(p.split()[1].rstrip(",")) + 1 if op == "s_nop" else 1
        if ws >= 64:
            return ws, ws
    return None, ws


def _check(path):
    ins = _stream(path)
    sites, bad = 0, []
    for i, line in enumerate(ins):
        if line is None or not re.match(r"buffer_load_dword\w*\s.*\blds$", line):
            continue
        sites += 1
        desc = _sgprs(line.split(None, 1)[1].split(",")[1].strip())

        def valu_writes_desc(p):
            op, _, rest = p.partition(" ")
            return op.startswith("v_") and bool(_sgprs(rest.split(",")[0].strip()) & desc)

        def salu_writes_m0(p):
            op, _, rest = p.partition(" ")
            return op.startswith("s_") and rest.split(",")[0].strip() == "m0"

        for name, hit, need in (("descriptor SGPR", valu_writes_desc, SGPR_WAITS),
                                ("M0", salu_writes_m0, M0_WAITS)):
            found, ws = _waits_before(ins, i, hit)
            if (found is not None and found < need) or (found is None and ws < need):
                bad.append(f"line {i}: {line!r}: {ws} wait states after a {name} write")
    return sites, bad


def test_inline_lds_copies_carry_their_wait_states(tmp_path):
    assert SOURCES, "no kernel source issues inline LDS copies"
    with cf.ThreadPoolExecutor(len(SOURCES)) as ex:
        paths = list(ex.map(lambda s: _asm(s, str(tmp_path / (s + ".s"))), SOURCES))
    for src, path in zip(SOURCES, paths):
        sites, bad = _check(path)
        assert sites > 0, f"{src}: no LDS copies found in the assembly"
        assert not bad, f"{src}: {len(bad)} of {sites} copies short of wait states:\n" + \
            "\n".join(bad[:10])


def test_checker_flags_a_copy_without_waits(tmp_path):
    """The walk itself: a copy right after a readfirstlane into its descriptor, or right after
    an M0 write, is reported; five wait states in front clear both."""
    p = tmp_path / "t.s"
    p.write_text("k:\n\tv_readfirstlane_b32 s14, v1\n\ts_mov_b32 m0, s2\n"
                 "\tbuffer_load_dwordx4 v8, s[12:15], 0 offen lds\n"
                 "\ts_nop 4\n\tbuffer_load_dwordx4 v9, s[12:15], 0 offen lds\n")
    sites, bad = _check(str(p))
    assert sites == 2 and len(bad) == 2 and all("line 3" in b for b in bad)
