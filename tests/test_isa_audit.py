"""Machine-code audit of the library's kernels (CPU only: hipcc emits the
gfx950 assembly here, nothing runs).

A vector-memory store of more than 8 bytes reads its data VGPRs after it
issues.  The compiler protects them (wait states before a VALU may overwrite
them) only when the store takes no SGPR offset; a buffer store with an SGPR
offset followed at once by a VALU write of its data was seen to store the new
value in part of the lanes.  The library therefore puts every offset of a wide
buffer store in the VGPR.  This test holds the assembly of every kernel to
that: no 12- or 16-byte buffer store with a non-zero SGPR offset, and no wide
store (buffer or global) whose data VGPRs a VALU instruction writes within two
wait states of it.
"""

import concurrent.futures as cf
import glob
import os
import re
import subprocess
import tempfile

import pytest

from kernelized_causal_attention_amd import build as b

WIDE_BUFFER = re.compile(r"^\s*buffer_store_dwordx[34]\s+v\[(\d+):(\d+)\],\s*v\d+,\s*s\[\d+:\d+\],\s*(\S+)")
WIDE_GLOBAL = re.compile(r"^\s*(?:global|flat)_store_dwordx[34]\s+v\[\d+:\d+\],\s*v\[(\d+):(\d+)\]")


def vgprs_written(line):
    parts = line.split(None, 1)
    if len(parts) < 2 or not parts[0].startswith("v_") or parts[0].startswith("v_cmp"):
        return set()
    dst = parts[1].split(",")[0].strip()
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", dst)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", dst)
    return {int(m.group(1))} if m else set()


def audit(lines):
    """(stores seen, [problems]) for one assembly listing."""
    seen, problems = 0, []
    for n, line in enumerate(lines):
        mb, mg = WIDE_BUFFER.match(line), WIDE_GLOBAL.match(line)
        if not (mb or mg):
            continue
        seen += 1
        m = mb or mg
        if mb and mb.group(3) != "0":
            problems.append(f"SGPR offset on a wide buffer store: {line.strip()}")
        data = set(range(int(m.group(1)), int(m.group(2)) + 1))
        k, waits = n + 1, 0
        while k < len(lines) and waits < 2:
            nxt = lines[k].strip()
            k += 1
            if not nxt or nxt.startswith((";", ".")) or nxt.endswith(":"):
                continue
            if nxt.startswith("s_nop"):
                waits += int(nxt.split()[1]) + 1
                continue
            if vgprs_written(nxt) & data:
                problems.append(f"data VGPRs overwritten {waits} wait states after: {line.strip()} || {nxt}")
                break
            waits += 1
    return seen, problems


def test_audit_flags_the_pattern():
    # the checker itself: an SGPR-offset store followed by a write of its data
    bad = ["  buffer_store_dwordx4 v[12:15], v0, s[8:11], s19 offen nt", "  v_or_b32_e32 v12, 0x800, v20"]
    seen, problems = audit(bad)
    assert seen == 1 and len(problems) == 2
    good = ["  buffer_store_dwordx4 v[12:15], v0, s[8:11], 0 offen nt", "  s_nop 1", "  v_or_b32_e32 v12, 0x800, v20"]
    assert audit(good) == (1, [])


def _assemble(src, out_dir):
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    cmd = [b.hipcc(), *b.COMMON, "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-2000:]}")
    return out


def test_no_wide_store_data_hazard_in_any_kernel():
    try:
        b.hipcc()
    except RuntimeError as e:
        pytest.skip(str(e))
    srcs = sorted(glob.glob(os.path.join(b.CSRC, "*.hip")))
    assert srcs
    with tempfile.TemporaryDirectory() as tmp, cf.ThreadPoolExecutor(min(8, len(srcs))) as ex:
        listings = list(ex.map(lambda s: _assemble(s, tmp), srcs))
        total, problems = 0, []
        for path in listings:
            seen, p = audit(open(path).read().splitlines())
            total += seen
            problems += [f"{os.path.basename(path)}: {x}" for x in p]
    assert total > 100, total  # the kernels' output stores were found
    assert not problems, "\n".join(problems[:20])
