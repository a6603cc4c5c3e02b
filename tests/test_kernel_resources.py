"""The GPU kernels keep their working state in registers: no scratch (private)
memory and no spilled registers.

A kernel whose ring of prefetched K/V tiles falls back to scratch still computes the
right answer -- no parity test notices -- but loses the overlap of its loads and runs
at a fraction of its speed.  This compiles every kernel source for gfx950 to device
assembly (code built here) and reads, for each kernel, the private-segment size and
VGPR spill count the compiler records in the code object's kernel metadata, plus any
scratch instruction in the text.  (Spilled SGPRs live in VGPR lanes, not in memory,
and are not counted.)  CPU only (the compiler cross-compiles).
"""

import os
import re
import subprocess
import tempfile

import pytest

from paged_kv_cache_reshape_amd import build as B

SOURCES = sorted(os.path.basename(s) for s in B.sources() if "__global__" in open(s).read())


@pytest.fixture(scope="module")
def kernels():
    """{source: [(kernel symbol, private bytes, vgpr spills, sgpr spills)], scratch instructions}."""
    out = {}
    with tempfile.TemporaryDirectory() as d:
        procs = []
        for f in SOURCES:
            asm = os.path.join(d, f + ".s")
            cmd = [B.hipcc(), *B.common_flags(), "--cuda-device-only", "-S", os.path.join(B.CSRC, f), "-o", asm]
            procs.append((f, asm, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE)))
        for f, asm, p in procs:
            _, err = p.communicate(timeout=900)
            assert p.returncode == 0, err.decode()[-2000:]
            text = open(asm).read()
            meta = text[text.index("amdhsa.kernels:"):]
            rows = []
            for e in meta.split("\n  - ")[1:]:
                name = re.search(r"\.name:\s+(\S+)", e)
                if not name:
                    continue
                field = lambda k: int(re.search(rf"\.{k}:\s+(\d+)", e).group(1))
                rows.append((name.group(1), field("private_segment_fixed_size"), field("vgpr_spill_count"),
                             field("sgpr_spill_count")))
            out[f] = (rows, len(re.findall(r"\bscratch_(load|store)", text)))
    return out


@pytest.mark.parametrize("source", SOURCES)
def test_no_scratch_and_no_spills(kernels, source):
    rows, scratch = kernels[source]
    assert rows, f"{source}: no kernels found"
    bad = [r for r in rows if r[1] or r[2]]
    assert not bad, f"{source}: kernels with scratch or spills: {bad[:4]}"
    assert scratch == 0, f"{source}: {scratch} scratch instructions"


def test_hot_kernels_are_present(kernels):
    names = " ".join(n for rows, _ in kernels.values() for n, *_ in rows)
    for k in ("decode_onepass_kernel", "decode_split_kernel", "reduce_kernel", "varlen_lds_kernel",
              "varlen_kernel", "write_kernel", "write_fp8_kernel", "decode_kernel"):
        assert k in names, k
