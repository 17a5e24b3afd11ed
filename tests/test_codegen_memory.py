"""Code-generation guard (CPU, needs hipcc): no kernel of the library writes
through the scalar data cache.  Every gfx950 kernel is compiled to assembly
and searched for scalar-memory stores, scalar atomics and scalar cache
write-back / discard instructions; the work counters must be vector-memory
atomics."""
import os
import re
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SCALAR_WRITES = re.compile(r"^\s*s_(store|buffer_store|scratch_store|atomic|buffer_atomic|"
                           r"dcache_wb|dcache_discard)\w*", re.M)


def _asm(src):
    sys.path.insert(0, ROOT)
    from paged_mqa_logits_02_amd import build
    cc = build.hipcc()
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        flags = [f for f in build.compile_flags(src) if f != "-fPIC"]
        r = subprocess.run([cc] + flags + ["--cuda-device-only", "-S",
                                           os.path.join(build.CSRC, src), "-o", out],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return open(out).read()


@pytest.mark.parametrize("src", ["mqa_logits.hip", "mqa_any.hip", "indexer.hip", "proxy.hip",
                                 "api.hip"])
def test_no_scalar_memory_writes(src):
    try:
        asm = _asm(src)
    except RuntimeError:
        pytest.skip("hipcc not available")
    bad = SCALAR_WRITES.findall(asm)
    assert not bad, "scalar-memory writes in %s: %s" % (src, sorted(set(bad)))
    if src == "mqa_logits.hip":
        assert re.search(r"^\s*global_atomic_add", asm, re.M), "work counter atomics not found"


def test_guard_detects_a_scalar_store():
    assert SCALAR_WRITES.search("\ts_store_dword s0, s[2:3], 0x0\n")
    assert SCALAR_WRITES.search("\ts_atomic_add s0, s[2:3], 0x0\n")
    assert not SCALAR_WRITES.search("\tglobal_atomic_add v1, v2, v3, s[2:3] sc0\n")
