"""Code-generation guard for the logits kernels (CPU: hipcc cross-compiles).

The page loop waits for page loads with exact vmcnt counts.  If any load the
compiler tracks stays pending on a path into the loop, the compiler inserts
`s_waitcnt vmcnt(0)` before the page's LDS operand reads, which drains the
whole page ring on every page (this happened once and cost 10-20% on the long
workloads with correct results).  The test compiles the kernels to gfx950
assembly with the library's own flags and checks that no basic block holding
a matrix instruction waits for vmcnt(0) before its first one."""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def drains_before_mfma(asm, kernel="17mqa_logits_kernel"):
    bad = []
    kernels = re.findall(r"^(_ZN4pmqa" + kernel + r"\S+):[^\n]*\n(.*?)^\s+s_endpgm", asm,
                         re.S | re.M)
    assert kernels, "no logits kernels found in the assembly"
    for name, body in kernels:
        for blk in re.split(r"^(?=\.LBB\S+:|; %bb\.\d+:)", body, flags=re.M):
            if "v_mfma" in blk and re.search(r"s_waitcnt\s+vmcnt\(0\)",
                                             blk[:blk.index("v_mfma")]):
                bad.append(name)
    return kernels, bad


# source, mangled kernel name stem, instances: the 64-head kernels (slots 1..4
# x {fp8, four mxfp4 scale layouts} x {fp32, bf16 out}) and the general FP8 kernels (1 or 2
# planes x {fp32, bf16 out})
SOURCES = [("mqa_logits.hip", "17mqa_logits_kernel", 40),
           ("mqa_any.hip", "21mqa_logits_any_kernel", 4)]


_ASM = {}


def device_asm(src):
    """gfx950 assembly of one library source, compiled with the library's flags."""
    if src in _ASM:
        return _ASM[src]
    import sys
    sys.path.insert(0, ROOT)
    from paged_mqa_logits_02_amd import build
    try:
        cc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    path = os.path.join(build.CSRC, src)
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        flags = [f for f in build.compile_flags(src) if f != "-fPIC"]
        r = subprocess.run([cc] + flags + ["--cuda-device-only", "-S", path, "-o", out],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        _ASM[src] = open(out).read()
    return _ASM[src]


@pytest.mark.parametrize("src,kernel,count", SOURCES, ids=[s[0] for s in SOURCES])
def test_page_loop_has_no_full_drain_before_the_matrix_work(src, kernel, count):
    asm = device_asm(src)
    kernels, bad = drains_before_mfma(asm, kernel)
    assert len(kernels) == count
    assert not bad, "vmcnt(0) before the matrix work in: %s" % sorted(set(bad))


def test_guard_detects_a_drain():
    asm = """_ZN4pmqa17mqa_logits_kernelILi4ELi0ELi0EEEvX:   ; @k
.LBB0_1:                                ; in Loop
\ts_barrier
\ts_waitcnt vmcnt(0)
\tds_read_b128 v[0:3], v4
\tv_mfma_f32_32x32x64_f8f6f4 v[10:25], v[34:41], v[0:7], 0
\ts_endpgm
"""
    _, bad = drains_before_mfma(asm)
    assert bad
    _, ok = drains_before_mfma(asm.replace("vmcnt(0)", "vmcnt(6)"))
    assert not ok


def vector_addressed_page_loads(asm, kernel="17mqa_logits_kernel"):
    """Page loads into LDS that take a 64-bit vector address (`..., off`)."""
    kernels = re.findall(r"^(_ZN4pmqa" + kernel + r"\S+):[^\n]*\n(.*?)^\s+s_endpgm", asm,
                         re.S | re.M)
    bad = [name for name, body in kernels
           if re.search(r"^\s*global_load_lds_dword\S*\s+v\[\d+:\d+\],\s*off", body, re.M)]
    return kernels, bad


def test_page_loads_take_a_scalar_base():
    """Every page load of the 64-head kernels takes the page base from scalar
    registers and the lane's 32-bit offset from one vector register: a 64-bit
    vector address costs a 64-bit vector add per load and two more registers
    per offset (measured: MXFP4 84 -> 80 us with the scalar-base form)."""
    kernels, bad = vector_addressed_page_loads(device_asm("mqa_logits.hip"))
    assert len(kernels) == 40
    assert not bad, "vector-addressed page loads in: %s" % sorted(set(bad))
    asm = """_ZN4pmqa17mqa_logits_kernelILi1ELi0ELi0EEEvX:   ; @k
\tglobal_load_lds_dwordx4 v[2:3], off nt
\ts_endpgm
"""
    assert vector_addressed_page_loads(asm)[1]
    assert not vector_addressed_page_loads(asm.replace("v[2:3], off", "v2, s[4:5]"))[1]


def kernel_body(asm, symbol_prefix):
    """Assembly of the one kernel whose symbol starts with symbol_prefix, from
    its label to the end-of-function marker."""
    m = re.search(r"^(%s\w*):.*?$(.*?)^\.Lfunc_end" % re.escape(symbol_prefix), asm, re.M | re.S)
    assert m, symbol_prefix
    return m.group(2)


def count_ops(body, op):
    return len(re.findall(r"^\s*%s(?:_e32|_e64)?\s" % re.escape(op), body, re.M))


def test_nvfp4_indexer_dequantises_pairs_with_two_instructions():
    """The NVFP4 indexer is paced by its dequantisation: each pair of e2m1
    values is widened to f16 and multiplied by its block's e4m3 scale with one
    packed f16 multiply (the query row and the four key tiles: 5 x 16 packed
    bytes per lane, 80 pairs).  The earlier form (fp32 widening, two fp32
    multiplies, a bf16 pack: four instructions per pair) ran 76 us against
    61 us at 8192 query rows."""
    body = kernel_body(device_asm("indexer.hip"), "_ZN4pmqa20indexer_nvfp4_kernel")
    assert count_ops(body, "v_cvt_scalef32_pk_f16_fp4") == 80
    assert count_ops(body, "v_pk_mul_f16") == 80
    assert count_ops(body, "v_mul_f32") == 0
    assert count_ops(body, "v_cvt_pk_bf16_f32") == 0
    # the counter sees the older form
    old = "_ZN4pmqa20indexer_nvfp4_kernelILi1EEEvX: ; @k\n\tv_mul_f32_e32 v1, v2, v3\n\ts_endpgm\n.Lfunc_end1:\n"
    assert count_ops(kernel_body(old, "_ZN4pmqa20indexer_nvfp4_kernel"), "v_mul_f32") == 1
