"""The C-ABI library: it loads, exports every function include/pmqa.h declares,
and its host-side validation returns the documented status codes.  None of
these calls reaches the GPU (each is rejected, or is a no-op, before any
launch), so they run without one.  Every case here must stay a rejection or a
no-op: the addresses are fake, so an accepted call would launch kernels on
them."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pmqa.h")

OK, NULL, SHAPE, UNSUP, ALIGN, WORKSPACE = 0, -1, -2, -3, -4, -5
FAKE = 0x10000  # an aligned, never dereferenced address


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def pm():
    from paged_mqa_logits_02_amd import LIB_PATH
    if not os.path.exists(LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    import paged_mqa_logits_02_amd as m
    return m


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("mqa_logits_fp8", "mqa_logits_mxfp4", "indexer_scores", "indexer_scores_nvfp4",
              "mqa_logits_schedule",
              "mqa_logits_schedule_ints", "mqa_logits_num_units", "mqa_logits_padded_seq_len",
              "mqa_logits_min_block_table_width", "mqa_logits_init", "mqa_logits_status_string"):
        assert n in names, n


def test_workspace_bytes(pm):
    assert pm.workspace_bytes() == 1024  # one 128-byte counter line per XCD


def test_library_exports_every_declared_symbol(pm):
    lib = ctypes.CDLL(pm.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_library_does_not_link_the_oracle(pm):
    import subprocess
    out = subprocess.run(["nm", "-D", pm.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in out


def test_helpers(pm):
    assert pm.padded_seq_len(0) == 0 and pm.padded_seq_len(-4) == 0
    assert pm.padded_seq_len(1) == 64 and pm.padded_seq_len(64) == 64
    assert pm.padded_seq_len(65) == 128 and pm.padded_seq_len(32768) == 32768
    assert pm.min_block_table_width(0) == 0 and pm.min_block_table_width(1) == 1
    assert pm.min_block_table_width(200) == 4 and pm.min_block_table_width(131072) == 2048
    assert pm.schedule_ints(1) == 8 + 3 * 2
    assert pm.schedule_ints(0) == -1 and pm.schedule_ints(1 << 21) == -1
    for s in (0, -1, -2, -3, -4, -5, -6, 17):
        assert isinstance(pm.status_string(s), str)


def _fp8(lib, **kw):
    a = dict(q=FAKE, kv=FAKE, ps=8448, npages=10, w=FAKE, sl=FAKE, bt=FAKE, bts=4, btw=4, B=2,
             N=1, H=64, D=128, out=FAKE, ors=256, maxc=256, od=0, acc=0, sched=None,
             ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.mqa_logits_fp8(a["q"], a["kv"], a["ps"], a["npages"], a["w"], a["sl"], a["bt"],
                              a["bts"], a["btw"], a["B"], a["N"], a["H"], a["D"], a["out"],
                              a["ors"], a["maxc"], a["od"], a["acc"], a["sched"], a["ws"],
                              a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,rc", [
    (dict(H=129), UNSUP), (dict(D=72), UNSUP), (dict(D=272, ps=64 * 276), UNSUP),
    (dict(H=0), SHAPE), (dict(D=0), SHAPE), (dict(acc=1), UNSUP),
    (dict(od=2), UNSUP), (dict(N=9), UNSUP), (dict(N=65), SHAPE), (dict(N=0), SHAPE),
    (dict(maxc=100), SHAPE), (dict(H=32, D=256), SHAPE), (dict(D=64, ps=64 * 68 - 16), SHAPE),
    (dict(maxc=-64), SHAPE), (dict(B=-1), SHAPE), (dict(B=8193), SHAPE),
    (dict(q=None), NULL), (dict(kv=None), NULL), (dict(out=None), NULL), (dict(sl=None), NULL),
    (dict(ps=8440), SHAPE), (dict(ps=8448 + 8), ALIGN), (dict(btw=3), SHAPE),
    (dict(bts=3), SHAPE), (dict(ors=200), SHAPE), (dict(npages=0), SHAPE),
    (dict(q=FAKE + 8), ALIGN), (dict(w=FAKE + 4), ALIGN), (dict(sl=FAKE + 2), ALIGN),
    (dict(B=0), OK), (dict(maxc=0, ors=0), OK),
    (dict(ws=FAKE, wsb=1023), WORKSPACE), (dict(ws=FAKE, wsb=0), WORKSPACE),
    (dict(ws=FAKE + 4, wsb=1024), ALIGN), (dict(ws=FAKE, wsb=1024, B=0), OK),
    (dict(ws=FAKE, wsb=1 << 20, B=-1), SHAPE), (dict(ws=None, wsb=3, B=0), OK),
])
def test_fp8_validation(pm, kw, rc):
    assert _fp8(pm.library(), **kw) == rc


def _mx(lib, **kw):
    a = dict(q=FAKE, qsf=FAKE, sfv=32, inter=0, kv=FAKE, ps=4352, npages=10, w=FAKE, sl=FAKE,
             bt=FAKE, bts=4, btw=4, B=2, N=2, H=64, D=128, out=FAKE, ors=256, maxc=256, od=1,
             sched=None, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.mqa_logits_mxfp4(a["q"], a["qsf"], a["sfv"], a["inter"], a["kv"], a["ps"],
                                a["npages"], a["w"], a["sl"], a["bt"], a["bts"], a["btw"], a["B"],
                                a["N"], a["H"], a["D"], a["out"], a["ors"], a["maxc"], a["od"],
                                a["sched"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,rc", [
    (dict(sfv=16), SHAPE), (dict(sfv=16, ps=4608, B=0), OK), (dict(sfv=8), UNSUP),
    (dict(sfv=64), UNSUP), (dict(sfv=0), UNSUP), (dict(inter=2), UNSUP), (dict(inter=-1), UNSUP),
    (dict(inter=1, B=0), OK), (dict(H=32), UNSUP), (dict(D=256), UNSUP),
    (dict(qsf=None), NULL), (dict(ps=4340), SHAPE), (dict(ps=4352 + 4), ALIGN),
    (dict(N=9), UNSUP), (dict(B=0), OK), (dict(ws=FAKE, wsb=512), WORKSPACE),
    (dict(ws=FAKE + 8, wsb=1024), ALIGN),
])
def test_mxfp4_validation(pm, kw, rc):
    assert _mx(pm.library(), **kw) == rc


def _idx(lib, **kw):
    a = dict(q=FAKE, rows=24, D=128, kc=FAKE, ps=16384, npages=384, bt=FAKE, bts=64, btw=64,
             nreq=6, lens=FAKE, reqs=FAKE, groups=6, offs=None, scores=FAKE, srs=4096,
             maxc=4096, stream=None)
    a.update(kw)
    return lib.indexer_scores(a["q"], a["rows"], a["D"], a["kc"], a["ps"], a["npages"], a["bt"],
                              a["bts"], a["btw"], a["nreq"], a["lens"], a["reqs"], a["groups"],
                              a["offs"], a["scores"], a["srs"], a["maxc"], a["stream"])


@pytest.mark.parametrize("kw,rc", [
    (dict(D=64), UNSUP), (dict(groups=5), SHAPE), (dict(groups=2), SHAPE),
    (dict(groups=65536, rows=65536), SHAPE), (dict(maxc=4000), SHAPE),
    (dict(maxc=65536 * 64, btw=65536, bts=65536, srs=65536 * 64), SHAPE),
    (dict(ps=16384 - 16), SHAPE), (dict(ps=16384 + 8), ALIGN), (dict(btw=32), SHAPE),
    (dict(srs=100), SHAPE), (dict(scores=None), NULL), (dict(reqs=None), NULL),
    (dict(q=FAKE + 2), ALIGN), (dict(nreq=0), SHAPE), (dict(groups=0), OK),
])
def test_indexer_validation(pm, kw, rc):
    assert _idx(pm.library(), **kw) == rc


def _idx4(lib, **kw):
    a = dict(q=FAKE, qs=FAKE, rows=24, D=128, kc=FAKE, ps=4096, ks=FAKE, sps=512, npages=384,
             bt=FAKE, bts=64, btw=64, nreq=6, lens=FAKE, reqs=FAKE, groups=6, offs=None,
             scores=FAKE, srs=4096, maxc=4096, stream=None)
    a.update(kw)
    return lib.indexer_scores_nvfp4(a["q"], a["qs"], a["rows"], a["D"], a["kc"], a["ps"],
                                    a["ks"], a["sps"], a["npages"], a["bt"], a["bts"], a["btw"],
                                    a["nreq"], a["lens"], a["reqs"], a["groups"], a["offs"],
                                    a["scores"], a["srs"], a["maxc"], a["stream"])


@pytest.mark.parametrize("kw,rc", [
    (dict(D=64), UNSUP), (dict(groups=5), SHAPE), (dict(ps=4096 - 16), SHAPE),
    (dict(ps=4096 + 8), ALIGN), (dict(sps=504), SHAPE), (dict(sps=516), ALIGN),
    (dict(qs=None), NULL), (dict(ks=None), NULL), (dict(q=None), NULL),
    (dict(qs=FAKE + 1), ALIGN), (dict(q=FAKE + 8), ALIGN), (dict(btw=32), SHAPE),
    (dict(maxc=65536 * 64, btw=65536, bts=65536, srs=65536 * 64), SHAPE), (dict(groups=0), OK),
])
def test_indexer_nvfp4_validation(pm, kw, rc):
    assert _idx4(pm.library(), **kw) == rc


def test_schedule_validation(pm):
    lib = pm.library()
    assert lib.mqa_logits_schedule(FAKE, 4, 9, 0, 256, 8, FAKE, None) == UNSUP
    assert lib.mqa_logits_schedule(FAKE, 4, 1, 2, 256, 8, FAKE, None) == UNSUP
    assert lib.mqa_logits_schedule(FAKE, 4, 1, 0, 100, 8, FAKE, None) == SHAPE
    assert lib.mqa_logits_schedule(FAKE, 4, 1, 0, 256, -1, FAKE, None) == SHAPE
    assert lib.mqa_logits_schedule(FAKE, 4, 1, 0, 256, 8, None, None) == NULL
    assert lib.mqa_logits_schedule(FAKE + 2, 4, 1, 0, 256, 8, FAKE, None) == ALIGN
    assert lib.mqa_logits_num_units(0, 9, 0) == UNSUP


def test_read_calibration_library_rejects_bad_arguments(pm):
    """The page-gather read-rate kernel of bench.py --read-calibration lives in
    its own library; its argument checks run before any launch."""
    path = os.path.join(ROOT, "paged_mqa_logits_02_amd", "libpmqa_calib.so")
    if not os.path.exists(path):
        import __graft_entry__
        __graft_entry__.build()
    lib = ctypes.CDLL(path)
    fn = lib.pmqa_calib_read_pages
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_void_p,
                   ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    good = dict(pool=FAKE, stride=8448, size=8448, ids=FAKE, n=4, out=FAKE, grid=4)
    for bad in (dict(pool=None), dict(ids=None), dict(out=None), dict(n=0), dict(grid=0),
                dict(size=8), dict(size=8450), dict(size=40000, stride=40000),
                dict(stride=8000), dict(stride=8456)):
        a = dict(good, **bad)
        assert fn(a["pool"], a["stride"], a["size"], a["ids"], a["n"], a["out"], a["grid"],
                  None) == -1, bad
    out = __import__("subprocess").run(["nm", "-D", pm.LIB_PATH], capture_output=True,
                                       text=True).stdout
    assert "pmqa_calib" not in out  # not part of the logits library
