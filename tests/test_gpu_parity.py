"""GPU parity: the HIP path against the CPU oracle, through the C ABI.

Written sets are compared exactly (sentinel-filled outputs); values within
|gpu - ref| <= 2e-3*A + 1e-5 (fp32 out) or 1e-2*A + 1e-5 (bf16 out), with
A = s_p * sum_h |w| * relu(q.k); exact-arithmetic inputs bit-exactly."""
import copy

import numpy as np
import pytest
import torch

import oracle
import synth
import fixtures_util
from fixtures_util import (extent, indexer_from_case, load_golden, mqa_from_case)
from gpu_util import (DEV, DevIndexer, DevMqa, check_cells, check_dense, check_indexer,
                      check_sampled, check_values, host_out, page_edge_cells, pm, say, tol_for)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    pm().init()
    yield
    torch.cuda.synchronize()


# ----------------------------------------------------------- small / exact


def test_tiny_fp8_config():
    inp = synth.make_config("tiny_fp8")
    dm = DevMqa(inp)
    say("tiny_fp8: B=2 N=1 seq_lens=%s" % inp.seq_lens.tolist())
    r = check_dense(dm, dm.run(), "tiny_fp8")
    say("tiny_fp8 max err/tol %.3g" % r)


@pytest.mark.parametrize("case", load_golden("fp8_logits_cases.json")["cases"],
                         ids=lambda c: c["name"])
def test_fp8_golden_bit_exact(case):
    inp = mqa_from_case(case, "fp8")
    got, wrote = host_out(DevMqa(inp).run())
    E = extent(case["seq_len"], inp.max_context)
    assert wrote[0, :E].all() and not wrote[0, E:].any()
    for col, v in case["expected"].items():
        assert got[0, int(col)] == v, (case["name"], col, got[0, int(col)])


@pytest.mark.parametrize("case", load_golden("mxfp4_logits_cases.json")["cases"],
                         ids=lambda c: c["name"])
def test_mxfp4_golden_bit_exact(case):
    inp = mqa_from_case(case, "mxfp4")
    for dtype in (torch.float32, torch.bfloat16):
        got, _ = host_out(DevMqa(inp).run(dtype=dtype))
        for col, v in case["expected"].items():
            assert got[0, int(col)] == v, (case["name"], col, dtype)


@pytest.mark.parametrize("case", load_golden("indexer_cases.json")["cases"],
                         ids=lambda c: c["name"])
def test_indexer_golden_bit_exact(case):
    di = DevIndexer(indexer_from_case(case))
    got, wrote = host_out(di.run())
    L = case["context_length"]
    assert wrote[:, :L].all() and not wrote[:, L:].any()
    for r, exp in enumerate(case["expected"]):
        for col, v in exp.items():
            if int(col) < L:
                assert got[r, int(col)] == v


RAGGED = [0, 1, 63, 64, 65, 200, 700, 1000, -5, 3000, 129, 2048]


@pytest.mark.parametrize("variant", ["fp8", "mxfp4"])
@pytest.mark.parametrize("next_n", [1, 2, 3, 4])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_batch(variant, next_n, dtype):
    """Empty, one-token, page-boundary, negative and over-long (clamped)
    lengths; every next_n; both output types."""
    inp = synth.make_mqa_inputs(RAGGED, next_n, variant=variant, max_context=2048, bt_width=40,
                                seed=100 + next_n, w_std=0.5, out_dtype=dtype, extra_pages=5)
    say("ragged %s N=%d %s" % (variant, next_n, dtype))
    dm = DevMqa(inp)
    check_dense(dm, dm.run(), "ragged %s N=%d %s" % (variant, next_n, dtype))


def _exact_inputs(variant, next_n, seed, grid=(0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0)):
    """Values on a coarse dyadic grid, so every partial sum is exact in fp32."""
    rng = np.random.default_rng(seed)
    inp = synth.make_mqa_inputs([300, 64, 1, 129], next_n, variant=variant, max_context=320,
                                bt_width=5, seed=seed)
    grid = np.array(grid, dtype=np.float32)
    qf = rng.choice(grid, (inp.batch, next_n, 64, 128)).astype(np.float32)
    kf = rng.choice(grid, (inp.num_pages, 64, 128)).astype(np.float32)
    if variant == "fp8":
        inp.q = synth.encode_e4m3(qf)
        inp.kv[:, : 64 * 128] = synth.encode_e4m3(kf).reshape(inp.num_pages, -1)
        sp = np.ldexp(1.0, rng.integers(-4, 4, (inp.num_pages, 64))).astype(np.float32)
        inp.kv[:, 64 * 128: 64 * 128 + 256] = sp.view(np.uint8)
    else:
        inp.q, inp.q_sf = synth.quantize_mxfp4(qf)
        inp.q_sf[:] = 127
        packed, _ = synth.quantize_mxfp4(kf)
        inp.kv[:, : 64 * 64] = packed.reshape(inp.num_pages, -1)
        inp.kv[:, 64 * 64: 64 * 64 + 256] = 127
    inp.weights[:] = rng.choice(np.array([0.5, -0.5, 1.0, -1.0, 2.0, -2.0], np.float32),
                                inp.weights.shape)
    return inp


@pytest.mark.parametrize("variant", ["fp8", "mxfp4"])
@pytest.mark.parametrize("next_n", [1, 4])
def test_exact_arithmetic_bit_exact(variant, next_n):
    """fp32 output: the rectifier and weighted head sum run in fp32, so on the
    dyadic grid (partial sums exact in fp32) the result equals the oracle."""
    inp = _exact_inputs(variant, next_n, 200 + next_n)
    ref, _, written = oracle.mqa_logits_for(inp)
    dm = DevMqa(inp)
    got, wrote = host_out(dm.run(dtype=torch.float32))
    assert np.array_equal(wrote, written)
    assert np.array_equal(got[written], ref[written])


@pytest.mark.parametrize("variant", ["fp8", "mxfp4"])
@pytest.mark.parametrize("next_n", [1, 2, 3, 4, 6])
def test_bf16_head_sum_on_matrix_unit_exact(variant, next_n):
    """bf16 output sums the heads on the matrix unit: every rectified score and
    weight is rounded to bf16 once before the sum.  With q, k in {0, +-1} (unit
    block scales for MXFP4, s_p = 2^k for FP8) every score is an integer of
    magnitude <= 128 (exact in bf16) and the weights are powers of two, so the
    result must equal the oracle's bf16 rounding bit for bit; the fp32 output
    of the same inputs must equal the oracle exactly."""
    inp = _exact_inputs(variant, next_n, 230 + next_n, grid=(0.0, 1.0, -1.0))
    ref, _, written = oracle.mqa_logits_for(inp)
    say("%s N=%d bf16 head sum on the matrix unit, %d cells" % (variant, next_n,
                                                                int(written.sum())))
    dm = DevMqa(inp)
    gotb, wroteb = host_out(dm.run(dtype=torch.bfloat16))
    assert np.array_equal(wroteb, written)
    refb = torch.from_numpy(ref[written]).float().bfloat16().double().numpy()
    assert np.array_equal(gotb[written], refb)
    got, _ = host_out(dm.run(dtype=torch.float32))
    assert np.array_equal(got[written], ref[written])


@pytest.mark.parametrize("variant", ["fp8", "mxfp4"])
@pytest.mark.parametrize("next_n", [1, 4])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_extreme_magnitudes(variant, next_n, dtype):
    """Scores far from 1: FP8 q and k at +-448 (|q.k| up to 128 * 448^2, about
    2.6e7) with large and tiny weights; MXFP4 with e8m0 block scales from 2^-20
    to 2^20 (scores up to ~2^45).  Both output paths (the fp32 epilogue and the
    bf16 head sum) must stay within the tolerance without overflow."""
    rng = np.random.default_rng(240 + next_n)
    inp = synth.make_mqa_inputs([300, 64, 1, 129], next_n, variant=variant, max_context=320,
                                bt_width=5, seed=241 + next_n, out_dtype=dtype)
    if variant == "fp8":
        sign = lambda shape: np.where(rng.random(shape) < 0.5, -448.0, 448.0)  # noqa: E731
        qf = sign((inp.batch, next_n, 64, 128)) * (rng.random((inp.batch, next_n, 64, 128)) < 0.9)
        kf = sign((inp.num_pages, 64, 128))
        inp.q = synth.encode_e4m3(qf.astype(np.float32))
        inp.kv[:, : 64 * 128] = synth.encode_e4m3(kf.astype(np.float32)).reshape(inp.num_pages, -1)
    else:
        inp.q_sf[:] = rng.integers(127 - 20, 127 + 21, inp.q_sf.shape).astype(np.uint8)
        sf = rng.integers(127 - 20, 127 + 21, (inp.num_pages, 64, 4)).astype(np.uint8)
        inp.kv[:, 64 * 64: 64 * 64 + 256] = sf.reshape(inp.num_pages, -1)
    w = rng.standard_normal(inp.weights.shape).astype(np.float32)
    w *= np.ldexp(1.0, rng.integers(-12, 13, w.shape)).astype(np.float32)
    inp.weights[:] = w
    say("extreme magnitudes %s N=%d %s" % (variant, next_n, dtype))
    dm = DevMqa(inp)
    check_dense(dm, dm.run(), "extreme %s N=%d %s" % (variant, next_n, dtype))


def test_one_head_fp8_equals_rectified_indexer_on_gpu():
    rng = np.random.default_rng(20)
    grid = np.array([0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0])
    inp = synth.make_mqa_inputs([100], 1, max_context=128, bt_width=2, seed=21)
    qf = np.zeros((1, 1, 64, 128), dtype=np.float32)
    qf[0, 0, 0] = rng.choice(grid, 128)
    inp.q = synth.encode_e4m3(qf)
    kf = rng.choice(grid, (inp.num_pages, 64, 128)).astype(np.float32)
    inp.kv[:, : 64 * 128] = synth.encode_e4m3(kf).reshape(inp.num_pages, -1)
    inp.kv[:, 64 * 128: 64 * 128 + 256] = np.ones((inp.num_pages, 64), np.float32).view(np.uint8)
    inp.weights[:] = 0.0
    inp.weights[0, 0] = 1.0
    fp8, _ = host_out(DevMqa(inp).run())
    kc = synth.encode_bf16(kf).view(np.uint8).reshape(inp.num_pages, -1)
    ix = synth.IndexerInputs(synth.encode_bf16(qf[0, 0, :1]), kc, 64 * 128 * 2, inp.block_table,
                             np.array([128], np.int32), np.array([0], np.int32),
                             np.array([0, 1], np.int32), 128)
    sc, _ = host_out(DevIndexer(ix).run())
    assert np.array_equal(np.maximum(sc[0, :128], 0.0), fp8[0, :128])


# ----------------------------------------------------------- indexer config


@pytest.mark.parametrize("uniform", [None, 4, 1, 8])
def test_indexer_config(uniform):
    ix = synth.make_config("indexer_bf16", uniform_group=uniform)
    say("indexer groups=%d uniform=%s lens=%s" % (ix.groups, uniform, ix.context_lengths.tolist()))
    di = DevIndexer(ix)
    check_indexer(di, di.run(), "indexer uniform=%s" % uniform)


def test_indexer_strided_pages():
    """Pages any multiple of 16 bytes apart: a view into a cache that holds
    each page's keys and then other bytes."""
    ix = synth.make_config("indexer_bf16")
    wide = synth.make_config("indexer_bf16", page_stride=64 * 128 * 2 + 16 * 37)
    a, _ = host_out(DevIndexer(ix).run())
    b, _ = host_out(DevIndexer(wide).run())
    assert np.array_equal(a.view(np.uint64), b.view(np.uint64))


# ------------------------------------------------------ NVFP4 indexer


@pytest.mark.parametrize("case", load_golden("indexer_nvfp4_cases.json")["cases"],
                         ids=lambda c: c["name"])
def test_indexer_nvfp4_golden_bit_exact(case):
    from fixtures_util import nvfp4_indexer_from_case
    di = DevIndexer(nvfp4_indexer_from_case(case))
    got, wrote = host_out(di.run())
    L = case["context_length"]
    assert wrote[:, :L].all() and not wrote[:, L:].any()
    for r, exp in enumerate(case["expected"]):
        for col, v in exp.items():
            if int(col) < L:
                assert got[r, int(col)] == v


@pytest.mark.parametrize("uniform", [None, 4, 1, 8])
def test_indexer_nvfp4_config(uniform):
    ix = synth.make_config("indexer_nvfp4", uniform_group=uniform)
    say("nvfp4 indexer groups=%d uniform=%s" % (ix.groups, uniform))
    di = DevIndexer(ix)
    check_indexer(di, di.run(), "nvfp4 indexer uniform=%s" % uniform)


@pytest.mark.parametrize("name", ["indexer_bf16_8k", "indexer_nvfp4_8k"])
def test_indexer_8192_rows_dense(name):
    """The bandwidth-sized indexer workloads the bench times (8192 query rows in
    groups of 1..8 over 512 requests of 64 pages), every written cell against
    the dense oracle."""
    ix = synth.make_config(name)
    say("%s groups=%d rows=%d" % (name, ix.groups, ix.rows))
    di = DevIndexer(ix)
    check_indexer(di, di.run(), name)


def test_indexer_nvfp4_fused_pages():
    """Keys and scales as two views of one cache holding each page's keys and
    then their scales (page stride a multiple of 16, not of the key size):
    bit-identical to separate buffers."""
    ix = synth.make_config("indexer_nvfp4")
    P = ix.key_cache.shape[0]
    stride = 4096 + 512 + 16 * 3
    fused = np.zeros((P, stride), dtype=np.uint8)
    fused[:, :4096] = ix.key_cache[:, :4096]
    fused[:, 4096:4608] = ix.key_scales[:, :512]
    dev = torch.from_numpy(fused).to(DEV)
    a, _ = host_out(DevIndexer(ix).run())
    b, _ = host_out(DevIndexer(ix, key_cache=dev[:, :4096], key_scales=dev[:, 4096:4608]).run())
    assert np.array_equal(a.view(np.uint64), b.view(np.uint64))


def test_indexer_nvfp4_out_of_range_page_is_nan():
    ix = synth.make_config("indexer_nvfp4")
    g = int(np.argmax(ix.context_lengths))
    bad = copy.copy(ix)
    bad.block_table = ix.block_table.copy()
    bad.block_table[ix.requests[g], 0] = ix.key_cache.shape[0] + 3
    got, wrote = host_out(DevIndexer(bad).run())
    ref, amag, written = oracle.indexer_scores_for(ix)
    assert np.array_equal(wrote, written)
    poison = np.zeros_like(written)
    poison[:, :64] = True
    rows_of = np.zeros(ix.rows, dtype=bool)
    offs = ix.row_offsets()
    for h in range(ix.groups):
        if ix.requests[h] == ix.requests[g] and ix.context_lengths[h] > 0:
            rows_of[offs[h]:offs[h + 1]] = True
    poison &= rows_of[:, None] & written
    assert poison.any() and np.isnan(got[poison]).all()
    ok = written & ~poison
    check_values(got[ok], ref[ok], np.abs(ref[ok]) + 0 * amag[ok], (2e-3, 1e-5), "valid pages")


# ------------------------------------------------------- full-size configs


@pytest.mark.parametrize("name,mode", [
    (n, m) for n in ("decode_fp8", "verify_fp8", "mxfp4")
    for m in ("in_call", "schedule", "work_counter")
] + [("verify_fp8_bf16", "in_call"), ("mxfp4_n4", "in_call")])
def test_full_size_config(name, mode):
    inp = synth.make_config(name)
    say("%s %s: B=%d N=%d pages=%d positions=%d" % (name, mode, inp.batch, inp.next_n,
                                                    inp.num_pages, inp.kv_positions()))
    dm = DevMqa(inp)
    sched = None
    if mode == "schedule":
        sched = pm().mqa_logits_schedule(dm.sl, inp.next_n,
                                         0 if inp.variant == "fp8" else 1,
                                         max_context=inp.max_context)
    ws = pm().workspace(DEV) if mode == "work_counter" else None
    out = dm.run(schedule=sched, workspace=ws)
    what = "%s %s" % (name, mode)
    if ws is not None:
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0, "the work counter was not left at zero"
    if name == "decode_fp8":
        # every written cell (about 0.6 M) against the dense oracle
        r = check_dense(dm, out, what)
        say("%s: dense, max err/tol %.3g" % (what, r))
        return
    r = check_sampled(dm, out, np.random.default_rng(7), what)
    rows, cols = page_edge_cells(inp)
    re = check_cells(dm, out, rows, cols, what + " page edges")
    say("%s max err/tol %.3g sampled, %.3g over the first and last column of all %d pages x rows"
        % (what, r, re, rows.size // 2))


# ------------------------------------------------------- schedule / graphs


def _mid_inputs(variant="fp8", next_n=2, seed=300):
    lens = np.random.default_rng(seed).integers(0, 3000, 23)
    lens[3] = 0
    return synth.make_mqa_inputs(lens, next_n, variant=variant, max_context=3072, bt_width=48,
                                 seed=seed)


@pytest.mark.parametrize("variant", ["fp8", "mxfp4"])
@pytest.mark.parametrize("next_n", [2, 4])
def test_schedule_any_unit_count_bit_identical(variant, next_n):
    """Any unit count, and the default one (next_n 4 FP8: the split weighted
    by dispatch round, in the kernel and in the schedule), gives the in-call
    result bit for bit."""
    inp = _mid_inputs(variant, next_n=next_n)
    dm = DevMqa(inp)
    base, wb = host_out(dm.run())
    v = 0 if variant == "fp8" else 1
    for U in (1, 7, 256, 1024, 5000, 0):
        sched = pm().mqa_logits_schedule(dm.sl, inp.next_n, v, max_context=inp.max_context,
                                         num_units=U)
        got, wg = host_out(dm.run(schedule=sched))
        assert np.array_equal(wb, wg), U
        assert np.array_equal(got.view(np.uint64), base.view(np.uint64)), U
    check_dense(dm, dm.run(), "mid %s" % variant)


def test_schedule_entries_name_each_units_request_and_page():
    """Each unit entry of a schedule holds (request, page, flat item) of its
    first item: the request is the last one whose page prefix is <= the item
    (requests with no pages are skipped), the page the offset into it, and the
    end entry (request B, page 0).  A regression test: the entries were once
    computed with a wave-uniform search on per-lane items.  (Layout: 8 header
    ints, then 3 ints per unit and one end entry.)"""
    inp = _mid_inputs("fp8", next_n=2)
    dm = DevMqa(inp)
    B = len(inp.seq_lens)
    tiles = np.minimum((inp.seq_lens.astype(np.int64) + 63) // 64, inp.max_context // 64)
    prefix = np.concatenate([[0], np.cumsum(tiles)])
    for U in (7, 64, 1000):
        sched = pm().mqa_logits_schedule(dm.sl, inp.next_n, 0, max_context=inp.max_context,
                                         num_units=U).cpu().numpy()
        assert sched[1] == U and sched[5] == B and sched[6] == prefix[-1]
        e = sched[8:8 + 3 * (U + 1)].reshape(U + 1, 3)
        f = e[:, 2].astype(np.int64)
        assert f[0] == 0 and f[-1] == prefix[-1] and np.all(np.diff(f) >= 0)
        b = np.searchsorted(prefix, f[:-1], side="right") - 1
        assert np.array_equal(e[:-1, 0], b), U
        assert np.array_equal(e[:-1, 1], f[:-1] - prefix[b]), U
        assert list(e[-1, :2]) == [B, 0]


def test_mxfp4_grid_keeps_at_most_six_workgroups_per_cu():
    """MXFP4 launches one range per resident workgroup and at most 6 per CU
    (7 fit some layouts by registers and LDS and ran slower); FP8 keeps what
    its registers and LDS allow."""
    cus = torch.cuda.get_device_properties(DEV).multi_processor_count
    for next_n in (1, 2, 3, 4):
        u = pm().num_units(next_n, 1)
        assert u % cus == 0 and 1 <= u // cus <= 6, (next_n, u, cus)
        f = pm().num_units(next_n, 0)
        assert f % cus == 0 and f // cus >= 1, (next_n, f, cus)


def test_schedule_for_other_arguments_is_ignored():
    inp = _mid_inputs("fp8", next_n=2)
    dm = DevMqa(inp)
    base, _ = host_out(dm.run())
    wrong = pm().mqa_logits_schedule(dm.sl, 3, 0, max_context=inp.max_context, num_units=64)
    got, _ = host_out(dm.run(schedule=wrong))
    assert np.array_equal(got.view(np.uint64), base.view(np.uint64))


@pytest.mark.parametrize("variant", ["fp8", "mxfp4"])
def test_schedule_built_before_lengths_grew_is_ignored(variant):
    """A schedule built for the same batch, next_n, variant and max_context but
    shorter seq_lens (as a decode loop that reused it would pass) covers fewer
    items; the kernel sees that its total differs from the current lengths'
    and splits the call itself, so every item is scored."""
    inp = _mid_inputs(variant, next_n=2)
    dm = DevMqa(inp)
    base, wrote0 = host_out(dm.run())
    shorter = torch.clamp(dm.sl - 130, min=0)
    stale = pm().mqa_logits_schedule(shorter, 2, 0 if variant == "fp8" else 1,
                                     max_context=inp.max_context)
    got, wrote = host_out(dm.run(schedule=stale))
    assert np.array_equal(wrote, wrote0)
    assert np.array_equal(got.view(np.uint64), base.view(np.uint64))


def test_repeat_runs_bit_identical():
    inp = _mid_inputs("fp8", next_n=4, seed=301)
    dm = DevMqa(inp)
    a, _ = host_out(dm.run())
    for _ in range(3):
        b, _ = host_out(dm.run())
        assert np.array_equal(a.view(np.uint64), b.view(np.uint64))


def _graph_inputs(variant, seed):
    """Same shapes for every seed: 23 requests, a full block table of
    23 x 48 valid page ids, random lengths."""
    lens = np.random.default_rng(seed).integers(0, 3000, 23)
    lens[seed % 23] = 0
    return synth.make_mqa_inputs(lens, 2, variant=variant, max_context=3072, bt_width=48,
                                 seed=seed, full_table=True)


@pytest.mark.parametrize("variant", ["fp8", "mxfp4"])
def test_graph_replay_with_changed_inputs(variant):
    """Schedule + logits captured once; seq_lens, q, weights, pages and the
    block table change between replays; every replay matches the oracle for
    the inputs of that replay."""
    inp = _graph_inputs(variant, 302)
    dm = DevMqa(inp)
    v = 0 if variant == "fp8" else 1
    U = pm().num_units(inp.next_n, v)
    sched = torch.empty(pm().schedule_ints(U), dtype=torch.int32, device=DEV)
    out = dm.new_out()
    dm.run(out=out)  # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pm().mqa_logits_schedule(dm.sl, inp.next_n, v, max_context=inp.max_context,
                                 num_units=U, out=sched)
        dm.run(out=out, schedule=sched)
    for rep in range(3):
        new = _graph_inputs(variant, 400 + rep)
        dm.sl.copy_(torch.from_numpy(new.seq_lens))
        dm.q.copy_(torch.from_numpy(new.q))
        if new.q_sf is not None:
            dm.q_sf.copy_(torch.from_numpy(new.q_sf))
        dm.w.copy_(torch.from_numpy(new.weights))
        dm.kv.copy_(torch.from_numpy(new.kv))
        dm.bt.copy_(torch.from_numpy(new.block_table))
        fresh = dm.new_out()
        out.copy_(fresh)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        dm.inp = new
        check_dense(dm, out, "%s replay %d" % (variant, rep))


@pytest.mark.parametrize("variant,next_n", [("fp8", 1), ("fp8", 2), ("fp8", 4), ("fp8", 6),
                                            ("mxfp4", 2), ("mxfp4", 3)])
def test_work_counter_bit_identical_and_left_zero(variant, next_n):
    """With a workspace the last items of the call go to whichever workgroups
    finish first: the logits are bit-identical to the static split, and
    every call (one or two launches) leaves the counter at zero."""
    inp = _mid_inputs(variant, next_n, seed=320 + next_n)
    dm = DevMqa(inp)
    say("work counter %s N=%d" % (variant, next_n))
    ref, wref = host_out(dm.run())
    ws = pm().workspace(DEV)
    for _ in range(3):
        got, wrote = host_out(dm.run(workspace=ws))
        assert np.array_equal(wrote, wref)
        assert np.array_equal(got.view(np.uint64), ref.view(np.uint64))
        assert int(ws.count_nonzero()) == 0


@pytest.mark.parametrize("variant", ["fp8", "mxfp4"])
def test_graph_replay_with_work_counter(variant):
    """A call with a workspace captured once and replayed with changed
    inputs: every replay matches the oracle and leaves the counter at zero
    (the graph holds no clearing of it)."""
    inp = _graph_inputs(variant, 305)
    dm = DevMqa(inp)
    ws = pm().workspace(DEV)
    out = dm.new_out()
    dm.run(out=out, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dm.run(out=out, workspace=ws)
    for rep in range(3):
        new = _graph_inputs(variant, 410 + rep)
        dm.sl.copy_(torch.from_numpy(new.seq_lens))
        dm.q.copy_(torch.from_numpy(new.q))
        if new.q_sf is not None:
            dm.q_sf.copy_(torch.from_numpy(new.q_sf))
        dm.w.copy_(torch.from_numpy(new.weights))
        dm.kv.copy_(torch.from_numpy(new.kv))
        dm.bt.copy_(torch.from_numpy(new.block_table))
        out.copy_(dm.new_out())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0
        dm.inp = new
        check_dense(dm, out, "%s work-counter replay %d" % (variant, rep))


# ------------------------------------------------------------- invariants


def test_strided_pages_identical():
    a_in = _mid_inputs("fp8", next_n=1, seed=303)
    b_in = synth.make_mqa_inputs(a_in.seq_lens, 1, max_context=3072, bt_width=48, seed=303,
                                 page_stride=8448 + 16 * 5)
    assert np.array_equal(a_in.kv, b_in.kv[:, :8448])
    a, _ = host_out(DevMqa(a_in).run())
    b, _ = host_out(DevMqa(b_in).run())
    assert np.array_equal(a.view(np.uint64), b.view(np.uint64))


def test_page_permutation_bit_exact():
    inp = _mid_inputs("fp8", next_n=3, seed=304)
    base, _ = host_out(DevMqa(inp).run())
    perm = np.random.default_rng(1).permutation(inp.num_pages)
    p2 = copy.copy(inp)
    p2.kv = np.empty_like(inp.kv)
    p2.kv[perm] = inp.kv
    bt = inp.block_table.copy()
    bt[bt >= 0] = perm[bt[bt >= 0]]
    p2.block_table = bt
    got, _ = host_out(DevMqa(p2).run())
    assert np.array_equal(got.view(np.uint64), base.view(np.uint64))


def test_sp_power_of_two_scaling_exact():
    inp = _mid_inputs("fp8", next_n=1, seed=305)
    base, wrote = host_out(DevMqa(inp).run())
    sc = copy.copy(inp)
    sc.kv = inp.kv.copy()
    s = sc.kv[:, 8192:8448].copy().view(np.float32) * np.float32(8.0)
    sc.kv[:, 8192:8448] = s.view(np.uint8)
    got, _ = host_out(DevMqa(sc).run())
    assert np.array_equal(got[wrote], base[wrote] * 8.0)


def test_poisoned_unread_data_never_reaches_outputs():
    """Pages no request owns hold NaN codes (e4m3 0x7F, NaN scales); block-table
    entries past each length are -1; zero-length requests have garbage rows."""
    inp = synth.make_mqa_inputs([500, 0, 64, 1300], 2, max_context=1536, bt_width=24, seed=306,
                                extra_pages=6)
    used = set(inp.block_table[inp.block_table >= 0].tolist())
    for p in range(inp.num_pages):
        if p not in used:
            inp.kv[p, :] = 0x7F
            inp.kv[p, 8192:8448] = np.full(64, np.nan, np.float32).view(np.uint8)
    dm = DevMqa(inp)
    got, wrote = host_out(dm.run())
    assert not np.isnan(got[wrote]).any()
    check_dense(dm, dm.run(), "poisoned")


@pytest.mark.parametrize("variant", ["fp8", "mxfp4"])
def test_prepared_call_matches_direct_call(variant):
    """A PreparedCall (arguments marshalled once) issues the same call: its
    output is bit-identical to the direct call's, with and without a
    schedule, on every repeat."""
    inp = _mid_inputs(variant, next_n=2, seed=310)
    dm = DevMqa(inp)
    ref, _ = host_out(dm.run())
    m = pm()
    v = 0 if variant == "fp8" else 1
    sched_call = m.prepare_mqa_logits_schedule(dm.sl, inp.next_n, v, max_context=inp.max_context)
    for schedule in (None, sched_call.out):
        out = dm.new_out()
        if variant == "fp8":
            call = m.prepare_mqa_logits_fp8(dm.q, dm.kv, dm.w, dm.sl, dm.bt,
                                            max_context=inp.max_context, out=out,
                                            schedule_meta=schedule)
        else:
            call = m.prepare_mqa_logits_mxfp4(dm.q, dm.q_sf, dm.kv, dm.w, dm.sl, dm.bt,
                                              max_context=inp.max_context, out=out,
                                              schedule_meta=schedule)
        for _ in range(2):
            if schedule is not None:
                sched_call()
            got, _ = host_out(call())
            assert np.array_equal(got.view(np.uint64), ref.view(np.uint64))


@pytest.mark.parametrize("variant", ["fp8", "mxfp4"])
def test_out_of_range_page_id_gives_nan_for_that_page_only(variant):
    """A block-table entry outside [0, num_pages) is never dereferenced: the
    outputs of that page (every slot row of the request, the page's 64
    columns) are NaN, and every other written cell is as with a valid table.
    (Entries just past the pool, the int32 extremes and a small negative id;
    a request's first page is among them, which a range may start with.)"""
    inp = _mid_inputs(variant, next_n=2, seed=311)
    tiles = np.where(inp.seq_lens > 0, (inp.seq_lens + 63) // 64, 0)
    b1, b2 = [int(b) for b in np.nonzero(tiles >= 3)[0][:2]]
    bad = copy.copy(inp)
    bad.block_table = inp.block_table.copy()
    bad.block_table[b1, 1] = inp.num_pages + 7
    bad.block_table[b1, 2] = 2**31 - 1
    bad.block_table[b2, 0] = -2**31
    bad.block_table[b2, 2] = -5
    out = DevMqa(bad).run()
    got, wrote = host_out(out)
    ref, amag, written = oracle.mqa_logits_for(inp)
    assert np.array_equal(wrote, written)
    N = inp.next_n
    poison = np.zeros_like(written)
    poison[b1 * N:(b1 + 1) * N, 64:192] = True
    poison[b2 * N:(b2 + 1) * N, 0:64] = True
    poison[b2 * N:(b2 + 1) * N, 128:192] = True
    assert np.array_equal(poison & written, poison)
    assert np.isnan(got[poison]).all()
    ok = written & ~poison
    check_values(got[ok], ref[ok], amag[ok], tol_for(out.dtype), "valid pages")


def test_largest_batch():
    """B = 8192 requests, the largest batch the entry points accept (the
    per-request page-count prefix then fills 32 KB of LDS): complete written
    set, sampled values, in-call split and schedule."""
    rng = np.random.default_rng(312)
    lens = rng.integers(0, 300, 8192)
    lens[::97] = 0
    inp = synth.make_mqa_inputs(lens, 1, max_context=320, bt_width=5, seed=312)
    dm = DevMqa(inp)
    check_sampled(dm, dm.run(), np.random.default_rng(5), "in-call")
    sched = pm().mqa_logits_schedule(dm.sl, 1, 0, max_context=inp.max_context)
    check_sampled(dm, dm.run(schedule=sched), np.random.default_rng(6), "schedule")


# ------------------------------------------------------- strided views


@pytest.mark.parametrize("variant,H,D", [("fp8", 64, 128), ("mxfp4", 64, 128), ("fp8", 40, 80)],
                         ids=["fp8", "mxfp4", "fp8_general"])
def test_strided_output_and_block_table(variant, H, D):
    """out rows wider than max_context (a view into a wider buffer) and a block
    table that is a column slice of a wider table: values bit-identical to the
    dense layouts, and the columns past max_context untouched."""
    lens = np.random.default_rng(320).integers(0, 3000, 23)
    lens[5] = 0
    inp = synth.make_mqa_inputs(lens, 2, variant=variant, num_heads=H, head_dim=D,
                                max_context=3072, bt_width=48, seed=320)
    dm = DevMqa(inp)
    ref, ref_wrote = host_out(dm.run())
    m = pm()
    out_dtype = torch.float32 if inp.out_dtype == "f32" else torch.bfloat16
    wide = torch.empty((inp.rows, inp.max_context + 100), dtype=out_dtype, device=DEV)
    if out_dtype == torch.float32:
        wide.view(torch.int32).fill_(0x7FC0FFEE)
    else:
        wide.view(torch.int16).fill_(0x7FC1)
    view = wide[:, : inp.max_context]
    bt_wide = torch.full((inp.batch, 48 + 13), -1, dtype=torch.int32, device=DEV)
    bt_wide[:, :48] = dm.bt
    bt_view = bt_wide[:, :48]
    if variant == "fp8":
        m.mqa_logits_fp8(dm.q, dm.kv, dm.w, dm.sl, bt_view, max_context=inp.max_context, out=view)
    else:
        m.mqa_logits_mxfp4(dm.q, dm.q_sf, dm.kv, dm.w, dm.sl, bt_view,
                           max_context=inp.max_context, out=view)
    torch.cuda.synchronize()
    got, wrote = host_out(view.contiguous())
    assert np.array_equal(wrote, ref_wrote)
    assert np.array_equal(got[wrote], ref[wrote])
    tail = wide[:, inp.max_context:].contiguous().cpu()
    if out_dtype == torch.float32:
        assert (tail.view(torch.int32) == 0x7FC0FFEE).all()
    else:
        assert (tail.view(torch.int16) == 0x7FC1).all()


def test_indexer_strided_scores_and_block_table():
    ix = synth.make_config("indexer_bf16")
    di = DevIndexer(ix)
    ref, ref_wrote = host_out(di.run())
    wide = torch.empty((ix.rows, ix.max_context + 64), dtype=torch.float32, device=DEV)
    wide.view(torch.int32).fill_(0x7FC0FFEE)
    view = wide[:, : ix.max_context]
    W = di.bt.shape[1]
    bt_wide = torch.full((di.bt.shape[0], W + 7), -1, dtype=torch.int32, device=DEV)
    bt_wide[:, :W] = di.bt
    pm().indexer_scores(di.q, di.kc, bt_wide[:, :W], di.lens, requests=di.reqs, scores=view,
                        group_row_offsets=di.offs)
    torch.cuda.synchronize()
    got, wrote = host_out(view.contiguous())
    assert np.array_equal(wrote, ref_wrote)
    assert np.array_equal(got[wrote], ref[wrote])
    assert (wide[:, ix.max_context:].contiguous().cpu().view(torch.int32) == 0x7FC0FFEE).all()


# ------------------------------------------------- cancelling dot products


@pytest.mark.parametrize("next_n", [1, 4])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("one_hot", [True, False], ids=["one_hot", "dominant"])
def test_cancelling_dot_product_fp8(next_n, dtype, one_hot):
    """One dominant head whose q.k is a +-2^16 cancelling pair in one block of 8
    head_dim values plus a tail of products 2^-18 .. 2^-14 of the pair's (the
    whole logit).  gfx950's FP8 matrix instructions truncate every product
    below 2^-13 of its 8-value run's largest, which here drops the tail's part
    in the pair's run (about a fifth of the logit); the f16 products keep it."""
    inp = fixtures_util.cancelling_mqa_inputs("fp8", next_n, 300 + next_n, one_hot=one_hot,
                                              out_dtype=dtype)
    say("cancelling fp8 N=%d %s %s" % (next_n, dtype, "one-hot" if one_hot else "dominant"))
    dm = DevMqa(inp)
    r = check_dense(dm, dm.run(), "cancelling fp8 N=%d %s" % (next_n, dtype))
    say("  max err/tol %.3g" % r)


@pytest.mark.parametrize("next_n", [1, 2, 4])
def test_cancelling_dot_product_fp8_bit_exact(next_n):
    """The same class with one-hot power-of-two weights and power-of-two s_p:
    the exact result is representable in fp32 (the pair cancels inside one
    product of 8 values, the tail's partial sums are exact), so fp32 output
    must equal the oracle bit for bit, and bf16 output must equal its round to
    nearest even."""
    inp = fixtures_util.cancelling_mqa_inputs("fp8", next_n, 320 + next_n, pow2=True)
    ref, _, written = oracle.mqa_logits_for(inp)
    say("cancelling fp8 bit-exact N=%d, %d cells" % (next_n, int(written.sum())))
    dm = DevMqa(inp)
    got, wrote = host_out(dm.run(dtype=torch.float32))
    assert np.array_equal(wrote, written)
    assert np.array_equal(got[written], ref[written])
    gotb, wroteb = host_out(dm.run(dtype=torch.bfloat16))
    assert np.array_equal(wroteb, written)
    refb = torch.from_numpy(ref[written]).float().bfloat16().double().numpy()
    assert np.array_equal(gotb[written], refb)


@pytest.mark.parametrize("next_n", [1, 4])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("one_hot", [True, False], ids=["one_hot", "dominant"])
def test_cancelling_dot_product_mxfp4(next_n, dtype, one_hot):
    """MXFP4: a cancelling (6, 6) x (6, -6) pair with small products beside it
    in block 0, and the rest of the logit in a block whose e8m0 scale sits 2^14
    below the others.  The scaled FP4 products are exact and blocks add at fp32
    precision, so this holds without widening."""
    inp = fixtures_util.cancelling_mqa_inputs("mxfp4", next_n, 340 + next_n, one_hot=one_hot,
                                              out_dtype=dtype)
    say("cancelling mxfp4 N=%d %s %s" % (next_n, dtype, "one-hot" if one_hot else "dominant"))
    dm = DevMqa(inp)
    r = check_dense(dm, dm.run(), "cancelling mxfp4 N=%d %s" % (next_n, dtype))
    say("  max err/tol %.3g" % r)


def nvfp4_extreme_scale_inputs():
    """The indexer_nvfp4 workload with every query row reduced to one block of
    16 values (row r keeps block r mod 8, the rest of its codes zero) and the
    e4m3 scales of both sides drawn from the format's extremes: the smallest
    subnormal 2^-9, the largest subnormal 7 * 2^-9, the smallest normal 2^-6,
    1, the largest finite 448, and negatives.  Each score is then one scale
    product times a sum of 16 e2m1 products (a multiple of 1/4 of magnitude at
    most 576), exactly representable in fp32, so the kernel's f16 operands
    (e2m1 value times scale: 2^-10 .. 2688 in magnitude) and fp32 sums must
    reproduce the oracle bit for bit."""
    ix = copy.copy(synth.make_config("indexer_nvfp4"))
    ext = np.array([0x01, 0x07, 0x08, 0x38, 0x7E, 0x81, 0xFE, 0x3F], dtype=np.uint8)
    q = ix.query.copy()
    for r in range(ix.rows):
        keep = r % 8
        q[r, :8 * keep] = 0
        q[r, 8 * keep + 8:] = 0
    ix.query = q
    ix.query_scales = ext[(np.arange(ix.rows)[:, None] + np.arange(8)[None, :]) % 8].astype(np.uint8)
    ks = ix.key_scales.copy()
    P = ks.shape[0]
    k = np.arange(64)[None, :, None]
    j = np.arange(8)[None, None, :]
    p = np.arange(P)[:, None, None]
    ks[:, :512] = ext[(3 * k + j + p) % 8].reshape(P, 512)
    ix.key_scales = ks
    return ix


def test_indexer_nvfp4_extreme_scales_bit_exact():
    ix = nvfp4_extreme_scale_inputs()
    ref, _, written = oracle.indexer_scores_for(ix)
    exp = ref[written]
    assert np.array_equal(exp.astype(np.float32).astype(np.float64), exp)  # the premise
    assert np.abs(exp).max() > 1e6 and np.abs(exp[exp != 0]).min() < 1e-5
    say("nvfp4 indexer extreme scales: %d cells" % int(written.sum()))
    got, wrote = host_out(DevIndexer(ix).run())
    assert np.array_equal(wrote, written)
    assert np.array_equal(got[written], exp.astype(np.float32))
