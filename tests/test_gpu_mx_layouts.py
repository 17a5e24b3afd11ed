"""GPU parity of the MXFP4 scale layouts: one e8m0 code per 32 or per 16
values (sf_vec_size), key codes after all packed rows of a page or in each
token's record (is_kv_sf_interleaved), against the oracle through the C ABI.

Tolerances as in the other parity tests; exact-arithmetic inputs bit-exactly."""
import copy

import numpy as np
import pytest
import torch

import oracle
import synth
from fixtures_util import extent, load_golden, mqa_from_case
from gpu_util import (DevMqa, check_dense, check_sampled, check_values, host_out, pm, say,
                      tol_for)

pytestmark = pytest.mark.gpu

LAYOUTS = [(32, False), (16, False), (32, True), (16, True)]
NEW_LAYOUTS = LAYOUTS[1:]


def lid(layout):
    sfv, il = layout
    return "sf%d_%s" % (sfv, "records" if il else "trailing")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    pm().init()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("case", load_golden("mxfp4_layout_cases.json")["cases"],
                         ids=lambda c: c["name"])
def test_layout_golden_bit_exact(case):
    inp = mqa_from_case(case, "mxfp4")
    say("layout golden %s" % case["name"])
    E = extent(case["seq_len"], inp.max_context)
    for dtype in (torch.float32, torch.bfloat16):
        got, wrote = host_out(DevMqa(inp).run(dtype=dtype))
        assert wrote[0, :E].all() and not wrote[0, E:].any()
        for col, v in case["expected"].items():
            assert got[0, int(col)] == v, (case["name"], col, dtype, got[0, int(col)])


RAGGED = [0, 1, 63, 64, 65, 200, 700, 1000, -5, 3000, 129, 2048]


@pytest.mark.parametrize("layout", NEW_LAYOUTS, ids=lid)
@pytest.mark.parametrize("next_n", [1, 2, 3, 4, 6])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_batch(layout, next_n, dtype):
    """Empty, one-token, page-boundary, negative and over-long lengths; every
    kernel instance (next_n 1..4, and 6 as two launches); both outputs."""
    sfv, il = layout
    inp = synth.make_mqa_inputs(RAGGED, next_n, variant="mxfp4", max_context=2048, bt_width=40,
                                seed=500 + next_n, w_std=0.5, out_dtype=dtype, extra_pages=5,
                                sf_vec_size=sfv, kv_sf_interleaved=il)
    what = "ragged %s N=%d %s" % (lid(layout), next_n, dtype)
    say(what)
    dm = DevMqa(inp)
    check_dense(dm, dm.run(), what)


def _exact_inputs(layout, next_n, seed):
    """Values on a coarse dyadic grid with codes within 2^-2..2^2, so every
    partial sum is exact in fp32."""
    sfv, il = layout
    rng = np.random.default_rng(seed)
    inp = synth.make_mqa_inputs([300, 64, 1, 129], next_n, variant="mxfp4", max_context=320,
                                bt_width=5, seed=seed, sf_vec_size=sfv, kv_sf_interleaved=il)
    grid = np.array([0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0], dtype=np.float32)
    qf = rng.choice(grid, (inp.batch, next_n, 64, 128)).astype(np.float32)
    kf = rng.choice(grid, (inp.num_pages, 64, 128)).astype(np.float32)
    inp.q, _ = synth.quantize_mxfp4(qf, sfv)
    inp.q_sf = rng.integers(125, 130, (inp.batch, next_n, 64, 128 // sfv)).astype(np.uint8)
    packed, _ = synth.quantize_mxfp4(kf, sfv)
    codes = rng.integers(125, 130, (inp.num_pages, 64, 128 // sfv)).astype(np.uint8)
    pg = synth.mxfp4_page(packed, codes, il)
    inp.kv[:, :pg.shape[1]] = pg
    inp.weights[:] = rng.choice(np.array([0.5, -0.5, 1.0, -1.0, 2.0, -2.0], np.float32),
                                inp.weights.shape)
    return inp


@pytest.mark.parametrize("layout", LAYOUTS, ids=lid)
@pytest.mark.parametrize("next_n", [1, 2, 4])
def test_exact_arithmetic_bit_exact(layout, next_n):
    """fp32 output on dyadic values with per-block codes that differ: equal to
    the oracle bit for bit (the scaled FP4 products are exact, and so is every
    partial sum)."""
    inp = _exact_inputs(layout, next_n, 520 + next_n)
    say("exact %s N=%d" % (lid(layout), next_n))
    ref, _, written = oracle.mqa_logits_for(inp)
    got, wrote = host_out(DevMqa(inp).run(dtype=torch.float32))
    assert np.array_equal(wrote, written)
    assert np.array_equal(got[written], ref[written])


@pytest.mark.parametrize("sfv", [32, 16])
@pytest.mark.parametrize("next_n", [1, 3])
def test_records_equal_trailing_bit_for_bit(sfv, next_n):
    """The same keys and codes stored as token records or with the codes after
    all packed rows give bit-identical outputs (both outputs)."""
    a = synth.make_mqa_inputs([700, 65, 2048, 0, 1000], next_n, variant="mxfp4",
                              max_context=2048, bt_width=32, seed=540 + next_n, sf_vec_size=sfv)
    b = copy.copy(a)
    b.kv_sf_interleaved = True
    D = 128
    packed = a.kv[:, :64 * D // 2].reshape(-1, 64, D // 2)
    codes = a.kv[:, 64 * D // 2:64 * D // 2 + 64 * D // sfv].reshape(-1, 64, D // sfv)
    b.kv = np.zeros_like(a.kv)
    pg = synth.mxfp4_page(packed, codes, True)
    b.kv[:, :pg.shape[1]] = pg
    say("records vs trailing sf%d N=%d" % (sfv, next_n))
    for dtype in (torch.float32, torch.bfloat16):
        ga, wa = host_out(DevMqa(a).run(dtype=dtype))
        gb, wb = host_out(DevMqa(b).run(dtype=dtype))
        assert np.array_equal(wa, wb)
        assert np.array_equal(ga[wa].view(np.uint64), gb[wb].view(np.uint64))


@pytest.mark.parametrize("layout", NEW_LAYOUTS, ids=lid)
def test_schedule_bit_identical(layout):
    """A schedule built for the MXFP4 variant serves every scale layout: same
    bits as the in-call split."""
    sfv, il = layout
    lens = np.random.default_rng(550).integers(0, 3000, 23)
    lens[3] = 0
    inp = synth.make_mqa_inputs(lens, 2, variant="mxfp4", max_context=3072, bt_width=48,
                                seed=550, sf_vec_size=sfv, kv_sf_interleaved=il)
    dm = DevMqa(inp)
    say("schedule %s" % lid(layout))
    ref, _ = host_out(dm.run())
    for units in (0, 7, 1000):
        sched = pm().mqa_logits_schedule(dm.sl, 2, 1, max_context=inp.max_context,
                                         num_units=units)
        got, _ = host_out(dm.run(schedule=sched))
        assert np.array_equal(got.view(np.uint64), ref.view(np.uint64)), units


@pytest.mark.parametrize("layout", NEW_LAYOUTS, ids=lid)
def test_out_of_range_page_id_gives_nan_for_that_page_only(layout):
    sfv, il = layout
    lens = np.random.default_rng(560).integers(200, 3000, 9)
    inp = synth.make_mqa_inputs(lens, 2, variant="mxfp4", max_context=3072, bt_width=48,
                                seed=560, sf_vec_size=sfv, kv_sf_interleaved=il)
    bad = copy.copy(inp)
    bad.block_table = inp.block_table.copy()
    bad.block_table[1, 1] = inp.num_pages + 3
    bad.block_table[4, 2] = -1
    out = DevMqa(bad).run()
    got, wrote = host_out(out)
    ref, amag, written = oracle.mqa_logits_for(inp)
    assert np.array_equal(wrote, written)
    poison = np.zeros_like(written)
    poison[2:4, 64:128] = True
    poison[8:10, 128:192] = True
    assert np.isnan(got[poison]).all()
    ok = written & ~poison
    check_values(got[ok], ref[ok], amag[ok], tol_for(out.dtype), "valid pages " + lid(layout))


@pytest.mark.parametrize("name", ["mxfp4_sf16", "mxfp4_records", "mxfp4_sf16_records"])
def test_full_size_config(name):
    """The mxfp4 workload (B=64, next_n=2, 16K..128K tokens) in each other
    layout: complete written set, values at sampled cells."""
    inp = synth.make_config(name)
    say("%s: B=%d N=%d pages=%d" % (name, inp.batch, inp.next_n, inp.num_pages))
    dm = DevMqa(inp)
    r = check_sampled(dm, dm.run(), np.random.default_rng(17), name)
    say("%s max err/tol %.3g" % (name, r))
