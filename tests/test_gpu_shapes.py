"""GPU parity for the FP8 shapes beyond 64 heads x head_dim 128 and for next_n
above 4, through the C ABI, against the CPU oracle.

Other head counts and head_dims run the general FP8 kernel; next_n 5..8 runs
the slot passes (of the 64-head kernels, or of the general kernel).  Written
sets are compared exactly (sentinel-filled outputs); values within
|gpu - ref| <= 2e-3*A + 1e-5 (fp32 out) or 1e-2*A + 1e-5 (bf16 out), with
A = s_p * sum_h |w| * relu(q.k); exact-arithmetic inputs bit-exactly."""
import copy

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (DEV, DevMqa, check_dense, check_sampled, check_values, host_out, pm, say,
                      tol_for)

pytestmark = pytest.mark.gpu

RAGGED = [0, 1, 63, 64, 65, 200, 700, 1000, -5, 3000, 129, 2048]

# (num_heads, head_dim, next_n) for the general kernel: head counts off the
# 32-head padding, head_dims off the 128-byte planes, one and two planes, and
# next_n that needs more than one slot pass
GENERAL = [(1, 16, 1), (5, 48, 6), (32, 128, 2), (33, 144, 3), (64, 64, 4), (128, 256, 2),
           (16, 128, 8), (96, 192, 5), (128, 128, 3), (64, 256, 1), (64, 112, 2), (20, 80, 7)]


def _id(shape):
    return "H%d_D%d_N%d" % shape


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    pm().init()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("shape", GENERAL, ids=_id)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_general_shape_ragged(shape, dtype):
    H, D, N = shape
    inp = synth.make_mqa_inputs(RAGGED, N, num_heads=H, head_dim=D, max_context=2048,
                                bt_width=40, seed=500 + H + D + N, w_std=0.5, out_dtype=dtype,
                                extra_pages=5)
    what = "general %s %s" % (_id(shape), dtype)
    say(what)
    dm = DevMqa(inp)
    r = check_dense(dm, dm.run(), what)
    say("%s max err/tol %.3g" % (what, r))


@pytest.mark.parametrize("variant", ["fp8", "mxfp4"])
@pytest.mark.parametrize("next_n", [5, 6, 7, 8])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_next_n_above_4_ragged(variant, next_n, dtype):
    """64 heads x 128: the 64-head kernels in passes of up to 4 slots."""
    inp = synth.make_mqa_inputs(RAGGED, next_n, variant=variant, max_context=2048, bt_width=40,
                                seed=600 + next_n, w_std=0.5, out_dtype=dtype, extra_pages=5)
    what = "%s N=%d %s" % (variant, next_n, dtype)
    say(what)
    dm = DevMqa(inp)
    check_dense(dm, dm.run(), what)


def _exact_inputs(H, D, N, seed, grid=(0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0)):
    """Values on a coarse dyadic grid: before s_p every partial sum is a
    multiple of 2^-3 below 2^18, so exact in fp32 in any order; s_p = 2^k."""
    rng = np.random.default_rng(seed)
    inp = synth.make_mqa_inputs([300, 64, 1, 129], N, num_heads=H, head_dim=D, max_context=320,
                                bt_width=5, seed=seed)
    grid = np.array(grid, dtype=np.float32)
    inp.q = synth.encode_e4m3(rng.choice(grid, (inp.batch, N, H, D)).astype(np.float32))
    kf = rng.choice(grid, (inp.num_pages, 64, D)).astype(np.float32)
    inp.kv[:, : 64 * D] = synth.encode_e4m3(kf).reshape(inp.num_pages, -1)
    sp = np.ldexp(1.0, rng.integers(-4, 4, (inp.num_pages, 64))).astype(np.float32)
    inp.kv[:, 64 * D: 64 * D + 256] = sp.view(np.uint8)
    inp.weights[:] = rng.choice(np.array([0.5, -0.5, 1.0, -1.0, 2.0, -2.0], np.float32),
                                inp.weights.shape)
    return inp


@pytest.mark.parametrize("shape", [(5, 48, 6), (128, 256, 2), (33, 144, 3), (64, 128, 8),
                                   (64, 128, 5), (1, 16, 1)], ids=_id)
def test_exact_arithmetic_bit_exact(shape):
    inp = _exact_inputs(*shape, seed=700 + sum(shape))
    ref, _, written = oracle.mqa_logits_for(inp)
    dm = DevMqa(inp)
    got, wrote = host_out(dm.run(dtype=torch.float32))
    assert np.array_equal(wrote, written)
    assert np.array_equal(got[written], ref[written])
    if shape[:2] == (64, 128):
        # the 64-head kernels sum the heads of a bf16 output in bf16 products:
        # bit-exact where every rectified score is exact in bf16 (q, k in {0, +-1})
        inp = _exact_inputs(*shape, seed=750 + sum(shape), grid=(0.0, 1.0, -1.0))
        ref, _, written = oracle.mqa_logits_for(inp)
        dm = DevMqa(inp)
    gotb, _ = host_out(dm.run(dtype=torch.bfloat16))
    refb = torch.from_numpy(ref[written]).float().bfloat16().double().numpy()
    assert np.array_equal(gotb[written], refb)


def _mid(H, D, N, seed, variant="fp8"):
    lens = np.random.default_rng(seed).integers(0, 3000, 23)
    lens[3] = 0
    return synth.make_mqa_inputs(lens, N, variant=variant, num_heads=H, head_dim=D,
                                 max_context=3072, bt_width=48, seed=seed)


@pytest.mark.parametrize("shape", [(33, 144, 3), (64, 128, 6), (128, 256, 5)], ids=_id)
def test_schedule_any_unit_count_bit_identical(shape):
    """A schedule (any unit count, the same next_n) gives the in-call result
    bit for bit, for every pass of a call."""
    inp = _mid(*shape, seed=710 + shape[2])
    dm = DevMqa(inp)
    base, wb = host_out(dm.run())
    for U in (1, 7, 256, 5000, 0):
        sched = pm().mqa_logits_schedule(dm.sl, inp.next_n, 0, max_context=inp.max_context,
                                         num_units=U)
        got, wg = host_out(dm.run(schedule=sched))
        assert np.array_equal(wb, wg), U
        assert np.array_equal(got.view(np.uint64), base.view(np.uint64)), U
    check_dense(dm, dm.run(), "mid %s" % _id(shape))


@pytest.mark.parametrize("shape", [(33, 144, 3), (64, 128, 7)], ids=_id)
def test_out_of_range_page_id_gives_nan_for_that_page_only(shape):
    inp = _mid(*shape, seed=720 + shape[2])
    tiles = np.where(inp.seq_lens > 0, (inp.seq_lens + 63) // 64, 0)
    b1, b2 = [int(b) for b in np.nonzero(tiles >= 3)[0][:2]]
    bad = copy.copy(inp)
    bad.block_table = inp.block_table.copy()
    bad.block_table[b1, 1] = inp.num_pages + 7
    bad.block_table[b2, 2] = -5
    out = DevMqa(bad).run()
    got, wrote = host_out(out)
    ref, amag, written = oracle.mqa_logits_for(inp)
    assert np.array_equal(wrote, written)
    N = inp.next_n
    poison = np.zeros_like(written)
    poison[b1 * N:(b1 + 1) * N, 64:128] = True
    poison[b2 * N:(b2 + 1) * N, 128:192] = True
    assert np.array_equal(poison & written, poison)
    assert np.isnan(got[poison]).all()
    ok = written & ~poison
    check_values(got[ok], ref[ok], amag[ok], tol_for(out.dtype), "valid pages")


def test_poisoned_unread_data_never_reaches_outputs():
    """Unowned pages hold NaN codes and NaN scales; bytes of a page past its
    64 x head_dim keys and scales (a wider page stride) hold NaN codes too."""
    H, D = 40, 80
    stride = 64 * (D + 4) + 16 * 9
    inp = synth.make_mqa_inputs([500, 0, 64, 1300], 3, num_heads=H, head_dim=D,
                                max_context=1536, bt_width=24, seed=730, extra_pages=6,
                                page_stride=stride)
    inp.kv[:, 64 * (D + 4):] = 0x7F
    used = set(inp.block_table[inp.block_table >= 0].tolist())
    for p in range(inp.num_pages):
        if p not in used:
            inp.kv[p, :] = 0x7F
            inp.kv[p, 64 * D: 64 * D + 256] = np.full(64, np.nan, np.float32).view(np.uint8)
    dm = DevMqa(inp)
    got, wrote = host_out(dm.run())
    assert not np.isnan(got[wrote]).any()
    check_dense(dm, dm.run(), "poisoned general")


def test_largest_shape_and_batch():
    """128 heads x 256 and B = 8192: the most LDS the general kernel takes
    (two-plane ring, a 32 KB query slice, a full request prefix); complete
    written set and sampled values, in-call split and schedule."""
    rng = np.random.default_rng(740)
    lens = rng.integers(0, 300, 8192)
    lens[::97] = 0
    inp = synth.make_mqa_inputs(lens, 2, num_heads=128, head_dim=256, max_context=320,
                                bt_width=5, seed=740)
    dm = DevMqa(inp)
    check_sampled(dm, dm.run(), np.random.default_rng(1), "in-call")
    sched = pm().mqa_logits_schedule(dm.sl, 2, 0, max_context=inp.max_context)
    check_sampled(dm, dm.run(schedule=sched), np.random.default_rng(2), "schedule")


@pytest.mark.parametrize("shape", [(96, 192, 3), (64, 128, 6)], ids=_id)
def test_graph_replay_general_and_passes(shape):
    """A call with several slot passes captured once with its schedule (96 x
    192: three launches of the general kernel, one slot each; 64 x 128, six
    slots: launches of 4 and 2 slots); replays with new inputs match the
    oracle."""
    H, D, N = shape

    def make(seed):
        lens = np.random.default_rng(seed).integers(0, 3000, 23)
        lens[seed % 23] = 0
        return synth.make_mqa_inputs(lens, N, num_heads=H, head_dim=D, max_context=3072,
                                     bt_width=48, seed=seed, full_table=True)

    inp = make(750)
    dm = DevMqa(inp)
    U = pm().num_units(N, 0)
    sched = torch.empty(pm().schedule_ints(U), dtype=torch.int32, device=DEV)
    out = dm.new_out()
    dm.run(out=out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pm().mqa_logits_schedule(dm.sl, N, 0, max_context=inp.max_context, num_units=U,
                                 out=sched)
        dm.run(out=out, schedule=sched)
    for rep in range(3):
        new = make(760 + rep)
        dm.sl.copy_(torch.from_numpy(new.seq_lens))
        dm.q.copy_(torch.from_numpy(new.q))
        dm.w.copy_(torch.from_numpy(new.weights))
        dm.kv.copy_(torch.from_numpy(new.kv))
        dm.bt.copy_(torch.from_numpy(new.block_table))
        out.copy_(dm.new_out())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        dm.inp = new
        check_dense(dm, out, "general replay %d" % rep)


@pytest.mark.parametrize("name", ["verify_fp8_n8", "verify_fp8_h32"])
def test_full_size_config(name):
    inp = synth.make_config(name)
    say("%s: B=%d N=%d H=%d D=%d pages=%d positions=%d" % (
        name, inp.batch, inp.next_n, inp.num_heads, inp.head_dim, inp.num_pages,
        inp.kv_positions()))
    dm = DevMqa(inp)
    r = check_sampled(dm, dm.run(), np.random.default_rng(8), name)
    say("%s max err/tol %.3g" % (name, r))
