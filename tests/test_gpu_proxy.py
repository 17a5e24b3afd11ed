"""GPU parity of the block-max proxy score (FlashInfer
"flashinfer.msa_ops.msa_proxy_score_fp4") against the oracle, through the C ABI.

Every output is compared: -inf and NaN positions exactly, finite values within
|gpu - ref| <= 1e-5 * A, A = the largest |g| * sum_d |q_d k_d| over the block's
visible keys (products are exact in f16; 128 fp32 additions and two fp32
roundings of the scale add at most ~7.7e-6 * A).  Dyadic inputs bit-exactly."""
import copy

import numpy as np
import pytest
import torch

import oracle
import synth
from fixtures_util import expected_value, load_golden, proxy_from_case
from gpu_util import DEV, pm, say

pytestmark = pytest.mark.gpu

REL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    pm().init()
    yield
    torch.cuda.synchronize()


class DevProxy:
    """Device copies of a synth.ProxyInputs."""

    def __init__(self, inp):
        self.inp = inp
        t = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
        self.q = t(inp.q)
        self.qs = t(inp.q_scale)
        self.ks = t(inp.k_scale)
        self.cu_q = t(inp.cu_q)
        self.cu_k = t(inp.cu_k)
        self.pt = t(inp.page_table)
        self.su = t(inp.seqused_k)
        self.qo = t(inp.q_offset)
        if inp.paged:
            raw = t(inp.k)
            H = inp.num_kv_heads
            self.k = raw.as_strided((raw.shape[0], H, 128, 64), (raw.shape[1], 128 * 64, 64, 1))
        else:
            self.k = t(inp.k)

    def run(self, output=None, max_seqlen_q=None):
        inp = self.inp
        return pm().msa_proxy_score_fp4(
            self.q, self.k, self.qs, self.ks, inp.q_global_scale, inp.k_global_scale, self.cu_q,
            self.cu_k, page_table=self.pt, seqused_k=self.su, causal=inp.causal,
            max_seqlen_q=max_seqlen_q, max_k_tiles=inp.max_k_tiles, output=output,
            reduce_heads=inp.reduce_heads, q_offset=self.qo)


def host(out):
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def check(got, ref, amag, what=""):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    ninf_g, ninf_r = got == -np.inf, ref == -np.inf
    assert np.array_equal(ninf_g, ninf_r), "%s: -inf cells differ (%d vs %d)" % (
        what, int(ninf_g.sum()), int(ninf_r.sum()))
    assert np.array_equal(np.isnan(got), np.isnan(ref)), "%s: NaN cells differ" % what
    fin = np.isfinite(ref)
    err = np.abs(got[fin] - ref[fin])
    lim = REL * amag[fin] + 1e-30
    bad = ~(err <= lim)
    if bad.any():
        i = int(np.argmax(np.where(bad, err / lim, 0)))
        raise AssertionError("%s: %d of %d values out of tolerance; worst got %r ref %r A %r" % (
            what, int(bad.sum()), bad.size, got[fin][i], ref[fin][i], amag[fin][i]))
    return float(np.max(err / lim)) if err.size else 0.0


@pytest.mark.parametrize("case", load_golden("proxy_score_cases.json")["cases"],
                         ids=lambda c: c["name"])
def test_golden_bit_exact(case):
    inp = proxy_from_case(case)
    say("proxy golden %s" % case["name"])
    got = host(DevProxy(inp).run())
    ref, _ = oracle.proxy_score_fp4_for(inp)
    for e in case["expected"]:
        assert got[e["h"], e["t"], e["i"]] == expected_value(e["value"]), e
    assert np.array_equal(got, ref)


SHAPES = [  # (Hq, Hkv): group 1, 4, 8, 16, 48, 64
    (4, 4), (8, 2), (64, 8), (32, 2), (48, 1), (64, 1)]


@pytest.mark.parametrize("paged", [True, False], ids=["paged", "flat"])
@pytest.mark.parametrize("hq,hkv", SHAPES, ids=["%dx%d" % s for s in SHAPES])
@pytest.mark.parametrize("reduce_heads", [False, True], ids=["per_head", "reduce"])
def test_ragged_causal(paged, hq, hkv, reduce_heads):
    """Requests with 0, 1, 3, 4 and 9 query tokens and 0 .. 700 keys (block
    boundaries, a partly filled last block), causal with the default offset;
    every output against the dense oracle."""
    q_lens = [1, 3, 0, 4, 9, 1, 2]
    k_lens = [130, 0, 50, 400, 700, 128, 1]
    inp = synth.make_proxy_inputs(q_lens, k_lens, num_qo_heads=hq, num_kv_heads=hkv,
                                  paged=paged, causal=True, reduce_heads=reduce_heads, seed=40,
                                  max_k_tiles=7, extra_pages=3)
    what = "proxy %s %dx%d %s" % ("paged" if paged else "flat", hq, hkv,
                                  "reduce" if reduce_heads else "per-head")
    say(what)
    ref, amag = oracle.proxy_score_fp4_for(inp)
    check(host(DevProxy(inp).run()), ref, amag, what)


@pytest.mark.parametrize("variant", ["non_causal", "explicit_offsets", "negative_scale",
                                     "truncated_tiles", "tokens_outside", "long_q"])
def test_options(variant):
    kw = dict(num_qo_heads=16, num_kv_heads=2, paged=True, causal=True, seed=50,
              max_k_tiles=6, extra_pages=2)
    q_lens, k_lens = [2, 1, 5, 3], [300, 129, 640, 0]
    if variant == "non_causal":
        kw["causal"] = False
    elif variant == "explicit_offsets":
        kw["q_offset"] = [0, -5, 200, 10]
    elif variant == "truncated_tiles":
        kw["max_k_tiles"] = 2
    elif variant == "long_q":
        q_lens, k_lens = [40, 70], [300, 900]
        kw["max_k_tiles"] = 8
    inp = synth.make_proxy_inputs(q_lens, k_lens, **kw)
    if variant == "negative_scale":
        inp.q_global_scale = -inp.q_global_scale * 3.0
    if variant == "tokens_outside":
        # two extra query rows past cu_seqlens_q[-1]: they belong to no request
        inp.q = np.concatenate([inp.q, inp.q[:2]], axis=0)
        inp.q_scale = np.concatenate([inp.q_scale, inp.q_scale[:2 * inp.num_qo_heads]], axis=0)
    say("proxy option %s" % variant)
    ref, amag = oracle.proxy_score_fp4_for(inp)
    check(host(DevProxy(inp).run()), ref, amag, variant)


@pytest.mark.parametrize("reduce_heads", [False, True], ids=["per_head", "reduce"])
def test_dyadic_bit_exact(reduce_heads):
    """Power-of-two scales and e2m1 values: every partial sum is exact in
    fp32, so the result equals the oracle bit for bit."""
    inp = synth.make_proxy_inputs([1, 4, 2], [500, 260, 131], num_qo_heads=16, num_kv_heads=4,
                                  causal=True, reduce_heads=reduce_heads, seed=60, max_k_tiles=5)
    rng = np.random.default_rng(61)
    pow2 = np.array([0x30, 0x38, 0x40, 0x28], np.uint8)  # 0.5, 1, 2, 0.25 in e4m3
    inp.q_scale = rng.choice(pow2, inp.q_scale.shape)
    inp.k_scale = rng.choice(pow2, inp.k_scale.shape)
    inp.q_global_scale, inp.k_global_scale = 0.5, 4.0
    say("proxy dyadic %s" % reduce_heads)
    ref, _ = oracle.proxy_score_fp4_for(inp)
    got = host(DevProxy(inp).run())
    assert np.array_equal(got, ref)


def test_out_of_range_page_is_nan_there_only():
    inp = synth.make_proxy_inputs([2, 1, 3], [400, 300, 500], num_qo_heads=8, num_kv_heads=2,
                                  seed=70, max_k_tiles=4)
    bad = copy.copy(inp)
    bad.page_table = inp.page_table.copy()
    bad.page_table[0, 1] = inp.num_pages + 9
    bad.page_table[2, 3] = -3
    say("proxy bad page ids")
    ref, amag = oracle.proxy_score_fp4_for(bad)
    assert np.isnan(ref).any()
    check(host(DevProxy(bad).run()), ref, amag, "bad pages")


def test_flat_keys_outside_buffer_are_nan():
    inp = synth.make_proxy_inputs([1, 2], [200, 100], num_qo_heads=4, num_kv_heads=1,
                                  paged=False, seed=71, max_k_tiles=2)
    bad = copy.copy(inp)
    bad.cu_k = inp.cu_k.copy()
    bad.cu_k[2] = inp.cu_k[2] + 50  # request 1 claims 50 keys past the end
    dp = DevProxy(bad)
    got = host(dp.run())
    # request 1 (tokens 1, 2): every visible block NaN; request 0 unchanged
    ref0, amag0 = oracle.proxy_score_fp4_for(inp)
    assert np.isnan(got[:, 0, 1:3]).all()
    check(got[:, :, :1], ref0[:, :, :1], amag0[:, :, :1], "request 0")


def test_repeat_bit_identical_and_prepared_call():
    inp = synth.make_proxy_inputs([1, 4, 2, 1], [900, 300, 0, 77], num_qo_heads=64,
                                  num_kv_heads=8, seed=80, max_k_tiles=8)
    dp = DevProxy(inp)
    a = host(dp.run())
    b = host(dp.run())
    assert np.array_equal(a.view(np.uint64), b.view(np.uint64))
    out = torch.empty_like(torch.from_numpy(a.astype(np.float32))).to(DEV)
    call = pm().prepare_msa_proxy_score_fp4(
        dp.q, dp.k, dp.qs, dp.ks, inp.q_global_scale, inp.k_global_scale, dp.cu_q,
        page_table=dp.pt, seqused_k=dp.su, max_k_tiles=inp.max_k_tiles, output=out)
    for _ in range(2):
        c = host(call())
        assert np.array_equal(a.view(np.uint64), c.view(np.uint64))


@pytest.mark.parametrize("name", ["proxy_decode", "proxy_verify"])
def test_full_size_config(name):
    """64 requests, 16K-128K keys, 64 query heads over 8 KV heads: sampled
    cells against the oracle (every head of the first and last block of
    every request, random cells), the -inf region exactly."""
    inp = synth.make_config(name)
    say("%s: B=%d total_q=%d pages=%d" % (name, inp.batch, inp.total_q, inp.num_pages))
    got = host(DevProxy(inp).run(max_seqlen_q=int(np.max(np.diff(inp.cu_q)))))
    rng = np.random.default_rng(5)
    hs, ts, is_ = [], [], []
    L = inp.key_lengths()
    for r in range(inp.batch):
        T = int(min((L[r] + 127) // 128, inp.max_k_tiles))
        for i in range(int(inp.cu_q[r]), int(inp.cu_q[r + 1])):
            for t in {0, max(T - 1, 0), min(T, inp.max_k_tiles - 1)}:
                h = int(rng.integers(0, inp.out_heads))
                hs.append(h), ts.append(t), is_.append(i)
    n = 400
    hs += rng.integers(0, inp.out_heads, n).tolist()
    ts += rng.integers(0, inp.max_k_tiles, n).tolist()
    is_ += rng.integers(0, inp.total_q, n).tolist()
    ref, amag = oracle.proxy_score_fp4_points_for(inp, hs, ts, is_)
    r = check(got[hs, ts, is_], ref, amag, name)
    # the -inf region exactly: token p of a request (default offset Lk - Lq)
    # sees keys up to min(Lk - 1, Lk - Lq + p), so block t is -inf iff it
    # starts past that key
    lq = np.diff(inp.cu_q)
    tok_L = np.repeat(L, lq)
    tok_p = np.concatenate([np.arange(n) for n in lq])
    lim = np.minimum(tok_L - 1, tok_L - np.repeat(lq, lq) + tok_p)
    tok_T = np.where(lim < 0, 0, np.minimum(lim // 128 + 1, inp.max_k_tiles))
    expect_ninf = np.arange(inp.max_k_tiles)[None, :, None] >= tok_T[None, None, :]
    assert np.array_equal(got == -np.inf, np.broadcast_to(expect_ninf, got.shape))
    say("%s max err/tol %.3g over %d sampled cells" % (name, r, len(hs)))
