"""Pins of the block-max proxy score oracle (FlashInfer
"flashinfer.msa_ops.msa_proxy_score_fp4": description, parameters, "Returns";
readings where the page defers to an absent one are in oracle.c).

Hand-worked cases (tests/golden/proxy_score_cases.json) fix the arithmetic,
the GQA head mapping, causal visibility, the page and scale-row addressing
and reduce_heads; the identities below tie the rest to the one-head NVFP4
indexer oracle (pinned by its own hand-worked cases) and to properties that
hold for any input."""
import copy

import numpy as np
import pytest

import oracle
import synth
from fixtures_util import expected_value, load_golden, proxy_from_case

CASES = load_golden("proxy_score_cases.json")["cases"]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c["name"])
def test_proxy_golden(case):
    ref, amag = oracle.proxy_score_fp4_for(proxy_from_case(case))
    for e in case["expected"]:
        assert ref[e["h"], e["t"], e["i"]] == expected_value(e["value"]), e


def _flat_one_head(L, seed, qgs, kgs):
    inp = synth.make_proxy_inputs([1], [L], num_qo_heads=1, num_kv_heads=1, paged=False,
                                  causal=False, seed=seed)
    inp.q_global_scale, inp.k_global_scale = qgs, kgs
    return inp


def _indexer_scores_of(inp):
    """The same query row and keys as one-head NVFP4 indexer inputs (pages of
    64 keys, identity block table), scored by the indexer oracle."""
    L = int(inp.cu_k[-1])
    P = (L + 63) // 64
    kc = np.zeros((P * 64, 64), np.uint8)
    ks = np.zeros((P * 64, 8), np.uint8)
    kc[:L] = inp.k[:, 0, :]
    ks[:L] = inp.k_scale
    ref, _, written = oracle.indexer_scores_nvfp4(
        inp.q[:, 0, :], inp.q_scale, kc.reshape(P, -1), 64 * 64, ks.reshape(P, -1), 64 * 8,
        np.arange(P, dtype=np.int32)[None, :], np.array([L], np.int32), np.array([0], np.int32),
        np.array([0, 1], np.int32), P * 64)
    assert written[0, :L].all()
    return ref[0, :L]


@pytest.mark.parametrize("qgs,kgs", [(0.75, 2.0), (-0.5, 0.25)])
def test_non_causal_one_head_is_block_max_of_indexer_scores(qgs, kgs):
    """One head, not causal: block t is g times the max (g > 0) or the min
    (g < 0) of the indexer scores of keys 128t .. 128t+127 -- the global
    scales multiply before the max."""
    L = 300
    inp = _flat_one_head(L, 11, qgs, kgs)
    ref, _ = oracle.proxy_score_fp4_for(inp)
    s = _indexer_scores_of(inp)
    g = qgs * kgs
    for t in range(inp.max_k_tiles):
        blk = s[128 * t:min(128 * t + 128, L)]
        want = g * (blk.max() if g > 0 else blk.min())
        assert ref[0, t, 0] == want


def _random(paged=True, causal=True, seed=3, reduce_heads=False, q_offset=None, q_lens=None,
            k_lens=None):
    q_lens = [1, 3, 0, 4, 2] if q_lens is None else q_lens
    k_lens = [130, 0, 50, 400, 257] if k_lens is None else k_lens
    return synth.make_proxy_inputs(q_lens, k_lens, num_qo_heads=6, num_kv_heads=3, paged=paged,
                                   causal=causal, q_offset=q_offset, reduce_heads=reduce_heads,
                                   seed=seed, max_k_tiles=5, extra_pages=2)


def test_reduce_heads_is_max_over_heads():
    inp = _random()
    per_head, _ = oracle.proxy_score_fp4_for(inp)
    red = copy.copy(inp)
    red.reduce_heads = True
    got, _ = oracle.proxy_score_fp4_for(red)
    assert got.shape == (1,) + per_head.shape[1:]
    assert np.array_equal(got[0], per_head.max(axis=0))


def _as_flat(inp):
    """The paged keys of inp rewritten as flat keys (same logical keys)."""
    L = inp.key_lengths()
    cu_k = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    Hkv = inp.num_kv_heads
    k = np.zeros((int(cu_k[-1]), Hkv, 64), np.uint8)
    ks = np.zeros((int(cu_k[-1]) * Hkv, 8), np.uint8)
    pages = inp.k[:, :Hkv * 128 * 64].reshape(-1, Hkv, 128, 64)
    for r in range(inp.batch):
        for kk in range(int(L[r])):
            page, tok = inp.page_table[r, kk // 128], kk % 128
            k[cu_k[r] + kk] = pages[page, :, tok]
            for j in range(Hkv):
                ks[(cu_k[r] + kk) * Hkv + j] = inp.k_scale[(page * Hkv + j) * 128 + tok]
    flat = copy.copy(inp)
    flat.paged, flat.k, flat.k_scale, flat.cu_k = False, k, ks, cu_k
    flat.page_table = flat.seqused_k = None
    flat.page_stride = 0
    return flat


def test_paged_equals_flat():
    inp = _random()
    a, _ = oracle.proxy_score_fp4_for(inp)
    b, _ = oracle.proxy_score_fp4_for(_as_flat(inp))
    assert np.array_equal(a, b)


def test_default_offset_is_keys_minus_queries():
    inp = _random()
    a, _ = oracle.proxy_score_fp4_for(inp)
    explicit = copy.copy(inp)
    explicit.q_offset = (inp.key_lengths() - np.diff(inp.cu_q)).astype(np.int32)
    b, _ = oracle.proxy_score_fp4_for(explicit)
    assert np.array_equal(a, b)


def test_causal_with_far_offset_equals_non_causal():
    inp = _random(q_offset=[10 ** 6] * 5)
    a, _ = oracle.proxy_score_fp4_for(inp)
    nc = copy.copy(inp)
    nc.causal = False
    b, _ = oracle.proxy_score_fp4_for(nc)
    assert np.array_equal(a, b)


def test_causal_masks_exactly_the_later_keys():
    """Token p of a request with offset o: block t is -inf iff 128t > o + p
    (or past the keys), and equals the non-causal value iff the whole block
    is visible."""
    inp = _random(q_offset=[0, 0, 0, 130, 200])
    ref, _ = oracle.proxy_score_fp4_for(inp)
    nc = copy.copy(inp)
    nc.causal = False
    full, _ = oracle.proxy_score_fp4_for(nc)
    L = inp.key_lengths()
    for r in range(inp.batch):
        for p in range(int(inp.cu_q[r + 1] - inp.cu_q[r])):
            i = inp.cu_q[r] + p
            lim = min(int(inp.q_offset[r]) + p, int(L[r]) - 1)
            for t in range(inp.max_k_tiles):
                if 128 * t > lim:
                    assert np.all(ref[:, t, i] == -np.inf)
                elif 128 * t + 127 <= lim:
                    assert np.array_equal(ref[:, t, i], full[:, t, i])
                else:
                    assert np.all(ref[:, t, i] <= full[:, t, i])


def test_global_scale_power_of_two_is_exact():
    inp = _random()
    a, _ = oracle.proxy_score_fp4_for(inp)
    b_in = copy.copy(inp)
    b_in.q_global_scale = inp.q_global_scale * 4.0
    b, _ = oracle.proxy_score_fp4_for(b_in)
    assert np.array_equal(b, 4.0 * a)


def test_tokens_outside_requests_and_empty_requests_are_minus_inf():
    inp = _random(q_lens=[2, 0, 1], k_lens=[0, 300, 20])
    ref, _ = oracle.proxy_score_fp4_for(inp)
    assert np.all(ref[:, :, 0:2] == -np.inf)  # request 0 has no keys
    assert np.all(np.isfinite(ref[:, 0, 2])) and np.all(ref[:, 1:, 2] == -np.inf)


def test_out_of_range_page_id_gives_nan_for_that_block_only():
    inp = _random()
    bad = copy.copy(inp)
    bad.page_table = inp.page_table.copy()
    bad.page_table[3, 1] = inp.num_pages + 5
    bad.page_table[4, 0] = -2
    a, _ = oracle.proxy_score_fp4_for(inp)
    b, _ = oracle.proxy_score_fp4_for(bad)
    poison = np.zeros(a.shape, bool)
    poison[:, 1, inp.cu_q[3]:inp.cu_q[4]] = True
    poison[:, 0, inp.cu_q[4]:inp.cu_q[5]] = True
    poison &= a != -np.inf
    assert poison.any() and np.isnan(b[poison]).all()
    assert np.array_equal(a[~poison], b[~poison])


def test_points_equal_dense():
    inp = _random(reduce_heads=False)
    ref, amag = oracle.proxy_score_fp4_for(inp)
    rng = np.random.default_rng(0)
    n = 400
    hs = rng.integers(0, ref.shape[0], n)
    ts = rng.integers(0, ref.shape[1], n)
    is_ = rng.integers(0, ref.shape[2], n)
    got, gm = oracle.proxy_score_fp4_points_for(inp, hs, ts, is_)
    assert np.array_equal(got, ref[hs, ts, is_])
    assert np.array_equal(gm, amag[hs, ts, is_])


def test_magnitude_bounds_the_value():
    inp = _random()
    ref, amag = oracle.proxy_score_fp4_for(inp)
    fin = np.isfinite(ref)
    assert np.all(np.abs(ref[fin]) <= amag[fin])
    assert np.all(amag[~fin] == 0)
