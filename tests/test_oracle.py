"""Pins for the CPU oracle, against things other than the oracle itself:
library casts for the formats, hand-worked examples, identities of the
rectifier that reduce the method to a matrix product, scaling invariants and
the output-contract rules of the pages.  CPU only."""
import copy
import math

import numpy as np
import pytest

import oracle
import synth
from fixtures_util import (E2M1_TABLE, decode_keys, decode_queries, extent, flip_key_signs,
                           indexer_from_case, load_golden, mqa_from_case, np_bf16, np_e4m3,
                           np_e8m0)

# ------------------------------------------------------------------ formats


def test_e4m3_decoder_matches_torch_for_all_codes():
    """OCP E4M3FN: every one of the 256 codes against torch's float8_e4m3fn."""
    ref = np_e4m3(np.arange(256, dtype=np.uint8))
    for c in range(256):
        v = oracle.e4m3(c)
        if math.isnan(ref[c]):
            assert math.isnan(v), c
        else:
            assert v == ref[c] and math.copysign(1, v) == math.copysign(1, ref[c]), c
    assert oracle.e4m3(0x7E) == 448.0 and oracle.e4m3(0x01) == 2.0 ** -9


def test_e8m0_decoder_matches_torch_for_all_codes():
    ref = np_e8m0(np.arange(256, dtype=np.uint8))
    for c in range(255):
        assert oracle.e8m0(c) == ref[c] == math.ldexp(1.0, c - 127), c
    assert math.isnan(oracle.e8m0(255))


def test_e2m1_decoder_matches_format_table():
    for c in range(16):
        mag = E2M1_TABLE[c & 7]
        assert oracle.e2m1(c) == (-mag if c & 8 else mag), c


def test_bf16_decoder_matches_torch():
    bits = np.array([0, 0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F, 0xC2F7, 0x3E80], dtype=np.uint16)
    ref = np_bf16(bits)
    for b, r in zip(bits, ref):
        assert oracle.bf16(int(b)) == r


def test_mxfp4_quantiser_packs_even_element_low():
    x = np.zeros(32, dtype=np.float32)
    x[0], x[1], x[2] = 6.0, -0.5, 3.0  # amax 6 -> shared exponent 0, code 127
    packed, sf = synth.quantize_mxfp4(x)
    assert sf.tolist() == [127]
    assert packed[0] == (0x7 | (0x9 << 4))  # 6.0 low, -0.5 high
    assert packed[1] == 0x5  # 3.0 low, 0 high


# ------------------------------------------------------------ golden examples


@pytest.mark.parametrize("case", load_golden("fp8_logits_cases.json")["cases"],
                         ids=lambda c: c["name"])
def test_fp8_golden(case):
    inp = mqa_from_case(case, "fp8")
    ref, amag, written = oracle.mqa_logits_for(inp)
    E = extent(case["seq_len"], inp.max_context)
    assert written[0, :E].all() and not written[0, E:].any()
    for col, v in case["expected"].items():
        assert ref[0, int(col)] == v, (case["name"], col)


@pytest.mark.parametrize("case", load_golden("mxfp4_logits_cases.json")["cases"],
                         ids=lambda c: c["name"])
def test_mxfp4_golden(case):
    inp = mqa_from_case(case, "mxfp4")
    ref, _, _ = oracle.mqa_logits_for(inp)
    for col, v in case["expected"].items():
        assert ref[0, int(col)] == v, (case["name"], col)


@pytest.mark.parametrize("case", load_golden("indexer_cases.json")["cases"],
                         ids=lambda c: c["name"])
def test_indexer_golden(case):
    inp = indexer_from_case(case)
    ref, _, written = oracle.indexer_scores_for(inp)
    L = case["context_length"]
    assert written[:, :L].all() and not written[:, L:].any()
    for r, exp in enumerate(case["expected"]):
        for col, v in exp.items():
            if int(col) < L:
                assert ref[r, int(col)] == v


# ------------------------------------------------- identities of the rectifier


def _small(variant, seed, next_n=2, lens=(37, 0, 130, 64)):
    return synth.make_mqa_inputs(list(lens), next_n, variant=variant, max_context=192,
                                 bt_width=3, seed=seed, w_std=1.0)


def _weighted_query_dot(inp, mode):
    """Per written cell, via numpy matrix products on independently decoded data:
    mode 'lin': s_p * sum_h w_h (q_h . k)     (relu(x) - relu(-x) = x)
    mode 'abs': s_p * sum_h w_h |q_h . k|     (relu(x) + relu(-x) = |x|)"""
    Q = decode_queries(inp)
    keys = decode_keys(inp)
    out = np.full((inp.rows, inp.max_context), np.nan)
    for b in range(inp.batch):
        k, s = keys[b]
        for t in range(inp.next_n):
            r = b * inp.next_n + t
            S = Q[b, t] @ k.T  # [H, E]
            if mode == "abs":
                S = np.abs(S)
            out[r, : k.shape[0]] = s * (inp.weights[r].astype(np.float64) @ S)
    return out


@pytest.mark.parametrize("variant", ["fp8", "mxfp4"])
def test_rectifier_difference_is_linear(variant):
    """oracle(k) - oracle(-k) = s_p * (sum_h w_h q_h) . k, checked against a
    float64 matrix product: pins decoding, layouts, weights, s_p, paging and
    the sign conventions."""
    inp = _small(variant, 11)
    neg = flip_key_signs(inp)
    r1, a1, w1 = oracle.mqa_logits_for(inp)
    r2, _, w2 = oracle.mqa_logits_for(neg)
    assert np.array_equal(w1, w2)
    lin = _weighted_query_dot(inp, "lin")
    m = w1
    np.testing.assert_allclose((r1 - r2)[m], lin[m], rtol=1e-12, atol=1e-9 * np.max(a1))
    assert np.array_equal(np.isnan(lin), ~m)


@pytest.mark.parametrize("variant", ["fp8", "mxfp4"])
def test_rectifier_sum_is_absolute(variant):
    """oracle(k) + oracle(-k) = s_p * sum_h w_h |q_h . k|: holds only when the
    rectifier is applied per head before the weighted sum."""
    inp = _small(variant, 12)
    r1, a1, m = oracle.mqa_logits_for(inp)
    r2, _, _ = oracle.mqa_logits_for(flip_key_signs(inp))
    ab = _weighted_query_dot(inp, "abs")
    np.testing.assert_allclose((r1 + r2)[m], ab[m], rtol=1e-12, atol=1e-9 * np.max(a1))


def test_one_head_reduces_to_rectified_dot_product():
    inp = synth.make_mqa_inputs([100, 20], 1, num_heads=1, max_context=128, bt_width=2, seed=13)
    inp.weights[:] = 1.0
    ref, _, m = oracle.mqa_logits_for(inp)
    Q = decode_queries(inp)
    for b, (k, s) in enumerate(decode_keys(inp)):
        exp = s * np.maximum(Q[b, 0, 0] @ k.T, 0.0)
        assert np.array_equal(ref[b, : k.shape[0]], exp)


def test_magnitude_is_weighted_rectified_sum():
    inp = _small("fp8", 14)
    _, amag, m = oracle.mqa_logits_for(inp)
    Q, keys = decode_queries(inp), decode_keys(inp)
    for b, (k, s) in enumerate(keys):
        for t in range(inp.next_n):
            r = b * inp.next_n + t
            exp = s * (np.abs(inp.weights[r]).astype(np.float64) @ np.maximum(Q[b, t] @ k.T, 0))
            np.testing.assert_allclose(amag[r, : k.shape[0]], exp, rtol=1e-12)


# -------------------------------------------------------------- invariants


def test_sp_power_of_two_scaling_is_exact():
    """FP8 result = s_p x the unscaled sum: scaling every s_p by 2^j scales
    every logit by exactly 2^j."""
    inp = _small("fp8", 15)
    base, _, m = oracle.mqa_logits_for(inp)
    for j in (-8, -3, 1, 4):
        import copy
        sc = copy.copy(inp)
        kv = inp.kv.copy()
        s = kv[:, 64 * 128: 64 * 128 + 256].copy().view(np.float32) * np.float32(2.0 ** j)
        kv[:, 64 * 128: 64 * 128 + 256] = s.view(np.uint8)
        sc.kv = kv
        r, _, _ = oracle.mqa_logits_for(sc)
        assert np.array_equal(r[m], base[m] * 2.0 ** j)


@pytest.mark.parametrize("variant", ["fp8", "mxfp4"])
def test_page_permutation_invariance(variant):
    inp = _small(variant, 16)
    base, _, m = oracle.mqa_logits_for(inp)
    rng = np.random.default_rng(0)
    perm = rng.permutation(inp.num_pages)
    import copy
    p2 = copy.copy(inp)
    p2.kv = np.empty_like(inp.kv)
    p2.kv[perm] = inp.kv
    bt = inp.block_table.copy()
    bt[bt >= 0] = perm[bt[bt >= 0]]
    p2.block_table = bt
    r, _, m2 = oracle.mqa_logits_for(p2)
    assert np.array_equal(m, m2) and np.array_equal(r[m], base[m])


def test_written_set_follows_extent_and_skips_empty_requests():
    """Rows of a request with seq_lens == 0 are never written; other rows are
    written over whole 64-token pages up to max_context."""
    lens = [0, 1, 63, 64, 65, 250, -3]
    inp = synth.make_mqa_inputs(lens, 3, max_context=192, bt_width=4, seed=17)
    _, _, m = oracle.mqa_logits_for(inp)
    for b, L in enumerate(lens):
        E = extent(L, 192)
        for t in range(3):
            r = b * 3 + t
            assert m[r, :E].all() and not m[r, E:].any(), (b, L)


@pytest.mark.parametrize("next_n", [1, 4])
def test_written_set_function_equals_dense_written_mask(next_n):
    """oracle.mqa_written (the written set every full-size GPU check takes) equals
    the dense oracle's written mask and the extent rule written out here, on
    lengths 0, negative, 1, 63, 64, 65 and beyond max_context (clamped)."""
    lens = [0, -7, 1, 63, 64, 65, 200, 256, 1000, 129]
    inp = synth.make_mqa_inputs(lens, next_n, max_context=256, bt_width=16, seed=19 + next_n)
    _, _, dense = oracle.mqa_logits_for(inp)
    fast = oracle.mqa_written(inp.seq_lens, inp.batch, next_n, inp.max_context)
    rule = np.zeros((len(lens) * next_n, 256), dtype=bool)
    for b, L in enumerate(lens):
        cols = 0 if L <= 0 else min(-(-L // 64) * 64, 256)
        rule[b * next_n:(b + 1) * next_n, :cols] = True
    assert np.array_equal(fast, dense)
    assert np.array_equal(fast, rule)


def test_meaningful_rows_equal_single_token_calls():
    """Row b*N+t holds the logits of query slot t; its meaningful columns
    0..L-N+t equal a next_n = 1 call with that slot's query and weights."""
    N = 4
    inp = synth.make_mqa_inputs([150, 70], N, max_context=192, bt_width=3, seed=18)
    full, _, _ = oracle.mqa_logits_for(inp)
    import copy
    for t in range(N):
        one = copy.copy(inp)
        one.next_n = 1
        one.q = np.ascontiguousarray(inp.q[:, t:t + 1])
        one.weights = np.ascontiguousarray(inp.weights.reshape(2, N, -1)[:, t])
        one.seq_lens = inp.seq_lens - N + t + 1
        r1, _, m1 = oracle.mqa_logits_for(one)
        for b in range(2):
            last = int(inp.seq_lens[b]) - N + t
            assert np.array_equal(full[b * N + t, : last + 1], r1[b, : last + 1])


def test_mxfp4_group_scale_changes_result_non_proportionally():
    """Raising one k group's e8m0 code by one doubles that group's share of
    every head score: the difference identity then moves by exactly that
    group's contribution, which is not a multiple of the old result."""
    inp = _small("mxfp4", 19, next_n=1, lens=(64,))
    import copy
    bumped = copy.copy(inp)
    kv = inp.kv.copy()
    sf_off = 64 * 64
    g = 2
    kv[:, sf_off + g: sf_off + 256: 4] += 1
    bumped.kv = kv
    d0 = oracle.mqa_logits_for(inp)[0] - oracle.mqa_logits_for(flip_key_signs(inp))[0]
    d1 = oracle.mqa_logits_for(bumped)[0] - oracle.mqa_logits_for(flip_key_signs(bumped))[0]
    Q = decode_queries(inp)[0, 0]  # [H, D]
    k = decode_keys(inp)[0][0]
    kg = np.zeros_like(k)
    kg[:, 32 * g: 32 * g + 32] = k[:, 32 * g: 32 * g + 32]
    contrib = inp.weights[0].astype(np.float64) @ (Q @ kg.T)
    np.testing.assert_allclose(d1[0, :64] - d0[0, :64], contrib, rtol=1e-12, atol=1e-9)
    ratio = d1[0, :64] / d0[0, :64]
    assert np.ptp(ratio) > 1e-3  # not one common factor


# ------------------------------------------- other head counts, dims, next_n

# (num_heads, head_dim, next_n): head counts that are not multiples of 16 or
# 32, head_dims that are not multiples of 128, and next_n above 4
OTHER_SHAPES = [(1, 16, 1), (3, 32, 5), (5, 48, 6), (33, 144, 3), (128, 256, 2), (64, 128, 8),
                (64, 128, 5)]


def _brute_force(inp):
    """The equation cell by cell in plain Python over independently decoded
    data: s_p * sum_h w[r,h] * max(0, sum_d q[b,t,h,d] k_p[d])."""
    Q = decode_queries(inp).tolist()
    W = inp.weights.astype(np.float64).tolist()
    out = {}
    for b, (k, s) in enumerate(decode_keys(inp)):
        kl = k.tolist()
        for t in range(inp.next_n):
            r = b * inp.next_n + t
            for p in range(len(kl)):
                acc = 0.0
                for h in range(inp.num_heads):
                    dot = 0.0
                    for d in range(inp.head_dim):
                        dot += Q[b][t][h][d] * kl[p][d]
                    acc += W[r][h] * max(dot, 0.0)
                out[r, p] = float(s[p]) * acc
    return out


@pytest.mark.parametrize("H,D,N", [(3, 32, 5), (1, 16, 2), (5, 48, 1), (2, 144, 7)])
def test_brute_force_at_other_shapes(H, D, N):
    inp = synth.make_mqa_inputs([70, 0, 5], N, num_heads=H, head_dim=D, max_context=128,
                                bt_width=2, seed=30 + H + D, w_std=1.0)
    ref, amag, m = oracle.mqa_logits_for(inp)
    bf = _brute_force(inp)
    assert int(m.sum()) == len(bf)
    for (r, p), v in bf.items():
        assert m[r, p]
        assert abs(ref[r, p] - v) <= 1e-12 * amag[r, p] + 1e-300, (r, p)


@pytest.mark.parametrize("H,D,N", OTHER_SHAPES)
def test_rectifier_identities_at_other_shapes(H, D, N):
    """The difference and sum identities of the rectifier (see above) at head
    counts, head_dims and next_n other than 64, 128 and 1..4."""
    inp = synth.make_mqa_inputs([37, 0, 130, 64], N, num_heads=H, head_dim=D, max_context=192,
                                bt_width=3, seed=40 + N, w_std=1.0)
    r1, a1, m = oracle.mqa_logits_for(inp)
    r2, _, m2 = oracle.mqa_logits_for(flip_key_signs(inp))
    assert np.array_equal(m, m2)
    lin = _weighted_query_dot(inp, "lin")
    ab = _weighted_query_dot(inp, "abs")
    np.testing.assert_allclose((r1 - r2)[m], lin[m], rtol=1e-12, atol=1e-9 * np.max(a1))
    np.testing.assert_allclose((r1 + r2)[m], ab[m], rtol=1e-12, atol=1e-9 * np.max(a1))
    assert np.array_equal(np.isnan(lin), ~m)


# ------------------------------------------------------------------ indexer


@pytest.mark.parametrize("uniform", [None, 4])
def test_indexer_is_plain_dot_product(uniform):
    inp = synth.make_config("indexer_bf16", uniform_group=uniform)
    ref, amag, m = oracle.indexer_scores_for(inp)
    q = np_bf16(inp.query)
    offs = inp.row_offsets()
    for g in range(inp.groups):
        L = min(int(inp.context_lengths[g]), inp.max_context)
        rows = slice(offs[g], offs[g + 1])
        if L <= 0:
            assert not m[rows].any()
            continue
        pages = inp.block_table[inp.requests[g], : (L + 63) // 64]
        keys = np_bf16(inp.key_cache[pages, : 64 * 128 * 2].copy().view(np.uint16)).reshape(-1, 128)[:L]
        np.testing.assert_allclose(ref[rows, :L], q[rows] @ keys.T, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(amag[rows, :L], np.abs(q[rows]) @ np.abs(keys).T, rtol=1e-12)
        assert m[rows, :L].all() and not m[rows, L:].any()


def test_one_head_fp8_equals_rectified_indexer():
    """The indexer is the one-head case of the logits: with a one-hot weight,
    s_p = 1 and values exact in both e4m3 and bf16, max(score, 0) equals the
    FP8 logit exactly."""
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
    fp8, _, m = oracle.mqa_logits_for(inp)
    kc = synth.encode_bf16(kf).view(np.uint8).reshape(inp.num_pages, -1)
    ix = synth.IndexerInputs(synth.encode_bf16(qf[0, 0, :1]), kc, 64 * 128 * 2, inp.block_table,
                             np.array([128], np.int32), np.array([0], np.int32),
                             np.array([0, 1], np.int32), 128)
    sc, _, _ = oracle.indexer_scores_for(ix)
    assert np.array_equal(np.maximum(sc[0, :128], 0.0), fp8[0, :128])


def test_points_agree_with_dense():
    inp = _small("fp8", 22, next_n=3)
    ref, amag, m = oracle.mqa_logits_for(inp)
    rng = np.random.default_rng(1)
    rows = rng.integers(0, inp.rows, 300)
    cols = rng.integers(0, inp.max_context, 300)
    r, a, w = oracle.mqa_logits_points_for(inp, rows, cols)
    assert np.array_equal(w, m[rows, cols])
    assert np.array_equal(r[w], ref[rows, cols][w])
    assert np.array_equal(a[w], amag[rows, cols][w])


def test_generator_is_deterministic():
    a = synth.make_config("tiny_fp8")
    b = synth.make_config("tiny_fp8")
    assert np.array_equal(a.kv, b.kv) and np.array_equal(a.q, b.q)
    assert np.array_equal(a.weights, b.weights) and np.array_equal(a.block_table, b.block_table)
    assert sorted(a.block_table.ravel().tolist()) == list(range(8))


# ------------------------------------------------------- NVFP4 indexer scores


def test_golden_indexer_nvfp4():
    """Hand-worked NVFP4 cases (codes in, exact values out)."""
    from fixtures_util import nvfp4_indexer_from_case
    for case in load_golden("indexer_nvfp4_cases.json")["cases"]:
        ix = nvfp4_indexer_from_case(case)
        ref, _, written = oracle.indexer_scores_for(ix)
        L = case["context_length"]
        assert written[:, :L].all() and not written[:, L:].any(), case["name"]
        for r, exp in enumerate(case["expected"]):
            for col, v in exp.items():
                assert ref[r, int(col)] == v, (case["name"], r, col, ref[r, int(col)], v)


def _nvfp4_small(seed, **kw):
    kw.setdefault("rows", 12)
    kw.setdefault("num_requests", 3)
    kw.setdefault("bt_width", 4)
    kw.setdefault("max_context", 256)
    kw.setdefault("max_len", 256)
    return synth.make_indexer_inputs(seed=seed, fmt="nvfp4", **kw)


def test_nvfp4_matches_independent_decode():
    """float64 matmul of values decoded independently (torch's e4m3 cast, the
    e2m1 table), gathered through the block table."""
    from fixtures_util import np_nvfp4
    ix = _nvfp4_small(21)
    ref, _, written = oracle.indexer_scores_for(ix)
    q = np_nvfp4(ix.query, ix.query_scales)
    P = ix.key_cache.shape[0]
    keys = np_nvfp4(ix.key_cache[:, :64 * 64].reshape(P, 64, 64),
                    ix.key_scales[:, :64 * 8].reshape(P, 64, 8))
    offs = ix.row_offsets()
    checked = 0
    for g in range(ix.groups):
        L = min(max(int(ix.context_lengths[g]), 0), ix.max_context)
        if L == 0:
            continue
        pages = ix.block_table[ix.requests[g]]
        kmat = np.concatenate([keys[pages[i]] for i in range((L + 63) // 64)])[:L]
        exp = q[offs[g]:offs[g + 1]] @ kmat.T
        np.testing.assert_allclose(ref[offs[g]:offs[g + 1], :L], exp, rtol=1e-12, atol=1e-12)
        checked += exp.size
    assert checked > 500


def test_nvfp4_equals_bf16_indexer_on_dequantised_inputs():
    """An E2M1 value times an E4M3 scale has at most 6 significant bits, so it
    is exact in bf16: the NVFP4 path must equal the BF16 path of the oracle
    on the dequantised tensors, bit for bit."""
    from fixtures_util import np_nvfp4
    ix = _nvfp4_small(22)
    P = ix.key_cache.shape[0]
    q = np_nvfp4(ix.query, ix.query_scales).astype(np.float32)
    keys = np_nvfp4(ix.key_cache[:, :4096].reshape(P, 64, 64),
                    ix.key_scales[:, :512].reshape(P, 64, 8)).astype(np.float32)
    qb, kb = synth.encode_bf16(q), synth.encode_bf16(keys)
    from fixtures_util import np_bf16
    assert np.array_equal(np_bf16(qb), q.astype(np.float64))
    assert np.array_equal(np_bf16(kb), keys.astype(np.float64))
    ref_nv, amag_nv, w_nv = oracle.indexer_scores_for(ix)
    ref_bf, amag_bf, w_bf = oracle.indexer_scores(qb, kb.view(np.uint8).reshape(P, -1), 64 * 256,
                                                  ix.block_table, ix.context_lengths,
                                                  ix.requests, ix.row_offsets(), ix.max_context)
    assert np.array_equal(w_nv, w_bf)
    assert np.array_equal(ref_nv[w_nv], ref_bf[w_bf])
    assert np.array_equal(amag_nv[w_nv], amag_bf[w_bf])


def test_nvfp4_key_scale_doubling_is_exact():
    """Raising every key scale's exponent by one doubles every score exactly."""
    ix = _nvfp4_small(23)
    ks = ix.key_scales.copy()
    e = (ks >> 3) & 15
    assert ((e >= 1) & (e < 14)).all()  # normal scales, no overflow into the NaN code
    ks = ks + np.uint8(8)
    ix2 = copy.copy(ix)
    ix2.key_scales = ks
    ref, _, w = oracle.indexer_scores_for(ix)
    ref2, _, w2 = oracle.indexer_scores_for(ix2)
    assert np.array_equal(w, w2)
    assert np.array_equal(ref2[w], 2.0 * ref[w])


# ------------------------------------------- the cancelling-input fixture


def _fp8_run_truncated_dots(q, k):
    """q [H, D] x k [T, D] -> [H, T], summed the way gfx950's FP8 matrix
    instructions were measured to sum: within each aligned run of 8 head_dim
    values every product is truncated toward zero to a multiple of 2^(E-13),
    E the exponent of the run's largest product; the runs add exactly."""
    p = q[:, None, :] * k[None, :, :]
    runs = p.reshape(p.shape[0], p.shape[1], -1, 8)
    m = np.max(np.abs(runs), axis=-1, keepdims=True)
    e = np.floor(np.log2(np.where(m > 0, m, 1.0)))
    u = np.ldexp(1.0, (e - 13).astype(np.int64))
    t = np.sign(runs) * np.floor(np.abs(runs) / u) * u
    return t.sum(axis=(-1, -2))


@pytest.mark.parametrize("next_n", [1, 4])
def test_cancelling_fixture_defeats_fp8_run_truncation(next_n):
    """The GPU tests' cancelling inputs are meant to fail a kernel that sums
    with the FP8 matrix instructions.  Assembling the logits from dot
    products summed in that truncated way violates 2e-3*A on most cells, while
    the same assembly from exact float64 dot products matches the oracle."""
    from fixtures_util import cancelling_mqa_inputs
    inp = cancelling_mqa_inputs("fp8", next_n, 300 + next_n)
    ref, amag, written = oracle.mqa_logits_for(inp)
    q = decode_queries(inp)
    N = next_n
    bad = total = 0
    for b, (k, sp) in enumerate(decode_keys(inp)):
        for t in range(N):
            r = b * N + t
            w = inp.weights[r].astype(np.float64)
            trunc = _fp8_run_truncated_dots(q[b, t], k)
            exact = q[b, t] @ k.T
            lt = sp * (w @ np.maximum(trunc, 0.0))
            le = sp * (w @ np.maximum(exact, 0.0))
            E = k.shape[0]
            assert written[r, :E].all()
            np.testing.assert_allclose(le, ref[r, :E], rtol=1e-12, atol=1e-12)
            tol = 2e-3 * amag[r, :E] + 1e-5
            bad += int(np.sum(np.abs(lt - ref[r, :E]) > tol))
            total += E
    assert total > 0 and bad > 0.9 * total, (bad, total)


# ---------------------------------------------- MXFP4 scale layouts (readings)

MX_LAYOUTS = [(32, False), (16, False), (32, True), (16, True)]


@pytest.mark.parametrize("case", load_golden("mxfp4_layout_cases.json")["cases"],
                         ids=lambda c: c["name"])
def test_mxfp4_layout_golden(case):
    inp = mqa_from_case(case, "mxfp4")
    ref, _, written = oracle.mqa_logits_for(inp)
    E = extent(case["seq_len"], inp.max_context)
    assert written[0, :E].all() and not written[0, E:].any()
    for col, v in case["expected"].items():
        assert ref[0, int(col)] == v, (case["name"], col)


@pytest.mark.parametrize("sfv,il", MX_LAYOUTS)
def test_mxfp4_layout_rectifier_identities(sfv, il):
    """The two rectifier identities, against float64 matrix products of values
    decoded independently (numpy, library e8m0 cast) in each scale layout."""
    inp = synth.make_mqa_inputs([37, 0, 130, 64], 2, variant="mxfp4", max_context=192,
                                bt_width=3, seed=13, sf_vec_size=sfv, kv_sf_interleaved=il)
    r1, a1, m = oracle.mqa_logits_for(inp)
    r2, _, m2 = oracle.mqa_logits_for(flip_key_signs(inp))
    assert np.array_equal(m, m2)
    lin = _weighted_query_dot(inp, "lin")
    ab = _weighted_query_dot(inp, "abs")
    np.testing.assert_allclose((r1 - r2)[m], lin[m], rtol=1e-12, atol=1e-9 * np.max(a1))
    np.testing.assert_allclose((r1 + r2)[m], ab[m], rtol=1e-12, atol=1e-9 * np.max(a1))


@pytest.mark.parametrize("sfv", [32, 16])
def test_mxfp4_interleaved_records_equal_trailing_codes(sfv):
    """Rearranging every page from the trailing layout (all packed rows, then
    all codes) into token records (packed row, then that token's codes) --
    done here with plain slicing -- leaves every logit bit-identical."""
    inp = synth.make_mqa_inputs([300, 1, 129], 3, variant="mxfp4", max_context=320,
                                bt_width=5, seed=14, sf_vec_size=sfv)
    base, _, m = oracle.mqa_logits_for(inp)
    D, nsf, P = 128, 128 // sfv, inp.num_pages
    rec = copy.copy(inp)
    kv = np.zeros_like(inp.kv)
    for t in range(64):
        kv[:, t * (D // 2 + nsf): t * (D // 2 + nsf) + D // 2] = inp.kv[:, t * D // 2:(t + 1) * D // 2]
        kv[:, t * (D // 2 + nsf) + D // 2:(t + 1) * (D // 2 + nsf)] = \
            inp.kv[:, 64 * D // 2 + t * nsf: 64 * D // 2 + (t + 1) * nsf]
    rec.kv, rec.kv_sf_interleaved = kv, True
    got, _, m2 = oracle.mqa_logits_for(rec)
    assert np.array_equal(m, m2) and np.array_equal(got[m], base[m])


def test_mxfp4_sixteen_value_codes_that_pair_up_equal_thirty_two():
    """With sf_vec_size = 16, giving both halves of every 32-value block the
    same code must equal the sf_vec_size = 32 layout with that code."""
    inp = synth.make_mqa_inputs([200, 64], 2, variant="mxfp4", max_context=256, bt_width=4,
                                seed=15, sf_vec_size=32)
    base, _, m = oracle.mqa_logits_for(inp)
    D, P = 128, inp.num_pages
    s16 = copy.copy(inp)
    s16.q_sf = np.repeat(inp.q_sf, 2, axis=-1)
    packed = inp.kv[:, : 64 * D // 2]
    codes = inp.kv[:, 64 * D // 2: 64 * D // 2 + 64 * 4].reshape(P, 64, 4)
    s16.kv = np.concatenate([packed, np.repeat(codes, 2, axis=-1).reshape(P, -1)], axis=1)
    s16.page_stride, s16.sf_vec_size = s16.kv.shape[1], 16
    got, _, m2 = oracle.mqa_logits_for(s16)
    assert np.array_equal(m, m2) and np.array_equal(got[m], base[m])
