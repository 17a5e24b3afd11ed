"""Helpers shared by the tests: golden-fixture builders, independent decoders
(numpy/torch library casts, not the oracle's) and the parity comparison."""
from __future__ import annotations

import json
import os

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# OCP MX e2m1 magnitudes by 3-bit code (sign is bit 3), from the format table.
E2M1_TABLE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])

F32_SENTINEL = 0x7FC0FFEE  # a NaN payload no finite write produces
BF16_SENTINEL = 0x7FC1


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------- independent decoders


def np_e4m3(codes):
    import torch
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()


def np_e8m0(codes):
    import torch
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(
        torch.float8_e8m0fnu).to(torch.float64).numpy()


def np_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(
        torch.bfloat16).to(torch.float64).numpy()


def np_e2m1_unpack(packed):
    """u8 [..., D/2] -> float64 [..., D], even element in the low nibble."""
    lo = packed & 15
    hi = packed >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(packed.shape[:-1] + (packed.shape[-1] * 2,))
    mag = E2M1_TABLE[nib & 7]
    return np.where(nib & 8, -mag, mag)


def e2m1_code(v):
    mag = abs(v)
    idx = int(np.nonzero(E2M1_TABLE == mag)[0][0])
    return idx | (8 if v < 0 else 0)


def mx_page_fields(pg, D, sfv, interleaved):
    """(packed u8 [64, D/2], codes u8 [64, D/sfv]) of one MXFP4 page's bytes:
    all packed rows then all codes, or 64 records of packed bytes + codes."""
    nsf = D // sfv
    if interleaved:
        rec = pg[: 64 * (D // 2 + nsf)].reshape(64, D // 2 + nsf)
        return rec[:, : D // 2], rec[:, D // 2:]
    return pg[: 64 * D // 2].reshape(64, D // 2), pg[64 * D // 2: 64 * D // 2 + 64 * nsf].reshape(
        64, nsf)


def decode_keys(inp):
    """Per request: (k float64 [E_b, D], s float64 [E_b]) over the written extent."""
    out = []
    D = inp.head_dim
    sfv = getattr(inp, "sf_vec_size", 32)
    il = getattr(inp, "kv_sf_interleaved", False)
    for b in range(inp.batch):
        L = int(inp.seq_lens[b])
        E = 0 if L <= 0 else min((L + 63) // 64 * 64, inp.max_context)
        ks, ss = [], []
        for j in range(E // 64):
            pg = inp.kv[inp.block_table[b, j]]
            if inp.variant == "fp8":
                ks.append(np_e4m3(pg[: 64 * D].reshape(64, D)))
                ss.append(pg[64 * D: 64 * D + 256].view(np.float32).astype(np.float64))
            else:
                packed, codes = mx_page_fields(pg, D, sfv, il)
                vals = np_e2m1_unpack(packed)
                ks.append(vals * np.repeat(np_e8m0(codes), sfv, axis=1))
                ss.append(np.ones(64))
        out.append((np.concatenate(ks) if ks else np.zeros((0, D)),
                    np.concatenate(ss) if ss else np.zeros(0)))
    return out


def decode_queries(inp):
    """float64 [B, N, H, D]."""
    if inp.variant == "fp8":
        return np_e4m3(inp.q)
    vals = np_e2m1_unpack(inp.q)
    sf = np_e8m0(inp.q_sf)
    return vals * np.repeat(sf, getattr(inp, "sf_vec_size", 32), axis=-1)


def flip_key_signs(inp):
    """A copy of ``inp`` whose key values are negated (scales unchanged)."""
    import copy
    out = copy.copy(inp)
    kv = inp.kv.copy()
    D = inp.head_dim
    if inp.variant == "fp8":
        kv[:, : 64 * D] ^= 0x80
    elif getattr(inp, "kv_sf_interleaved", False):
        rec = D // 2 + D // getattr(inp, "sf_vec_size", 32)
        view = kv[:, : 64 * rec].reshape(kv.shape[0], 64, rec)
        view[:, :, : D // 2] ^= 0x88
    else:
        kv[:, : 64 * D // 2] ^= 0x88
    out.kv = kv
    return out


# ----------------------------------------------------------- fixture builders


def mqa_from_case(case, variant):
    H, D = 64, 128
    P = case["num_pages"]
    stride = synth.page_bytes(variant, D)
    kv = np.zeros((P, stride), dtype=np.uint8)
    bt = np.array([case["block_table"]], dtype=np.int32)
    w = np.zeros((1, H), dtype=np.float32)
    if variant == "fp8":
        qf = np.zeros((1, 1, H, D), dtype=np.float32)
        for hd in case["heads"]:
            w[0, hd["h"]] = hd["w"]
            for d, v in hd["q"].items():
                qf[0, 0, hd["h"], int(d)] = v
        q = synth.encode_e4m3(qf)
        assert np.array_equal(np_e4m3(q), qf.astype(np.float64)), "fixture value not exact in e4m3"
        q_sf = None
        kv[:, 64 * D: 64 * D + 256] = np.ones((P, 64), dtype=np.float32).view(np.uint8)
        for tk in case["tokens"]:
            p = tk["pos"]
            page, slot = case["block_table"][p // 64], p % 64
            kf = np.zeros(D, dtype=np.float32)
            for d, v in tk["k"].items():
                kf[int(d)] = v
            codes = synth.encode_e4m3(kf)
            assert np.array_equal(np_e4m3(codes), kf.astype(np.float64))
            kv[page, slot * D:(slot + 1) * D] = codes
            kv[page, 64 * D + 4 * slot: 64 * D + 4 * slot + 4] = np.array(
                [tk["s"]], dtype=np.float32).view(np.uint8)
    else:
        sfv = case.get("sf_vec_size", 32)
        il = bool(case.get("interleaved", False))
        nsf = D // sfv
        stride = synth.page_bytes(variant, D, sfv)
        kv = np.zeros((P, stride), dtype=np.uint8)
        q = np.zeros((1, 1, H, D // 2), dtype=np.uint8)
        q_sf = np.full((1, 1, H, nsf), 127, dtype=np.uint8)
        packed = np.zeros((P, 64, D // 2), dtype=np.uint8)
        codes = np.full((P, 64, nsf), 127, dtype=np.uint8)
        for hd in case["heads"]:
            w[0, hd["h"]] = hd["w"]
            for d, v in hd["q"].items():
                d = int(d)
                q[0, 0, hd["h"], d // 2] |= e2m1_code(v) << (4 * (d & 1))
            for g, c in hd.get("sf", {}).items():
                q_sf[0, 0, hd["h"], int(g)] = c
        for tk in case["tokens"]:
            p = tk["pos"]
            page, slot = case["block_table"][p // 64], p % 64
            for d, v in tk["k"].items():
                d = int(d)
                packed[page, slot, d // 2] |= e2m1_code(v) << (4 * (d & 1))
            for g, c in tk.get("sf", {}).items():
                codes[page, slot, int(g)] = c
        if il:  # 64 records: a token's packed bytes, then its codes
            kv[:, :] = np.concatenate([packed, codes], axis=2).reshape(P, -1)
        else:
            kv[:, :] = np.concatenate([packed.reshape(P, -1), codes.reshape(P, -1)], axis=1)
    L = case["seq_len"]
    max_context = max(64, (L + 63) // 64 * 64)
    inp = synth.MqaInputs(variant, 1, 1, H, D, max_context, q, q_sf, kv, stride, w,
                          np.array([L], dtype=np.int32), bt,
                          "f32" if variant == "fp8" else "bf16", case["name"])
    if variant != "fp8":
        inp.sf_vec_size, inp.kv_sf_interleaved = sfv, il
    return inp


def indexer_from_case(case):
    D = 128
    P = case["num_pages"]
    rows = len(case["rows"])
    qf = np.zeros((rows, D), dtype=np.float32)
    for r, row in enumerate(case["rows"]):
        for d, v in row["q"].items():
            qf[r, int(d)] = v
    q = synth.encode_bf16(qf)
    keys = np.zeros((P, 64, D), dtype=np.float32)
    for tk in case["tokens"]:
        p = tk["pos"]
        page, slot = case["block_table"][p // 64], p % 64
        for d, v in tk["k"].items():
            keys[page, slot, int(d)] = v
    kc = synth.encode_bf16(keys).view(np.uint8).reshape(P, -1).copy()
    L = case["context_length"]
    max_context = max(64, (L + 63) // 64 * 64)
    bt = np.array([case["block_table"]], dtype=np.int32)
    return synth.IndexerInputs(q, kc, 64 * D * 2, bt, np.array([L], dtype=np.int32),
                               np.array([0], dtype=np.int32),
                               np.array([0, rows], dtype=np.int32), max_context, case["name"])


def nvfp4_indexer_from_case(case):
    """IndexerInputs (fmt nvfp4) from a golden case given as E2M1 / E4M3 codes."""
    D, P = 128, case["num_pages"]
    rows = len(case["rows"])
    qn = np.zeros((rows, D), dtype=np.uint8)
    qs = np.full((rows, D // 16), 0x38, dtype=np.uint8)
    for r, row in enumerate(case["rows"]):
        for d, c in row["q"].items():
            qn[r, int(d)] = int(c, 16)
        for b, c in row.get("qs", {}).items():
            qs[r, int(b)] = int(c, 16)
    kn = np.zeros((P, 64, D), dtype=np.uint8)
    ks = np.full((P, 64, D // 16), 0x38, dtype=np.uint8)
    for tk in case["tokens"]:
        p = tk["pos"]
        page, slot = case["block_table"][p // 64], p % 64
        for d, c in tk["k"].items():
            kn[page, slot, int(d)] = int(c, 16)
        for b, c in tk.get("ks", {}).items():
            ks[page, slot, int(b)] = int(c, 16)
    pack = lambda n: (n[..., 0::2] | (n[..., 1::2] << 4)).astype(np.uint8)
    L = case["context_length"]
    max_context = max(64, (L + 63) // 64 * 64)
    bt = np.array([case["block_table"]], dtype=np.int32)
    return synth.IndexerInputs(pack(qn), pack(kn).reshape(P, -1).copy(), 64 * D // 2, bt,
                               np.array([L], dtype=np.int32), np.array([0], dtype=np.int32),
                               np.array([0, rows], dtype=np.int32), max_context, case["name"],
                               "nvfp4", qs, ks.reshape(P, -1).copy(), 64 * D // 16)


def np_nvfp4(packed, scales):
    """Dequantised float64 values of NVFP4 data: u8 [..., D/2] packed e2m1 and
    u8 [..., D/16] e4m3 scales -> float64 [..., D]."""
    v = np_e2m1_unpack(packed)
    return v * np.repeat(np_e4m3(scales), 16, axis=-1)


# ---------------------------------------------------------------- comparison


def extent(L, max_context):
    return 0 if L <= 0 else min((L + 63) // 64 * 64, max_context)


# ------------------------------------------------ cancelling dot products


def pack_e2m1(v):
    """Values on the e2m1 grid -> packed u8 [..., D/2], even element in the low
    nibble (exact; asserts that every value is on the grid)."""
    mag = np.abs(v)
    idx = np.searchsorted(E2M1_TABLE, mag)
    assert np.all(E2M1_TABLE[np.minimum(idx, 7)] == mag), "value not on the e2m1 grid"
    nib = (idx | np.where(v < 0, 8, 0)).astype(np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def cancelling_mqa_inputs(variant, next_n, seed, *, one_hot=True, out_dtype="f32", pow2=False):
    """Inputs whose logits rest on a cancelling dot product.

    Every query slot has one dominant head h* (one-hot weights, or weights
    2^10 above the rest).  FP8: h*'s q and every key carry a pair q = (256,
    256), k = (256, -256) in one aligned block of 8 head_dim values, whose
    products (+-2^16) cancel, plus a tail of positive products in [2^-18,
    2^-14] of the pair's (values in [0.5, 2]) over the rest of that block and
    24 other positions; the tail is the whole dot product.  MXFP4: the pair
    is (6, 6) x (6, -6) in block 0 with small products beside it, and the
    tail sits in block 2 of h*, whose e8m0 scale is 2^-14 (the other blocks'
    is 1).  The other heads and key values are small random values.  With
    pow2 (one-hot only) weights and s_p are powers of two, so the exact
    result is representable and the sum of the tail is exact in fp32."""
    rng = np.random.default_rng(seed)
    inp = synth.make_mqa_inputs([300, 64, 1, 129, 700], next_n, variant=variant, max_context=768,
                                bt_width=12, seed=seed, out_dtype=out_dtype)
    B, N, H, D, P = inp.batch, next_n, 64, 128, inp.num_pages
    w = np.zeros((B * N, H), np.float32)
    if variant == "fp8":
        small = lambda shape: np.where(rng.random(shape) < 0.5, -1.0, 1.0) * rng.uniform(  # noqa
            0.5, 2.0, shape)
        blk = int(rng.integers(0, 16))
        d1, d2 = 8 * blk + int(rng.integers(0, 4)), 8 * blk + 4 + int(rng.integers(0, 4))
        in_blk = [d for d in range(8 * blk, 8 * blk + 8) if d not in (d1, d2)]
        others = [d for d in range(D) if d // 8 != blk]
        tail = np.array(in_blk + rng.choice(others, 24, replace=False).tolist())
        kf = small((P, 64, D))
        kf[:, :, d1], kf[:, :, d2] = 256.0, -256.0
        kf[:, :, tail] = rng.uniform(0.5, 2.0, (P, 64, tail.size))
        qf = small((B, N, H, D))
        for r in range(B * N):
            b, t = divmod(r, N)
            h = int(rng.integers(0, H))
            qf[b, t, h] = 0.0
            qf[b, t, h, d1] = qf[b, t, h, d2] = 256.0
            qf[b, t, h, tail] = rng.uniform(0.5, 2.0, tail.size)
            sign = 1.0 if rng.random() < 0.75 else -1.0
            if one_hot:
                w[r, h] = sign * (2.0 ** int(rng.integers(-2, 3)) if pow2 else rng.uniform(0.5, 2.0))
            else:
                w[r] = rng.standard_normal(H) * 2.0 ** -10
                w[r, h] = sign * rng.uniform(0.5, 2.0)
        inp.q = synth.encode_e4m3(qf.astype(np.float32))
        inp.kv[:, : 64 * D] = synth.encode_e4m3(kf.astype(np.float32)).reshape(P, -1)
        if pow2:
            sp = np.ldexp(1.0, rng.integers(-3, 4, (P, 64))).astype(np.float32)
        else:
            sp = rng.uniform(0.25, 4.0, (P, 64)).astype(np.float32)
        inp.kv[:, 64 * D: 64 * D + 256] = sp.view(np.uint8)
    else:
        grid = np.array([0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
        small = lambda shape: np.where(rng.random(shape) < 0.5, -1.0, 1.0) * rng.choice(  # noqa
            grid[:3], shape)
        kf = small((P, 64, D))
        kf[:, :, 0:32] = 0.0
        kf[:, :, 0], kf[:, :, 1] = 6.0, -6.0
        kf[:, :, 2:4] = 0.5
        kf[:, :, 64:96] = rng.choice(grid, (P, 64, 32))
        qf = small((B, N, H, D))
        q_sf = np.full((B, N, H, 4), 127, np.uint8)
        for r in range(B * N):
            b, t = divmod(r, N)
            h = int(rng.integers(0, H))
            qf[b, t, h] = 0.0
            qf[b, t, h, 0] = qf[b, t, h, 1] = 6.0
            qf[b, t, h, 2:4] = 0.5
            qf[b, t, h, 64:96] = rng.choice(grid, 32)
            q_sf[b, t, h, 2] = 127 - 14
            sign = 1.0 if rng.random() < 0.75 else -1.0
            if one_hot:
                w[r, h] = sign * 1024.0
            else:
                w[r] = rng.standard_normal(H)
                w[r, h] = sign * 1024.0 * rng.uniform(0.5, 2.0)
        pack = pack_e2m1
        inp.q = pack(qf)
        inp.q_sf = q_sf
        inp.kv[:, : 64 * D // 2] = pack(kf).reshape(P, -1)
        inp.kv[:, 64 * D // 2: 64 * D // 2 + 256] = 127
    inp.weights[:] = w
    return inp


# ------------------------------------------------------ block-max proxy score


def e4m3_code(v):
    """The e4m3 code of a value the format holds exactly."""
    c = int(synth.encode_e4m3(np.array([v], dtype=np.float32))[0])
    assert np_e4m3(np.array([c], np.uint8))[0] == v, "not exact in e4m3: %r" % v
    return c


def proxy_from_case(case):
    """synth.ProxyInputs from a golden case given as e2m1 values and e4m3 scale
    values per 16-element block (unlisted: value 0, scale 1.0)."""
    Hq, Hkv = case["Hq"], case["Hkv"]
    q_lens = np.array(case["q_lens"], np.int64)
    k_lens = np.array(case["k_lens"], np.int64)
    B = len(q_lens)
    cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    total_q = int(cu_q[-1])
    one = e4m3_code(1.0)
    qn = np.zeros((total_q, Hq, 128), np.uint8)
    qs = np.full((total_q, Hq, 8), one, np.uint8)
    for e in case["queries"]:
        for d, v in e["v"].items():
            qn[e["token"], e["head"], int(d)] = e2m1_code(v)
        for b, v in e.get("sf", {}).items():
            qs[e["token"], e["head"], int(b)] = e4m3_code(v)
    pack = lambda n: (n[..., 0::2] | (n[..., 1::2] << 4)).astype(np.uint8)
    if case["paged"]:
        P = case["num_pages"]
        pt = np.array(case["page_table"], np.int32)
        kn = np.zeros((P, Hkv, 128, 128), np.uint8)
        ks = np.full((P, Hkv, 128, 8), one, np.uint8)
        for e in case["keys"]:
            page, tok = pt[e["req"], e["pos"] // 128], e["pos"] % 128
            for d, v in e["v"].items():
                kn[page, e["kvh"], tok, int(d)] = e2m1_code(v)
            for b, v in e.get("sf", {}).items():
                ks[page, e["kvh"], tok, int(b)] = e4m3_code(v)
        k = pack(kn).reshape(P, -1).copy()
        k_scale = ks.reshape(-1, 8).copy()
        cu_k, seqused, stride = None, k_lens.astype(np.int32), Hkv * 128 * 64
    else:
        cu_k = np.concatenate([[0], np.cumsum(k_lens)]).astype(np.int32)
        kn = np.zeros((int(cu_k[-1]), Hkv, 128), np.uint8)
        ks = np.full((int(cu_k[-1]), Hkv, 8), one, np.uint8)
        for e in case["keys"]:
            row = cu_k[e["req"]] + e["pos"]
            for d, v in e["v"].items():
                kn[row, e["kvh"], int(d)] = e2m1_code(v)
            for b, v in e.get("sf", {}).items():
                ks[row, e["kvh"], int(b)] = e4m3_code(v)
        k = pack(kn)
        k_scale = ks.reshape(-1, 8).copy()
        pt, seqused, stride = None, None, 0
    qo = case.get("q_offset")
    return synth.ProxyInputs(pack(qn), qs.reshape(-1, 8).copy(), k, k_scale, bool(case["paged"]),
                             stride, cu_q, cu_k, pt, seqused, float(case["q_global_scale"]),
                             float(case["k_global_scale"]), Hq, Hkv, bool(case["causal"]),
                             None if qo is None else np.array(qo, np.int32),
                             int(case["max_k_tiles"]), bool(case["reduce_heads"]), case["name"])


def expected_value(v):
    return -np.inf if v == "-inf" else float(v)
