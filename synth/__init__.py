"""Seeded synthetic inputs for paged MQA logits and one-head indexer scores.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It only draws random numbers, quantises them to the storage formats
the operation consumes, and lays them out in pages.  It performs none of the
scoring arithmetic itself.

Formats (public standards, not taken from any implementation):
  * e4m3fn  - OCP 8-bit float, bias 7, max 448, NaN = 0x7F/0xFF, no infinity.
              Encoding uses torch's CPU cast (round to nearest even) after
              clamping to +-448, because the cast maps out-of-range values to NaN.
  * e2m1    - OCP MX 4-bit float {0, .5, 1, 1.5, 2, 3, 4, 6} with a sign bit,
              two per byte, the even element in the low nibble.
  * e8m0    - OCP MX scale, value 2**(code - 127).
  * bf16    - top half of an IEEE binary32, round to nearest even (torch cast).

Workloads follow the paged MQA logits page of the FlashInfer documentation
(flashinfer.attn_scores, introduction and output-contract note) and the
indexer_scores page (flashinfer.sdsa.indexer_scores, parameter list): pages of
64 tokens, a block table of int32 page ids per request, per-token FP8 scales in
a trailing region of each page, MXFP4 block scales per 32 elements.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

PAGE = 64  # tokens per KV page
INT32_MAX = 2**31 - 1

# --------------------------------------------------------------------------
# quantisers
# --------------------------------------------------------------------------


def encode_e4m3(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint8 e4m3fn codes (RNE, saturating at +-448)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.clamp_(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """uint8 e4m3fn codes -> float32 values (used only to quantise against a
    scale that is itself stored as e4m3)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float32).numpy()


def encode_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns (RNE)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def quantize_fp8_per_tensor(x: np.ndarray) -> np.ndarray:
    """Per-tensor e4m3 quantisation: scale = amax/448 (scale itself is dropped)."""
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    s = amax / 448.0 if amax > 0 else 1.0
    return encode_e4m3(x / np.float32(s))


def quantize_fp8_per_token(x: np.ndarray):
    """Per-row e4m3 quantisation.  Returns (codes uint8 [..., D], scales f32 [...])."""
    amax = np.max(np.abs(x), axis=-1)
    s = (amax / np.float32(448.0)).astype(np.float32)
    s[s == 0] = 1.0
    return encode_e4m3(x / s[..., None]), s


_E2M1_MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
# At a tie the even code wins: for each midpoint, True when the upper neighbour
# has the even code (so a tie rounds up).
_E2M1_TIE_UP = np.array([False, True, False, True, False, True, False])


def quantize_mxfp4(x: np.ndarray, block: int = 32):
    """OCP MX quantisation with `block`-element blocks along the last axis
    (32 in the OCP format; 16 for the sf_vec_size = 16 layout).

    shared exponent = floor(log2(amax)) - 2 (e2m1's largest exponent is 2),
    elements rounded to nearest even on the e2m1 grid and clamped to +-6.
    Returns (packed uint8 [..., D/2], scale codes uint8 [..., D/block]).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    D = x.shape[-1]
    assert D % block == 0
    xb = x.reshape(x.shape[:-1] + (D // block, block))
    amax = np.max(np.abs(xb), axis=-1)
    _, e = np.frexp(amax)  # amax = m * 2**e, m in [0.5, 1)
    shared = np.where(amax > 0, e.astype(np.int32) - 1 - 2, 0)
    code = np.clip(shared + 127, 1, 254).astype(np.int32)
    scale = np.ldexp(np.float32(1.0), code - 127).astype(np.float32)
    v = np.abs(xb) / scale[..., None]
    idx = np.zeros(v.shape, dtype=np.uint8)
    for mid, up in zip(_E2M1_MIDS, _E2M1_TIE_UP):
        idx += (v >= mid) if up else (v > mid)
    nib = idx | (np.signbit(xb).astype(np.uint8) << 3)
    nib = nib.reshape(x.shape)
    packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    return packed, code.astype(np.uint8)


def quantize_nvfp4(x: np.ndarray):
    """NVFP4 quantisation with 16-element blocks along the last axis.

    block scale = amax/6 (e2m1's largest magnitude) encoded as e4m3 (1.0 for
    an all-zero block); elements divided by the decoded scale, rounded to
    nearest even on the e2m1 grid and clamped to +-6.
    Returns (packed uint8 [..., D/2], e4m3 scale codes uint8 [..., D/16]).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    D = x.shape[-1]
    assert D % 16 == 0
    xb = x.reshape(x.shape[:-1] + (D // 16, 16))
    amax = np.max(np.abs(xb), axis=-1)
    code = encode_e4m3(np.where(amax > 0, amax / np.float32(6.0), np.float32(1.0)))
    scale = decode_e4m3(code)
    v = np.abs(xb) / scale[..., None]
    idx = np.zeros(v.shape, dtype=np.uint8)
    for mid, up in zip(_E2M1_MIDS, _E2M1_TIE_UP):
        idx += (v >= mid) if up else (v > mid)
    nib = idx | (np.signbit(xb).astype(np.uint8) << 3)
    nib = nib.reshape(x.shape)
    packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    return packed, code


# --------------------------------------------------------------------------
# paged MQA logits inputs
# --------------------------------------------------------------------------


@dataclasses.dataclass
class MqaInputs:
    variant: str  # "fp8" or "mxfp4"
    batch: int
    next_n: int
    num_heads: int
    head_dim: int
    max_context: int
    q: np.ndarray  # fp8: u8 [B,N,H,D]; mxfp4: u8 [B,N,H,D/2]
    q_sf: Optional[np.ndarray]  # mxfp4: u8 [B,N,H,D/sf_vec_size]; fp8: None
    kv: np.ndarray  # u8 [num_pages, page_stride]
    page_stride: int
    weights: np.ndarray  # f32 [B*N, H]
    seq_lens: np.ndarray  # i32 [B]
    block_table: np.ndarray  # i32 [B, W]
    out_dtype: str  # "f32" or "bf16"
    name: str = ""
    sf_vec_size: int = 32  # mxfp4: values per e8m0 code
    kv_sf_interleaved: bool = False  # mxfp4: each token's codes follow its packed bytes

    @property
    def num_pages(self) -> int:
        return self.kv.shape[0]

    @property
    def rows(self) -> int:
        return self.batch * self.next_n

    def kv_positions(self) -> int:
        return int(np.minimum(np.maximum(self.seq_lens, 0), self.max_context).sum())


def page_bytes(variant: str, head_dim: int, sf_vec_size: int = 32) -> int:
    """Minimum bytes of one page: 64 tokens of keys and their scales."""
    if variant == "fp8":
        return PAGE * head_dim + PAGE * 4
    return PAGE * (head_dim // 2) + PAGE * (head_dim // sf_vec_size)


def mxfp4_page(packed, sf, interleaved):
    """One MXFP4 page's bytes from packed keys u8 [..., 64, D/2] and codes
    u8 [..., 64, D/sfv]: all packed rows then all codes, or (interleaved) 64
    token records of packed bytes followed by that token's codes."""
    lead = packed.shape[:-2]
    if interleaved:
        return np.concatenate([packed, sf], axis=-1).reshape(lead + (-1,))
    return np.concatenate([packed.reshape(lead + (-1,)), sf.reshape(lead + (-1,))], axis=-1)


def _fill_pages(rng, variant, num_pages, head_dim, page_stride, chunk=2048, sf_vec_size=32,
                interleaved=False):
    """Every token slot of every page (tails included) holds valid data."""
    kv = np.zeros((num_pages, page_stride), dtype=np.uint8)
    kbytes = PAGE * head_dim if variant == "fp8" else PAGE * head_dim // 2
    for p0 in range(0, num_pages, chunk):
        p1 = min(num_pages, p0 + chunk)
        k = rng.standard_normal((p1 - p0, PAGE, head_dim), dtype=np.float32)
        if variant == "fp8":
            codes, s = quantize_fp8_per_token(k)
            kv[p0:p1, :kbytes] = codes.reshape(p1 - p0, -1)
            kv[p0:p1, kbytes:kbytes + PAGE * 4] = s.view(np.uint8).reshape(p1 - p0, -1)
        else:
            packed, sf = quantize_mxfp4(k, sf_vec_size)
            pg = mxfp4_page(packed, sf, interleaved)
            kv[p0:p1, :pg.shape[1]] = pg
    return kv


def make_mqa_inputs(seq_lens, next_n, *, variant="fp8", num_heads=64, head_dim=128,
                    max_context=None, bt_width=None, w_std=1.0, seed=0,
                    full_table=False, extra_pages=0, page_stride=None,
                    out_dtype=None, name="", sf_vec_size=32,
                    kv_sf_interleaved=False) -> MqaInputs:
    """Build one paged MQA logits workload.

    Physical page ids are a random permutation; request b owns the next
    ceil(L_b/64) of them in order.  Unused block-table entries are -1, unless
    ``full_table`` is set, in which case the table is a permutation of all
    pages (every entry a valid id).
    """
    rng = np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = int(seq_lens.shape[0])
    N, H, D = int(next_n), int(num_heads), int(head_dim)
    tiles = [(int(L) + PAGE - 1) // PAGE if L > 0 else 0 for L in seq_lens]
    if max_context is None:
        max_context = max(PAGE, max(tiles + [1]) * PAGE)
    if bt_width is None:
        bt_width = max(1, max_context // PAGE)
    need = sum(tiles)
    num_pages = B * bt_width if full_table else need + extra_pages
    num_pages = max(num_pages, 1)
    if page_stride is None:
        page_stride = page_bytes(variant, D, sf_vec_size)

    # draws: q, then weights, then page permutation, then page contents
    qf = rng.standard_normal((B, N, H, D), dtype=np.float32)
    if variant == "fp8":
        q = quantize_fp8_per_tensor(qf)
        q_sf = None
    else:
        q, q_sf = quantize_mxfp4(qf, sf_vec_size)
    weights = (rng.standard_normal((B * N, H), dtype=np.float32) * np.float32(w_std)).astype(np.float32)
    perm = rng.permutation(num_pages).astype(np.int32)
    if full_table:
        block_table = perm[: B * bt_width].reshape(B, bt_width).copy()
    else:
        block_table = np.full((B, bt_width), -1, dtype=np.int32)
        pos = 0
        for b, T in enumerate(tiles):
            T = min(T, bt_width)
            block_table[b, :T] = perm[pos:pos + T]
            pos += T
    kv = _fill_pages(rng, variant, num_pages, D, page_stride, sf_vec_size=sf_vec_size,
                     interleaved=kv_sf_interleaved)
    if out_dtype is None:
        out_dtype = "f32" if variant == "fp8" else "bf16"
    return MqaInputs(variant, B, N, H, D, int(max_context), q, q_sf, kv, int(page_stride),
                     weights, seq_lens, block_table, out_dtype, name, int(sf_vec_size),
                     bool(kv_sf_interleaved))


# --------------------------------------------------------------------------
# one-head indexer_scores inputs
# --------------------------------------------------------------------------


@dataclasses.dataclass
class IndexerInputs:
    query: np.ndarray  # u16 bf16 bits [rows, 128]
    key_cache: np.ndarray  # u8 [pages, page_stride] (bf16 [64,128] at offset 0)
    page_stride: int
    block_table: np.ndarray  # i32 [requests, W]
    context_lengths: np.ndarray  # i32 [groups]
    requests: np.ndarray  # i32 [groups]
    group_row_offsets: Optional[np.ndarray]  # i32 [groups+1] or None (uniform)
    max_context: int
    name: str = ""
    # NVFP4 inputs: query u8 [rows, 64] packed e2m1 and key pages u8 [64, 64]
    # packed e2m1 at offset 0 of each key_cache page; e4m3 scales per 16 values
    fmt: str = "bf16"
    query_scales: Optional[np.ndarray] = None  # u8 [rows, 8]
    key_scales: Optional[np.ndarray] = None  # u8 [pages, scale_page_stride] ([64, 8] at offset 0)
    scale_page_stride: int = 0

    @property
    def rows(self) -> int:
        return self.query.shape[0]

    @property
    def groups(self) -> int:
        return self.context_lengths.shape[0]

    def row_offsets(self) -> np.ndarray:
        if self.group_row_offsets is not None:
            return self.group_row_offsets
        G = self.rows // self.groups
        return np.arange(self.groups + 1, dtype=np.int32) * G

    def kv_positions(self) -> int:
        return int(np.minimum(np.maximum(self.context_lengths, 0), self.max_context).sum())


def make_indexer_inputs(*, rows=24, num_requests=6, bt_width=64, max_context=4096,
                        group_sizes=None, uniform_group=None, max_len=4096,
                        zero_group=True, seed=2, page_stride=None, head_dim=128,
                        name="", fmt="bf16", scale_page_stride=None) -> IndexerInputs:
    rng = np.random.default_rng(seed)
    if uniform_group is not None:
        assert rows % uniform_group == 0
        sizes = [uniform_group] * (rows // uniform_group)
    elif group_sizes is not None:
        sizes = list(group_sizes)
    else:
        sizes, left = [], rows
        while left > 0:
            g = int(min(int(rng.integers(1, 9)), left))
            sizes.append(g)
            left -= g
    assert sum(sizes) == rows and all(1 <= g <= 8 for g in sizes)
    groups = len(sizes)
    num_pages = num_requests * bt_width
    qs = ks = None
    if fmt == "bf16":
        if page_stride is None:
            page_stride = PAGE * head_dim * 2
        q = encode_bf16(rng.standard_normal((rows, head_dim), dtype=np.float32))
        keys = encode_bf16(rng.standard_normal((num_pages, PAGE, head_dim), dtype=np.float32))
        key_cache = np.zeros((num_pages, page_stride), dtype=np.uint8)
        key_cache[:, : PAGE * head_dim * 2] = keys.view(np.uint8).reshape(num_pages, -1)
    elif fmt == "nvfp4":
        if page_stride is None:
            page_stride = PAGE * head_dim // 2
        if scale_page_stride is None:
            scale_page_stride = PAGE * head_dim // 16
        q, qs = quantize_nvfp4(rng.standard_normal((rows, head_dim), dtype=np.float32))
        kp, kc = quantize_nvfp4(rng.standard_normal((num_pages, PAGE, head_dim),
                                                    dtype=np.float32))
        key_cache = np.zeros((num_pages, page_stride), dtype=np.uint8)
        key_cache[:, : PAGE * head_dim // 2] = kp.reshape(num_pages, -1)
        ks = np.zeros((num_pages, scale_page_stride), dtype=np.uint8)
        ks[:, : PAGE * head_dim // 16] = kc.reshape(num_pages, -1)
    else:
        raise ValueError(fmt)
    block_table = rng.permutation(num_pages).astype(np.int32).reshape(num_requests, bt_width)
    lengths = rng.integers(0, max_len + 1, size=groups).astype(np.int32)
    reqs = rng.integers(0, num_requests, size=groups).astype(np.int32)
    if zero_group:
        zg = int(rng.integers(0, groups))
        lengths[zg] = 0
        reqs[zg] = INT32_MAX  # a 0-length group reads nothing; any value is allowed
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    return IndexerInputs(q, key_cache, int(page_stride), block_table, lengths, reqs,
                         None if uniform_group is not None else offs, int(max_context), name,
                         fmt, qs, ks, int(scale_page_stride or 0))


# --------------------------------------------------------------------------
# block-max proxy score inputs (NVFP4 query and keys)
# --------------------------------------------------------------------------

PROXY_BLOCK = 128  # keys per KV block (the paged K's page)


@dataclasses.dataclass
class ProxyInputs:
    q: np.ndarray            # u8 [total_q, Hq, 64] packed e2m1
    q_scale: np.ndarray      # u8 [total_q * Hq, 8] e4m3, row = token * Hq + head
    k: np.ndarray            # paged: u8 [num_pages, page_stride]; flat: u8 [total_k, Hkv, 64]
    k_scale: np.ndarray      # u8 [rows, 8] e4m3 (paged row (page*Hkv + kvh)*128 + token)
    paged: bool
    page_stride: int         # paged: bytes between pages (>= Hkv * 128 * 64)
    cu_q: np.ndarray         # int32 [B+1]
    cu_k: Optional[np.ndarray]        # flat: int32 [B+1]
    page_table: Optional[np.ndarray]  # paged: int32 [B, width]
    seqused_k: Optional[np.ndarray]   # paged: int32 [B]
    q_global_scale: float
    k_global_scale: float
    num_qo_heads: int
    num_kv_heads: int
    causal: bool
    q_offset: Optional[np.ndarray]    # int32 [B] or None (bottom-right default)
    max_k_tiles: int
    reduce_heads: bool
    name: str = ""

    @property
    def batch(self) -> int:
        return int(self.cu_q.shape[0]) - 1

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.k.shape[0]) if self.paged else 0

    @property
    def out_heads(self) -> int:
        return 1 if self.reduce_heads else self.num_qo_heads

    def key_lengths(self) -> np.ndarray:
        if self.paged:
            L = np.maximum(self.seqused_k.astype(np.int64), 0)
            return np.minimum(L, self.page_table.shape[1] * PROXY_BLOCK)
        return np.maximum(np.diff(self.cu_k.astype(np.int64)), 0)

    def kv_positions(self) -> int:
        """Keys per KV head summed over requests (block-granular reads)."""
        L = self.key_lengths()
        return int(np.sum(np.minimum((L + PROXY_BLOCK - 1) // PROXY_BLOCK, self.max_k_tiles))
                   * PROXY_BLOCK)


def _random_nvfp4_rows(rng, shape_rows, scale_lo=0x30, scale_hi=0x48):
    """Random packed e2m1 rows (64 bytes) and e4m3 scales (8 per row, codes in
    [scale_lo, scale_hi): values about 2^-1 .. 2^2): for sizes too large to
    quantise float data."""
    packed = rng.integers(0, 256, size=tuple(shape_rows) + (64,), dtype=np.uint8)
    scales = rng.integers(scale_lo, scale_hi, size=(int(np.prod(shape_rows)), 8), dtype=np.uint8)
    return packed, scales


def make_proxy_inputs(q_lens, k_lens, *, num_qo_heads=64, num_kv_heads=8, paged=True,
                      causal=True, q_offset=None, max_k_tiles=None, reduce_heads=False,
                      pt_width=None, extra_pages=0, page_stride=None, seed=0,
                      quantize=True, name="") -> ProxyInputs:
    """One block-max proxy score workload.

    q_lens / k_lens: query tokens and keys per request.  Query rows are N(0,1)
    data quantised to NVFP4 with a per-tensor global scale 448*6/amax (the
    inverse is q_global_scale); keys likewise when ``quantize``, else random
    codes (large workloads).  Paged keys take ceil(L/128) pages per request
    from a random permutation; unused page-table entries are -1.
    """
    rng = np.random.default_rng(seed)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    k_lens = np.asarray(k_lens, dtype=np.int64)
    B = int(q_lens.shape[0])
    Hq, Hkv = int(num_qo_heads), int(num_kv_heads)
    cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    total_q = int(cu_q[-1])
    xq = rng.standard_normal((total_q, Hq, 128), dtype=np.float32)
    gq = np.float32(448.0 * 6.0) / np.float32(max(float(np.max(np.abs(xq))), 1e-30))
    q, qs = quantize_nvfp4(xq * gq)
    q_scale = qs.reshape(total_q * Hq, 8)
    q_global = float(np.float32(1.0) / gq)
    kl = np.maximum(k_lens, 0)
    blocks = [int((L + PROXY_BLOCK - 1) // PROXY_BLOCK) for L in kl]
    if max_k_tiles is None:
        max_k_tiles = max(blocks + [1])
    k_global = 1.0
    if paged:
        if pt_width is None:
            pt_width = max(blocks + [1])
        num_pages = max(sum(min(b, pt_width) for b in blocks) + extra_pages, 1)
        if page_stride is None:
            page_stride = Hkv * PROXY_BLOCK * 64
        perm = rng.permutation(num_pages).astype(np.int32)
        page_table = np.full((B, pt_width), -1, dtype=np.int32)
        pos = 0
        for r, T in enumerate(blocks):
            T = min(T, pt_width)
            page_table[r, :T] = perm[pos:pos + T]
            pos += T
        k = np.zeros((num_pages, page_stride), dtype=np.uint8)
        if quantize:
            xk = rng.standard_normal((num_pages, Hkv, PROXY_BLOCK, 128), dtype=np.float32)
            gk = np.float32(448.0 * 6.0) / np.float32(max(float(np.max(np.abs(xk))), 1e-30))
            kp, ksc = quantize_nvfp4(xk * gk)
            k_global = float(np.float32(1.0) / gk)
        else:
            kp, ksc = _random_nvfp4_rows(rng, (num_pages, Hkv, PROXY_BLOCK))
            k_global = 1.0 / 64.0
        k[:, :Hkv * PROXY_BLOCK * 64] = kp.reshape(num_pages, -1)
        k_scale = np.ascontiguousarray(ksc.reshape(num_pages * Hkv * PROXY_BLOCK, 8))
        seqused = k_lens.astype(np.int32)
        cu_k = None
    else:
        cu_k = np.concatenate([[0], np.cumsum(kl)]).astype(np.int32)
        total_k = int(cu_k[-1])
        if quantize:
            xk = rng.standard_normal((total_k, Hkv, 128), dtype=np.float32)
            gk = np.float32(448.0 * 6.0) / np.float32(max(float(np.max(np.abs(xk))), 1e-30))
            k, ksc = quantize_nvfp4(xk * gk)
            k_global = float(np.float32(1.0) / gk)
        else:
            k, ksc = _random_nvfp4_rows(rng, (total_k, Hkv))
            k_global = 1.0 / 64.0
        k_scale = np.ascontiguousarray(ksc.reshape(total_k * Hkv, 8))
        page_table = seqused = None
        page_stride = 0
    if q_offset is not None:
        q_offset = np.asarray(q_offset, dtype=np.int32)
    return ProxyInputs(q, q_scale, k, k_scale, bool(paged), int(page_stride), cu_q, cu_k,
                       page_table, seqused, q_global, k_global, Hq, Hkv, bool(causal), q_offset,
                       int(max_k_tiles), bool(reduce_heads), name)


# --------------------------------------------------------------------------
# named workloads
# --------------------------------------------------------------------------

SEEDS = {"tiny_fp8": 1, "indexer_bf16": 2, "decode_fp8": 3, "verify_fp8": 4, "mxfp4": 5,
         "indexer_nvfp4": 6, "verify_fp8_n8": 7, "verify_fp8_h32": 8, "verify_fp8_bf16": 4,
         "mxfp4_n4": 9, "mxfp4_sf16": 5, "mxfp4_records": 5, "mxfp4_sf16_records": 5,
         "proxy_decode": 10, "proxy_verify": 11, "indexer_bf16_8k": 12, "indexer_nvfp4_8k": 13}

# the MXFP4 scale layouts of the mxfp4 workload: (sf_vec_size, interleaved)
MX_LAYOUT_CONFIGS = {"mxfp4": (32, False), "mxfp4_sf16": (16, False),
                     "mxfp4_records": (32, True), "mxfp4_sf16_records": (16, True)}


def _lens(name, rng):
    if name == "decode_fp8":
        u = rng.uniform(math.log(1024), math.log(32768), size=64)
        return np.rint(np.exp(u)).astype(np.int32)
    if name in ("verify_fp8", "verify_fp8_h32", "verify_fp8_bf16"):
        return rng.integers(4096, 65536 + 1, size=128).astype(np.int32)
    if name == "verify_fp8_n8":
        return rng.integers(4096, 65536 + 1, size=64).astype(np.int32)
    if name in ("mxfp4_n4", "proxy_decode", "proxy_verify") or name in MX_LAYOUT_CONFIGS:
        return rng.integers(16384, 131072 + 1, size=64).astype(np.int32)
    raise KeyError(name)


def make_config(name: str, seed: Optional[int] = None, **overrides):
    """The named workloads.

    tiny_fp8     B=2, next_n=1, seq_lens {37, 200}, 8 pages, block table a
                 permutation of all 8, fp32 out [2, 256]
    indexer_bf16 24 rows in groups of 1..8 over 6 requests, bf16 keys
                 [384, 64, 128], one zero-length group, fp32 scores [24, 4096]
    indexer_nvfp4 the same shapes with NVFP4 query and keys (packed e2m1,
                 e4m3 scale per 16 values)
    decode_fp8   B=64, next_n=1, seq_lens log-uniform in 1K..32K, w ~ N(0, 0.1^2)
    verify_fp8   B=128, next_n=4, seq_lens uniform in 4K..64K, w ~ N(0, 0.1^2)
    mxfp4        B=64, next_n=2, seq_lens uniform in 16K..128K, bf16 out
    verify_fp8_n8  B=64, next_n=8, seq_lens uniform in 4K..64K, w ~ N(0, 0.1^2)
    verify_fp8_h32 B=128, next_n=2, 32 heads x 128, seq_lens uniform in 4K..64K,
                 w ~ N(0, 0.1^2)
    verify_fp8_bf16 verify_fp8 (same seed and lengths) with bf16 out
    mxfp4_n4     B=64, next_n=4, seq_lens uniform in 16K..128K, bf16 out
    mxfp4_sf16, mxfp4_records, mxfp4_sf16_records
                 mxfp4 (same seed and lengths) with one code per 16 values,
                 with each token's codes after its packed bytes, or both
    proxy_decode block-max proxy score: B=64 requests of 1 query token, 64
                 query heads over 8 KV heads (head_dim 128), paged NVFP4 keys,
                 key counts uniform in 16K..128K, causal, 1024 blocks per row
    proxy_verify the same with 4 query tokens per request
    indexer_bf16_8k, indexer_nvfp4_8k
                 8192 query rows in groups of 1..8 over 512 requests of up to
                 4096 keys (64 pages each), context lengths uniform in
                 0..4096, fp32 scores [8192, 4096]
    """
    if seed is None:
        seed = SEEDS[name]
    if name == "tiny_fp8":
        kw = dict(seq_lens=[37, 200], next_n=1, max_context=256, bt_width=4,
                  full_table=True, w_std=1.0)
    elif name in ("indexer_bf16", "indexer_nvfp4"):
        kw = dict(fmt="bf16" if name == "indexer_bf16" else "nvfp4")
        kw.update(overrides)
        return make_indexer_inputs(seed=seed, name=name, **kw)
    elif name in ("indexer_bf16_8k", "indexer_nvfp4_8k"):
        kw = dict(fmt="bf16" if name == "indexer_bf16_8k" else "nvfp4", rows=8192,
                  num_requests=512, bt_width=64, max_context=4096, max_len=4096)
        kw.update(overrides)
        return make_indexer_inputs(seed=seed, name=name, **kw)
    elif name in ("proxy_decode", "proxy_verify"):
        lens = _lens(name, np.random.default_rng(seed + 1000))
        lq = 1 if name == "proxy_decode" else 4
        kw = dict(q_lens=[lq] * len(lens), k_lens=lens, num_qo_heads=64, num_kv_heads=8,
                  paged=True, causal=True, max_k_tiles=1024, pt_width=1024, quantize=False)
        kw.update(overrides)
        return make_proxy_inputs(seed=seed, name=name, **kw)
    elif name in ("decode_fp8", "verify_fp8", "verify_fp8_n8", "verify_fp8_h32",
                  "verify_fp8_bf16", "mxfp4_n4") or name in MX_LAYOUT_CONFIGS:
        lens = _lens(name, np.random.default_rng(seed + 1000))
        if name == "decode_fp8":
            kw = dict(seq_lens=lens, next_n=1, max_context=32768, bt_width=512, w_std=0.1)
        elif name == "verify_fp8":
            kw = dict(seq_lens=lens, next_n=4, max_context=65536, bt_width=1024, w_std=0.1)
        elif name == "verify_fp8_n8":
            kw = dict(seq_lens=lens, next_n=8, max_context=65536, bt_width=1024, w_std=0.1)
        elif name == "verify_fp8_bf16":
            kw = dict(seq_lens=lens, next_n=4, max_context=65536, bt_width=1024, w_std=0.1,
                      out_dtype="bf16")
        elif name == "mxfp4_n4":
            kw = dict(seq_lens=lens, next_n=4, max_context=131072, bt_width=2048, w_std=1.0,
                      variant="mxfp4")
        elif name == "verify_fp8_h32":
            kw = dict(seq_lens=lens, next_n=2, max_context=65536, bt_width=1024, w_std=0.1,
                      num_heads=32)
        else:
            sfv, il = MX_LAYOUT_CONFIGS[name]
            kw = dict(seq_lens=lens, next_n=2, max_context=131072, bt_width=2048, w_std=1.0,
                      variant="mxfp4", sf_vec_size=sfv, kv_sf_interleaved=il)
    else:
        raise KeyError(name)
    kw.update(overrides)
    return make_mqa_inputs(seed=seed, name=name, **kw)
