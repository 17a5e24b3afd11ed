"""CPU oracle for paged MQA logits, one-head indexer scores and the block-max
proxy score (float64).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The GPU product path never imports
this package; the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, float64, its own format
decoders).  This module compiles it with gcc when the shared object is missing
or older than the source, and marshals numpy arrays into it.

Which passage each function follows:
  * ``mqa_logits``        - FlashInfer "flashinfer.attn_scores": the
                            introductory equation, the bullets on the per-head
                            rectifier and on s_p / MXFP4 block scales, and the
                            output-contract note.
  * ``indexer_scores`` / ``indexer_scores_nvfp4`` - FlashInfer
                            "flashinfer.sdsa.indexer_scores": description and
                            parameter list (BF16 inputs; NVFP4 inputs with
                            query_scales / key_scales).
  * ``proxy_score_fp4_for`` / ``proxy_score_fp4_points_for`` - FlashInfer
                            "flashinfer.msa_ops.msa_proxy_score_fp4":
                            description, parameter list and "Returns" (the
                            readings where it defers to an absent page are
                            in oracle.c).
  * ``e4m3``/``e2m1``/``e8m0``/``bf16`` - OCP 8-bit FP and OCP MX v1.0
                            format definitions.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-Wall", "-fopenmp", "-shared", "-fPIC",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
            lib.oracle_mqa_logits.argtypes = [ctypes.c_int, P, P, P, I64, P, P, P, I64,
                                              I32, I32, I32, I32, I32, I32, I32, P, P, P,
                                              ctypes.c_int]
            lib.oracle_mqa_logits_points.argtypes = [ctypes.c_int, P, P, P, I64, P, P, P, I64,
                                                     I32, I32, I32, I32, I32, I32, I32, I64, P,
                                                     P, P, P, P, ctypes.c_int]
            lib.oracle_mqa_written.argtypes = [P, I32, I32, I32, P]
            lib.oracle_indexer_scores.argtypes = [P, I32, I32, P, I64, P, I64, P, P, P, I32, I32,
                                                  P, P, P, ctypes.c_int]
            lib.oracle_indexer_scores_nvfp4.argtypes = [P, P, I32, I32, P, I64, P, I64, P, I64,
                                                        P, P, P, I32, I32, P, P, P, ctypes.c_int]
            D = ctypes.c_double
            proxy = [P, P, I32, I32, I32, P, P, ctypes.c_int, I64, I32, P, P, P, I64, I32, P,
                     I32, D, D, ctypes.c_int, P, I32, ctypes.c_int]
            lib.oracle_proxy_score_fp4.argtypes = proxy + [P, P, ctypes.c_int]
            lib.oracle_proxy_score_fp4_points.argtypes = proxy + [I64, P, P, P, P, P,
                                                                  ctypes.c_int]
            for f in ("oracle_e4m3", "oracle_e2m1", "oracle_e8m0"):
                getattr(lib, f).argtypes = [ctypes.c_uint8]
                getattr(lib, f).restype = ctypes.c_double
            lib.oracle_bf16.argtypes = [ctypes.c_uint16]
            lib.oracle_bf16.restype = ctypes.c_double
            lib.oracle_max_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    return max(1, min(os.cpu_count() or 1, 16))


# ------------------------------------------------------------------ decoders


def e4m3(code: int) -> float:
    return _load().oracle_e4m3(code)


def e2m1(nibble: int) -> float:
    return _load().oracle_e2m1(nibble)


def e8m0(code: int) -> float:
    return _load().oracle_e8m0(code)


def bf16(bits: int) -> float:
    return _load().oracle_bf16(bits)


# ---------------------------------------------------------------- MQA logits


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def mqa_logits(variant, q, q_sf, kv, page_stride, weights, seq_lens, block_table,
               batch, next_n, num_heads, head_dim, max_context, nthreads=None, *,
               sf_vec_size=32, kv_sf_interleaved=False):
    """Dense oracle.  Returns (ref, amag, written), each [batch*next_n, max_context].

    ref     float64 logits where written, NaN elsewhere
    amag    s_p * sum_h |w| * relu(q.k), the magnitude the tolerance scales with
    written bool, the cells the operation writes
    sf_vec_size / kv_sf_interleaved: the MXFP4 scale layout (see oracle.c)
    """
    lib = _load()
    rows = batch * next_n
    ref = np.full((rows, max_context), np.nan)
    amag = np.zeros((rows, max_context))
    written = np.zeros((rows, max_context), dtype=np.uint8)
    q, q_sf, kv = _c(q, np.uint8), _c(q_sf, np.uint8), _c(kv, np.uint8)
    w, sl, bt = _c(weights, np.float32), _c(seq_lens, np.int32), _c(block_table, np.int32)
    rc = lib.oracle_mqa_logits(0 if variant == "fp8" else 1, _ptr(q), _ptr(q_sf), _ptr(kv),
                               int(page_stride), _ptr(w), _ptr(sl), _ptr(bt), int(bt.shape[1]),
                               batch, next_n, num_heads, head_dim, max_context,
                               int(sf_vec_size), int(bool(kv_sf_interleaved)),
                               _ptr(ref), _ptr(amag), _ptr(written),
                               nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_mqa_logits: bad arguments (%d)" % rc)
    return ref, amag, written.astype(bool)


def mqa_logits_points(variant, q, q_sf, kv, page_stride, weights, seq_lens, block_table,
                      batch, next_n, num_heads, head_dim, max_context, rows, cols,
                      nthreads=None, *, sf_vec_size=32, kv_sf_interleaved=False):
    """Oracle at the given (row, column) cells.  Returns (ref, amag, written)."""
    lib = _load()
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    cols = np.ascontiguousarray(cols, dtype=np.int32)
    n = rows.shape[0]
    ref, amag = np.empty(n), np.empty(n)
    written = np.zeros(n, dtype=np.uint8)
    q, q_sf, kv = _c(q, np.uint8), _c(q_sf, np.uint8), _c(kv, np.uint8)
    w, sl, bt = _c(weights, np.float32), _c(seq_lens, np.int32), _c(block_table, np.int32)
    rc = lib.oracle_mqa_logits_points(0 if variant == "fp8" else 1, _ptr(q), _ptr(q_sf),
                                      _ptr(kv), int(page_stride), _ptr(w), _ptr(sl), _ptr(bt),
                                      int(bt.shape[1]), batch, next_n, num_heads, head_dim,
                                      max_context, int(sf_vec_size),
                                      int(bool(kv_sf_interleaved)), n, _ptr(rows), _ptr(cols),
                                      _ptr(ref),
                                      _ptr(amag), _ptr(written), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_mqa_logits_points: bad arguments (%d)" % rc)
    return ref, amag, written.astype(bool)


def mqa_logits_for(inp, nthreads=None):
    """Dense oracle for a ``synth.MqaInputs``."""
    return mqa_logits(inp.variant, inp.q, inp.q_sf, inp.kv, inp.page_stride, inp.weights,
                      inp.seq_lens, inp.block_table, inp.batch, inp.next_n, inp.num_heads,
                      inp.head_dim, inp.max_context, nthreads,
                      sf_vec_size=getattr(inp, "sf_vec_size", 32),
                      kv_sf_interleaved=getattr(inp, "kv_sf_interleaved", False))


def mqa_logits_points_for(inp, rows, cols, nthreads=None):
    return mqa_logits_points(inp.variant, inp.q, inp.q_sf, inp.kv, inp.page_stride,
                             inp.weights, inp.seq_lens, inp.block_table, inp.batch,
                             inp.next_n, inp.num_heads, inp.head_dim, inp.max_context,
                             rows, cols, nthreads,
                             sf_vec_size=getattr(inp, "sf_vec_size", 32),
                             kv_sf_interleaved=getattr(inp, "kv_sf_interleaved", False))


def mqa_written(seq_lens, batch, next_n, max_context):
    """The cells the operation writes, bool [batch*next_n, max_context]."""
    lib = _load()
    sl = _c(seq_lens, np.int32)
    written = np.zeros((batch * next_n, max_context), dtype=np.uint8)
    rc = lib.oracle_mqa_written(_ptr(sl), batch, next_n, max_context, _ptr(written))
    if rc != 0:
        raise ValueError("oracle_mqa_written: bad arguments (%d)" % rc)
    return written.astype(bool)


# ------------------------------------------------------------ indexer scores


def indexer_scores(query, key_cache, page_stride, block_table, context_lengths, requests,
                   row_offsets, max_context, nthreads=None):
    """Dense oracle.  Returns (ref, amag, written), each [rows, max_context];
    amag is sum_d |q_d k_d|."""
    lib = _load()
    q = _c(query, np.uint16)
    rows, D = q.shape
    kc = _c(key_cache, np.uint8)
    bt = _c(block_table, np.int32)
    cl, rq, ro = _c(context_lengths, np.int32), _c(requests, np.int32), _c(row_offsets, np.int32)
    groups = cl.shape[0]
    ref = np.full((rows, max_context), np.nan)
    amag = np.zeros((rows, max_context))
    written = np.zeros((rows, max_context), dtype=np.uint8)
    rc = lib.oracle_indexer_scores(_ptr(q), rows, D, _ptr(kc), int(page_stride), _ptr(bt),
                                   int(bt.shape[1]), _ptr(cl), _ptr(rq), _ptr(ro), groups,
                                   max_context, _ptr(ref), _ptr(amag), _ptr(written),
                                   nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_indexer_scores: bad arguments (%d)" % rc)
    return ref, amag, written.astype(bool)


def indexer_scores_nvfp4(query, query_scales, key_cache, page_stride, key_scales,
                         scale_page_stride, block_table, context_lengths, requests, row_offsets,
                         max_context, nthreads=None):
    """Dense oracle for NVFP4 query and keys (packed e2m1, e4m3 scale per 16
    values).  Returns (ref, amag, written), each [rows, max_context]."""
    lib = _load()
    q = _c(query, np.uint8)
    rows, half = q.shape
    qs = _c(query_scales, np.uint8)
    kc, ks = _c(key_cache, np.uint8), _c(key_scales, np.uint8)
    bt = _c(block_table, np.int32)
    cl, rq, ro = _c(context_lengths, np.int32), _c(requests, np.int32), _c(row_offsets, np.int32)
    groups = cl.shape[0]
    ref = np.full((rows, max_context), np.nan)
    amag = np.zeros((rows, max_context))
    written = np.zeros((rows, max_context), dtype=np.uint8)
    rc = lib.oracle_indexer_scores_nvfp4(_ptr(q), _ptr(qs), rows, 2 * half, _ptr(kc),
                                         int(page_stride), _ptr(ks), int(scale_page_stride),
                                         _ptr(bt), int(bt.shape[1]), _ptr(cl), _ptr(rq), _ptr(ro),
                                         groups, max_context, _ptr(ref), _ptr(amag),
                                         _ptr(written), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_indexer_scores_nvfp4: bad arguments (%d)" % rc)
    return ref, amag, written.astype(bool)


def indexer_scores_for(inp, nthreads=None):
    if getattr(inp, "fmt", "bf16") == "nvfp4":
        return indexer_scores_nvfp4(inp.query, inp.query_scales, inp.key_cache, inp.page_stride,
                                    inp.key_scales, inp.scale_page_stride, inp.block_table,
                                    inp.context_lengths, inp.requests, inp.row_offsets(),
                                    inp.max_context, nthreads)
    return indexer_scores(inp.query, inp.key_cache, inp.page_stride, inp.block_table,
                          inp.context_lengths, inp.requests, inp.row_offsets(),
                          inp.max_context, nthreads)


# ------------------------------------------------------ block-max proxy score


def _proxy_common(inp):
    q, qs = _c(inp.q, np.uint8), _c(inp.q_scale, np.uint8)
    k, ks = _c(inp.k, np.uint8), _c(inp.k_scale, np.uint8)
    cu_q = _c(inp.cu_q, np.int32)
    cu_k = _c(inp.cu_k, np.int32)
    pt = _c(inp.page_table, np.int32)
    su = _c(inp.seqused_k, np.int32)
    qo = _c(inp.q_offset, np.int32)
    keep = (q, qs, k, ks, cu_q, cu_k, pt, su, qo)
    args = [_ptr(q), _ptr(qs), int(q.shape[0]), inp.num_qo_heads, inp.num_kv_heads, _ptr(k),
            _ptr(ks), int(inp.paged), int(inp.page_stride), int(k.shape[0]) if inp.paged else 0,
            _ptr(cu_q), _ptr(cu_k), _ptr(pt), int(pt.shape[1]) if pt is not None else 0,
            int(pt.shape[1]) if pt is not None else 0, _ptr(su), inp.batch,
            float(inp.q_global_scale), float(inp.k_global_scale), int(inp.causal), _ptr(qo),
            int(inp.max_k_tiles), int(inp.reduce_heads)]
    return args, keep


def proxy_score_fp4_for(inp, nthreads=None):
    """Dense oracle of the per-KV-block max proxy score (see oracle.c).
    Returns (ref, amag), each float64 [H_out, max_k_tiles, total_q]; ref is
    -inf where a block has no visible key, NaN for an out-of-range page id."""
    lib = _load()
    args, keep = _proxy_common(inp)
    shape = (inp.out_heads, inp.max_k_tiles, inp.total_q)
    ref = np.empty(shape)
    amag = np.empty(shape)
    rc = lib.oracle_proxy_score_fp4(*args, _ptr(ref), _ptr(amag), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_proxy_score_fp4: bad arguments (%d)" % rc)
    return ref, amag


def proxy_score_fp4_points_for(inp, hs, ts, is_, nthreads=None):
    """The same values at cells (hs[n], ts[n], is_[n])."""
    lib = _load()
    args, keep = _proxy_common(inp)
    hs, ts, is_ = _c(hs, np.int32), _c(ts, np.int32), _c(is_, np.int32)
    ref = np.empty(hs.shape[0])
    amag = np.empty(hs.shape[0])
    rc = lib.oracle_proxy_score_fp4_points(*args, int(hs.shape[0]), _ptr(hs), _ptr(ts), _ptr(is_),
                                           _ptr(ref), _ptr(amag), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_proxy_score_fp4_points: bad arguments (%d)" % rc)
    return ref, amag


def max_threads() -> int:
    return _load().oracle_max_threads()
