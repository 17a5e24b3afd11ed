"""Paged MQA logits for AMD Instinct MI355X (gfx950).

A thin binding over the C ABI of ``libpmqa.so`` (declared in
``include/pmqa.h``).  Every function here only marshals torch tensors into
device pointers, sizes and strides and passes torch's current HIP stream; all
computation runs in the library's HIP kernels.  There is no fallback: if the
library is missing or fails to load, importing this package raises.

Operations (FlashInfer documentation pages):
  * ``mqa_logits_fp8`` / ``mqa_logits_mxfp4`` - "flashinfer.attn_scores":
    logits[t, p] = s_p * sum_h w[t, h] * relu(q[t, h] . k_p), rectifier per
    head before the weighted sum, s_p only for FP8, MXFP4 block scales folded
    into q and k; output contract of the page's note.
  * ``indexer_scores`` - "flashinfer.sdsa.indexer_scores": one head, a plain
    dot product per (query row, key) for groups of 1..8 rows; BF16 inputs, or
    NVFP4 inputs with query_scales / key_scales.
  * ``mqa_logits_schedule`` and the helpers - "flashinfer.attn_scores",
    Scheduling and Setup.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpmqa.so")

F32, BF16 = 0, 1
VARIANT_FP8, VARIANT_MXFP4 = 0, 1
PAGE = 64

_STATUS = {0: "PMQA_OK", -1: "PMQA_ERR_NULL", -2: "PMQA_ERR_SHAPE", -3: "PMQA_ERR_UNSUPPORTED",
           -4: "PMQA_ERR_ALIGN", -6: "PMQA_ERR_HIP"}


class PmqaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s" % (where, status_string(status)))


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libpmqa.so is not built (%s); run __graft_entry__.build() or "
                          "python paged_mqa_logits_02_amd/build.py" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    SZ = ctypes.c_size_t
    lib.mqa_logits_fp8.argtypes = [P, P, I64, I32, P, P, P, I64, I32, I32, I32, I32, I32, P, I64,
                                   I32, I32, I32, P, P, SZ, P]
    lib.mqa_logits_mxfp4.argtypes = [P, P, I32, I32, P, I64, I32, P, P, P, I64, I32, I32, I32,
                                     I32, I32, P, I64, I32, I32, P, P, SZ, P]
    lib.mqa_logits_fp8_no_alloc.argtypes = [P, P, I64, I32, P, P, P, I64, I32, I32, I32, I32,
                                            I32, P, I64, I32, I32, I32, P, P]
    lib.mqa_logits_fp8_no_alloc.restype = ctypes.c_int
    lib.mqa_logits_workspace_bytes.argtypes = []
    lib.mqa_logits_workspace_bytes.restype = SZ
    lib.indexer_scores.argtypes = [P, I32, I32, P, I64, I32, P, I64, I32, I32, P, P, I32, P, P,
                                   I64, I32, P]
    lib.indexer_scores_nvfp4.argtypes = [P, P, I32, I32, P, I64, P, I64, I32, P, I64, I32, I32,
                                         P, P, I32, P, P, I64, I32, P]
    F32 = ctypes.c_float
    lib.msa_proxy_score_fp4.argtypes = [P, P, I32, I32, P, P, I32, I64, I32, I64, F32, F32, P, P,
                                        P, I64, I32, P, I32, I32, P, I32, I32, I32, P, P]
    lib.mqa_logits_schedule.argtypes = [P, I32, I32, I32, I32, I32, P, P]
    lib.mqa_logits_schedule_ints.argtypes = [I32]
    lib.mqa_logits_schedule_ints.restype = I64
    lib.mqa_logits_num_units.argtypes = [ctypes.c_int, I32, I32]
    lib.mqa_logits_num_units.restype = I32
    lib.mqa_logits_padded_seq_len.argtypes = [I32, I32, I32]
    lib.mqa_logits_padded_seq_len.restype = I32
    lib.mqa_logits_min_block_table_width.argtypes = [I32, I32, I32]
    lib.mqa_logits_min_block_table_width.restype = I32
    lib.mqa_logits_init.argtypes = [ctypes.c_int]
    lib.mqa_logits_status_string.argtypes = [ctypes.c_int]
    lib.mqa_logits_status_string.restype = ctypes.c_char_p
    for f in ("mqa_logits_fp8", "mqa_logits_mxfp4", "indexer_scores", "mqa_logits_schedule",
              "mqa_logits_init", "msa_proxy_score_fp4"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


_lib = _load()


def library():
    """The loaded ctypes handle of libpmqa.so."""
    return _lib


def status_string(status: int) -> str:
    return _lib.mqa_logits_status_string(int(status)).decode()


def _check(rc: int, where: str):
    if rc != 0:
        raise PmqaError(rc, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# ------------------------------------------------------- argument checks
#
# The C ABI takes raw device pointers and cannot see how large the buffers
# behind them are, so a tensor of the wrong dtype, shape or device would make
# the kernels read or write outside it.  Every tensor is therefore checked
# here before the call: type and dtype, then shape and size, then layout,
# then that it lives on the GPU (all on one device).  A bad argument raises
# ValueError and nothing is launched.

_BYTE_DTYPES = (torch.uint8, torch.int8, torch.float8_e4m3fn)
_I32 = (torch.int32,)


def _need(t, name, dtypes, dims=None):
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a torch.Tensor" % name)
    if t.dtype not in dtypes:
        raise ValueError("%s has dtype %s; expected one of %s" % (
            name, t.dtype, ", ".join(str(d) for d in dtypes)))
    if dims is not None and t.dim() not in ((dims,) if isinstance(dims, int) else dims):
        raise ValueError("%s has %d dimensions; expected %s" % (name, t.dim(), dims))
    return t


def _need_numel(t, name, n):
    if t.numel() < n:
        raise ValueError("%s has %d elements; at least %d are read" % (name, t.numel(), n))


def _need_contiguous(t, name):
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _need_device(tensors):
    """Every tensor on the same GPU; returns that device."""
    dev = None
    for name, t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("%s is on %s; every tensor must be on the GPU" % (name, t.device))
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("%s is on %s, the other tensors on %s" % (name, t.device, dev))
    return dev


def _need_page_bytes(t, name, min_bytes):
    """A paged cache: pages along dim 0, each page's bytes contiguous and at
    least min_bytes long."""
    if t.dim() < 2:
        raise ValueError("%s needs a page dimension" % name)
    per_page = t[0].numel() * t.element_size()
    if per_page < min_bytes:
        raise ValueError("%s holds %d bytes per page; a page needs %d" % (name, per_page,
                                                                           min_bytes))
    if not t[0].is_contiguous():
        raise ValueError("%s: page contents must be contiguous" % name)


def _need_rows(t, name, rows, cols):
    """A 2-D tensor whose first `rows` rows of `cols` elements are read or written."""
    if t.dim() != 2:
        raise ValueError("%s must be 2-D" % name)
    if t.shape[0] < rows or t.shape[1] < cols:
        raise ValueError("%s has shape %s; needs at least [%d, %d]" % (name, tuple(t.shape),
                                                                       rows, cols))
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("%s must have contiguous rows" % name)


def _check_schedule(schedule_meta):
    if schedule_meta is None:
        return
    _need(schedule_meta, "schedule_meta", _I32, 1)
    _need_numel(schedule_meta, "schedule_meta", schedule_ints(1))
    _need_contiguous(schedule_meta, "schedule_meta")


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _u8(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.uint8) if t.dtype != torch.uint8 and t.element_size() == 1 else t


def _rows_of(t: torch.Tensor):
    """(row stride in elements, row width) of a 2-D tensor whose rows are contiguous."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError("expected a 2-D tensor with contiguous rows")
    return t.stride(0), t.shape[1]


def _pages(t: torch.Tensor):
    """(page stride in bytes, number of pages) of a paged cache.

    Accepts [pages, bytes] uint8 (pages may be a strided view) or any tensor
    whose first dimension is the page index and whose page contents are
    contiguous."""
    if t.dim() < 2:
        raise ValueError("a paged cache needs a page dimension")
    inner = t[0]
    if not inner.is_contiguous():
        raise ValueError("page contents must be contiguous")
    return t.stride(0) * t.element_size(), t.shape[0]


# ---------------------------------------------------------------- helpers


def init(device=None) -> None:
    dev = torch.cuda.current_device() if device is None else int(device)
    _check(_lib.mqa_logits_init(dev), "mqa_logits_init")


def num_units(next_n: int, variant: int = VARIANT_FP8, device=None) -> int:
    dev = torch.cuda.current_device() if device is None else int(device)
    n = _lib.mqa_logits_num_units(dev, next_n, variant)
    _check(min(n, 0), "mqa_logits_num_units")
    return n


def padded_seq_len(seq_len: int, next_n: int = 1, variant: int = VARIANT_FP8) -> int:
    return _lib.mqa_logits_padded_seq_len(seq_len, next_n, variant)


def min_block_table_width(max_seq_len: int, next_n: int = 1, variant: int = VARIANT_FP8) -> int:
    return _lib.mqa_logits_min_block_table_width(max_seq_len, next_n, variant)


def schedule_ints(num_units_: int) -> int:
    return int(_lib.mqa_logits_schedule_ints(num_units_))


def mqa_logits_schedule(seq_lens: torch.Tensor, next_n: int, variant: int = VARIANT_FP8, *,
                        max_context: int, num_units: int = 0, out: torch.Tensor = None,
                        stream=None) -> torch.Tensor:
    """Builds the opaque work split on the GPU (int32 tensor).  Valid only
    while seq_lens is unchanged; pass the same next_n/variant/max_context to
    the logits call."""
    out, args = _schedule_args(seq_lens, next_n, variant, max_context, num_units, out, stream)
    _check(_lib.mqa_logits_schedule(*args), "mqa_logits_schedule")
    return out


def _schedule_args(seq_lens, next_n, variant, max_context, num_units_, out, stream):
    _need(seq_lens, "seq_lens", _I32, 1)
    _need_contiguous(seq_lens, "seq_lens")
    if out is not None:
        _need(out, "out", _I32, 1)
        _need_contiguous(out, "out")
    _need_device([("seq_lens", seq_lens), ("out", out)])
    if num_units_ == 0:
        num_units_ = num_units(next_n, variant, seq_lens.device.index)
    n = schedule_ints(num_units_)
    if n < 0:
        raise PmqaError(-2, "mqa_logits_schedule")
    if out is None:
        out = torch.empty(n, dtype=torch.int32, device=seq_lens.device)
    elif out.numel() < n or out.dtype != torch.int32:
        raise ValueError("schedule buffer too small")
    return out, (_ptr(seq_lens), seq_lens.shape[0], next_n, variant, max_context, num_units_,
                 _ptr(out), _stream(stream, seq_lens.device))


def prepare_mqa_logits_schedule(seq_lens: torch.Tensor, next_n: int, variant: int = VARIANT_FP8,
                                *, max_context: int, num_units: int = 0,
                                out: torch.Tensor = None, stream=None):
    """mqa_logits_schedule with its arguments marshalled once; returns a PreparedCall."""
    out, args = _schedule_args(seq_lens, next_n, variant, max_context, num_units, out, stream)
    return PreparedCall(_lib.mqa_logits_schedule, args, "mqa_logits_schedule", out, (seq_lens,))


# ---------------------------------------------------------------- operations


def _out_for(out, rows, max_context, dtype, device):
    if out is None:
        return torch.empty((rows, max_context), dtype=dtype, device=device)
    return out


def _dtype_code(dtype):
    if dtype == torch.float32:
        return F32
    if dtype == torch.bfloat16:
        return BF16
    raise ValueError("unsupported output dtype %s" % dtype)


def _check_mqa(q, q_sf, kv_fused, weights, seq_lens, block_table, out, schedule_meta,
               page_min_bytes, q_row_bytes):
    """Checks shared by both variants; q [B, N, H, q_row_bytes] bytes."""
    B, N, H = q.shape[:3]
    _need_contiguous(q, "q")
    if q.shape[3] * q.element_size() != q_row_bytes:
        raise ValueError("q rows hold %d bytes; expected %d" % (q.shape[3] * q.element_size(),
                                                               q_row_bytes))
    _need(kv_fused, "kv_fused", _BYTE_DTYPES)
    _need_page_bytes(kv_fused, "kv_fused", page_min_bytes)
    _need(weights, "weights", (torch.float32,))
    _need_numel(weights, "weights", B * N * H)
    _need_contiguous(weights, "weights")
    _need(seq_lens, "seq_lens", _I32, 1)
    _need_numel(seq_lens, "seq_lens", B)
    _need_contiguous(seq_lens, "seq_lens")
    _need(block_table, "block_table", _I32, 2)
    if block_table.shape[0] < B:
        raise ValueError("block_table has %d rows; batch is %d" % (block_table.shape[0], B))
    if out is not None:
        _need(out, "out", (torch.float32, torch.bfloat16), 2)
    _check_schedule(schedule_meta)
    return _need_device([("q", q), ("q_sf", q_sf), ("kv_fused", kv_fused),
                         ("weights", weights), ("seq_lens", seq_lens),
                         ("block_table", block_table), ("out", out),
                         ("schedule_meta", schedule_meta)])


def _workspace_args(workspace, device):
    """(pointer, bytes) of an optional workspace tensor (see workspace())."""
    if workspace is None:
        return None, 0
    if not isinstance(workspace, torch.Tensor):
        raise ValueError("workspace must be a torch.Tensor")
    _need_contiguous(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    if nbytes < workspace_bytes():
        raise ValueError("workspace holds %d bytes; %d are needed" % (nbytes, workspace_bytes()))
    if not workspace.is_cuda or workspace.device != device:
        raise ValueError("workspace is on %s; the other tensors on %s" % (workspace.device, device))
    return _ptr(workspace), nbytes


def workspace_bytes() -> int:
    """Bytes of the optional work-counter workspace of the logits calls."""
    return int(_lib.mqa_logits_workspace_bytes())


def workspace(device=None) -> torch.Tensor:
    """A zero-filled workspace for mqa_logits_fp8 / mqa_logits_mxfp4 (workspace=):
    every completed call leaves it zero-filled, so one allocation serves any
    number of calls that do not run at the same time."""
    if device is None:
        device = torch.device("cuda", torch.cuda.current_device())
    return torch.zeros(workspace_bytes(), dtype=torch.uint8, device=device)


def _fp8_args(q, kv_fused, weights, seq_lens, block_table, next_n, max_context, out,
              schedule_meta, output_dtype, acc_dtype, stream, workspace=None):
    _need(q, "q", _BYTE_DTYPES, 4)
    B, N, H, D = q.shape
    if next_n is not None and next_n != N:
        raise ValueError("next_n does not match q")
    _check_mqa(q, None, kv_fused, weights, seq_lens, block_table, out, schedule_meta,
               PAGE * (D + 4), D)
    bt_stride, bt_width = _rows_of(block_table)
    if max_context is None:
        max_context = out.shape[1] if out is not None else bt_width * PAGE
    out = _out_for(out, B * N, max_context, output_dtype, q.device)
    _need_rows(out, "out", B * N, max_context)
    ors, _ = _rows_of(out)
    ps, npages = _pages(kv_fused)
    acc = _dtype_code(acc_dtype) if acc_dtype in (torch.float32, torch.bfloat16) else 99
    wp, wb = _workspace_args(workspace, q.device)
    return out, (_ptr(q), _ptr(kv_fused), ps, npages, _ptr(weights), _ptr(seq_lens),
                 _ptr(block_table), bt_stride, bt_width, B, N, H, D, _ptr(out), ors, max_context,
                 _dtype_code(out.dtype), acc, _ptr(schedule_meta), wp, wb,
                 _stream(stream, q.device))


def mqa_logits_fp8(q, kv_fused, weights, seq_lens, block_table, next_n=None, *,
                   max_context=None, out=None, schedule_meta=None,
                   output_dtype=torch.float32, acc_dtype=torch.float32, stream=None,
                   workspace=None):
    """FP8 paged MQA logits; returns ``out`` [batch*next_n, max_context].

    q [batch, next_n, heads, head_dim] e4m3 (uint8 or float8_e4m3fn; heads
    1..128, head_dim a multiple of 16 up to 256, next_n 1..8); kv_fused
    [pages, page_bytes] uint8 (a strided view is fine); weights
    [batch*next_n, heads] fp32; seq_lens [batch] int32; block_table
    [batch, width] int32.  Columns at or beyond ceil(seq_len/64)*64 and rows
    of empty requests are not written (out=None allocates uninitialised
    memory).  workspace: None or workspace(), a work counter for the in-call
    split (the result does not depend on it)."""
    out, args = _fp8_args(q, kv_fused, weights, seq_lens, block_table, next_n, max_context, out,
                          schedule_meta, output_dtype, acc_dtype, stream, workspace)
    _check(_lib.mqa_logits_fp8(*args), "mqa_logits_fp8")
    return out


def mqa_logits_fp8_no_alloc(q, kv_fused, weights, seq_lens, block_table, next_n=None, *,
                            max_context=None, out=None, schedule_meta=None,
                            output_dtype=torch.float32, acc_dtype=torch.float32, stream=None):
    """mqa_logits_fp8 through the entry point that allocates nothing: its work
    counters are the library's per-GPU array (calls that overlap on one GPU
    race on it).  Pass ``out``: out=None allocates it here, in the binding."""
    out, args = _fp8_args(q, kv_fused, weights, seq_lens, block_table, next_n, max_context, out,
                          schedule_meta, output_dtype, acc_dtype, stream)
    args = args[:19] + args[21:]  # no workspace pointer and size
    _check(_lib.mqa_logits_fp8_no_alloc(*args), "mqa_logits_fp8_no_alloc")
    return out


def _mxfp4_args(q, q_sf, kv_fused, weights, seq_lens, block_table, next_n, sf_vec_size,
                is_kv_sf_interleaved, max_context, out, schedule_meta, output_dtype, stream,
                workspace=None):
    _need(q, "q", (torch.uint8, torch.int8), 4)
    B, N, H, Dh = q.shape
    if next_n is not None and next_n != N:
        raise ValueError("next_n does not match q")
    if sf_vec_size not in (16, 32):
        raise ValueError("sf_vec_size must be 16 or 32, got %r" % (sf_vec_size,))
    if is_kv_sf_interleaved not in (0, 1, False, True):
        raise ValueError("is_kv_sf_interleaved must be a bool, got %r" % (is_kv_sf_interleaved,))
    _need(q_sf, "q_sf", (torch.uint8, torch.int8, torch.float8_e8m0fnu), 4)
    if tuple(q_sf.shape[:3]) != (B, N, H) or q_sf.shape[3] * sf_vec_size != 2 * Dh:
        raise ValueError("q_sf has shape %s; expected [%d, %d, %d, %d]" % (
            tuple(q_sf.shape), B, N, H, 2 * Dh // sf_vec_size))
    _need_contiguous(q_sf, "q_sf")
    _check_mqa(q, q_sf, kv_fused, weights, seq_lens, block_table, out, schedule_meta,
               PAGE * (Dh + 2 * Dh // sf_vec_size), Dh)
    bt_stride, bt_width = _rows_of(block_table)
    if max_context is None:
        max_context = out.shape[1] if out is not None else bt_width * PAGE
    out = _out_for(out, B * N, max_context, output_dtype, q.device)
    _need_rows(out, "out", B * N, max_context)
    ors, _ = _rows_of(out)
    ps, npages = _pages(kv_fused)
    wp, wb = _workspace_args(workspace, q.device)
    return out, (_ptr(q), _ptr(q_sf), sf_vec_size, int(is_kv_sf_interleaved), _ptr(kv_fused), ps,
                 npages, _ptr(weights), _ptr(seq_lens), _ptr(block_table), bt_stride, bt_width,
                 B, N, H, Dh * 2, _ptr(out), ors, max_context, _dtype_code(out.dtype),
                 _ptr(schedule_meta), wp, wb, _stream(stream, q.device))


def mqa_logits_mxfp4(q, q_sf, kv_fused, weights, seq_lens, block_table, next_n=None, *,
                     sf_vec_size=32, is_kv_sf_interleaved=False, max_context=None, out=None,
                     schedule_meta=None, output_dtype=torch.bfloat16, stream=None,
                     workspace=None):
    """MXFP4 paged MQA logits; returns ``out`` [batch*next_n, max_context].

    q [batch, next_n, 64, 64] packed e2m1 uint8; q_sf [batch, next_n, 64,
    128 // sf_vec_size] e8m0 uint8 (sf_vec_size 32 or 16 values per code);
    kv_fused [pages, page_bytes] uint8.  A page holds 64 tokens: with
    is_kv_sf_interleaved False, 64x64 packed key bytes then 64 x (128 //
    sf_vec_size) e8m0 codes; with True, 64 records of a token's 64 packed
    bytes followed by its codes."""
    out, args = _mxfp4_args(q, q_sf, kv_fused, weights, seq_lens, block_table, next_n,
                            sf_vec_size, is_kv_sf_interleaved, max_context, out, schedule_meta,
                            output_dtype, stream, workspace)
    _check(_lib.mqa_logits_mxfp4(*args), "mqa_logits_mxfp4")
    return out


class PreparedCall:
    """One library call with its arguments marshalled once (device pointers,
    sizes, stream).  Calling it enqueues the same call again on the same
    stream; the tensors it was prepared from are kept alive and must keep
    their storage.  For launch-rate-bound callers (short calls issued from a
    host loop)."""

    def __init__(self, fn, args, where, out, keep):
        self._fn, self._args, self._where, self.out = fn, args, where, out
        self._keep = keep  # the tensors whose device pointers are in args

    def __call__(self):
        rc = self._fn(*self._args)
        if rc != 0:
            raise PmqaError(rc, self._where)
        return self.out


def prepare_mqa_logits_fp8(q, kv_fused, weights, seq_lens, block_table, next_n=None, *,
                           max_context=None, out=None, schedule_meta=None,
                           output_dtype=torch.float32, acc_dtype=torch.float32, stream=None,
                           workspace=None):
    """mqa_logits_fp8 with its arguments marshalled once; returns a PreparedCall."""
    out, args = _fp8_args(q, kv_fused, weights, seq_lens, block_table, next_n, max_context, out,
                          schedule_meta, output_dtype, acc_dtype, stream, workspace)
    return PreparedCall(_lib.mqa_logits_fp8, args, "mqa_logits_fp8", out,
                        (q, kv_fused, weights, seq_lens, block_table, schedule_meta, workspace))


def prepare_mqa_logits_mxfp4(q, q_sf, kv_fused, weights, seq_lens, block_table, next_n=None, *,
                             sf_vec_size=32, is_kv_sf_interleaved=False, max_context=None,
                             out=None, schedule_meta=None, output_dtype=torch.bfloat16,
                             stream=None, workspace=None):
    """mqa_logits_mxfp4 with its arguments marshalled once; returns a PreparedCall."""
    out, args = _mxfp4_args(q, q_sf, kv_fused, weights, seq_lens, block_table, next_n,
                            sf_vec_size, is_kv_sf_interleaved, max_context, out, schedule_meta,
                            output_dtype, stream, workspace)
    return PreparedCall(_lib.mqa_logits_mxfp4, args, "mqa_logits_mxfp4", out,
                        (q, q_sf, kv_fused, weights, seq_lens, block_table, schedule_meta,
                         workspace))


def indexer_scores(query, key_cache, block_table, context_lengths, *, requests, scores,
                   query_scales=None, key_scales=None, group_row_offsets=None, stream=None):
    """One-head indexer scores into ``scores`` [rows, max_context] fp32.

    BF16: query [rows, 128] bf16; key_cache [pages, 64, 128] bf16 or
    [pages, bytes] uint8 (pages may be strided views).
    NVFP4 (query_scales and key_scales given): query uint8 [rows, 64] packed
    e2m1, query_scales e4m3 [rows, 8]; key_cache uint8 [pages, 64, 64] (or
    [pages, bytes]), key_scales e4m3 [pages, 64, 8] (or [pages, bytes]), each
    paged by its own first-dimension stride.
    block_table [requests, width] int32; context_lengths / requests [groups]
    int32; group_row_offsets optional [groups+1] int32 (None: rows/groups
    rows per group)."""
    fn, args, where = _indexer_args(query, key_cache, block_table, context_lengths, requests,
                                    scores, query_scales, key_scales, group_row_offsets, stream)
    _check(fn(*args), where)
    return scores


def _check_indexer(query, key_cache, block_table, context_lengths, requests, scores,
                   query_scales, key_scales, group_row_offsets):
    nvfp4 = query_scales is not None or key_scales is not None
    if nvfp4:
        _need(query, "query", (torch.uint8, torch.int8), 2)
        if query_scales is None or key_scales is None:
            raise ValueError("NVFP4 inputs need both query_scales and key_scales")
        _need(query_scales, "query_scales", _BYTE_DTYPES)
        rows = query.shape[0]
        _need_numel(query_scales, "query_scales", rows * query.shape[1] // 8)
        _need_contiguous(query_scales, "query_scales")
        _need(key_cache, "key_cache", _BYTE_DTYPES)
        _need_page_bytes(key_cache, "key_cache", PAGE * query.shape[1])
        _need(key_scales, "key_scales", _BYTE_DTYPES)
        _need_page_bytes(key_scales, "key_scales", PAGE * query.shape[1] // 8)
    else:
        _need(query, "query", (torch.bfloat16,), 2)
        rows = query.shape[0]
        _need(key_cache, "key_cache", (torch.bfloat16,) + _BYTE_DTYPES)
        _need_page_bytes(key_cache, "key_cache", PAGE * query.shape[1] * 2)
    _need_contiguous(query, "query")
    _need(block_table, "block_table", _I32, 2)
    _need(context_lengths, "context_lengths", _I32, 1)
    _need_contiguous(context_lengths, "context_lengths")
    groups = context_lengths.shape[0]
    _need(requests, "requests", _I32, 1)
    _need_numel(requests, "requests", groups)
    _need_contiguous(requests, "requests")
    if group_row_offsets is not None:
        _need(group_row_offsets, "group_row_offsets", _I32, 1)
        _need_numel(group_row_offsets, "group_row_offsets", groups + 1)
        _need_contiguous(group_row_offsets, "group_row_offsets")
    _need(scores, "scores", (torch.float32,), 2)
    _need_rows(scores, "scores", rows, scores.shape[1])
    _need_device([("query", query), ("key_cache", key_cache), ("block_table", block_table),
                  ("context_lengths", context_lengths), ("requests", requests),
                  ("scores", scores), ("query_scales", query_scales),
                  ("key_scales", key_scales), ("group_row_offsets", group_row_offsets)])


def _indexer_args(query, key_cache, block_table, context_lengths, requests, scores,
                  query_scales, key_scales, group_row_offsets, stream):
    _check_indexer(query, key_cache, block_table, context_lengths, requests, scores,
                   query_scales, key_scales, group_row_offsets)
    bt_stride, bt_width = _rows_of(block_table)
    srs, max_context = _rows_of(scores)
    ps, npages = _pages(key_cache)
    common = (_ptr(block_table), bt_stride, bt_width, block_table.shape[0],
              _ptr(context_lengths), _ptr(requests), context_lengths.shape[0],
              _ptr(group_row_offsets), _ptr(scores), srs, max_context,
              _stream(stream, query.device))
    if query_scales is None and key_scales is None:
        rows, D = query.shape
        return (_lib.indexer_scores, (_ptr(query), rows, D, _ptr(key_cache), ps, npages) + common,
                "indexer_scores")
    if query_scales is None or key_scales is None:
        raise ValueError("NVFP4 inputs need both query_scales and key_scales")
    rows, half = query.shape
    sps, _ = _pages(key_scales)
    return (_lib.indexer_scores_nvfp4,
            (_ptr(query), _ptr(query_scales), rows, 2 * half, _ptr(key_cache), ps,
             _ptr(key_scales), sps, npages) + common, "indexer_scores_nvfp4")


def _proxy_args(q_fp4, k_fp4, q_scale, k_scale, q_global_scale, k_global_scale, cu_seqlens_q,
                cu_seqlens_k, page_table, seqused_k, causal, max_seqlen_q, max_k_tiles, output,
                reduce_heads, q_offset, stream):
    _need(q_fp4, "q_fp4", (torch.uint8, torch.int8), 3)
    _need_contiguous(q_fp4, "q_fp4")
    total_q, hq, half = q_fp4.shape
    if half != 64:
        raise ValueError("q_fp4 rows hold %d bytes; head_dim 128 needs 64" % half)
    _need(q_scale, "q_scale", _BYTE_DTYPES)
    _need_numel(q_scale, "q_scale", total_q * hq * 8)
    _need_contiguous(q_scale, "q_scale")
    _need(k_fp4, "k_fp4", (torch.uint8, torch.int8))
    _need(k_scale, "k_scale", _BYTE_DTYPES)
    _need_contiguous(k_scale, "k_scale")
    _need(cu_seqlens_q, "cu_seqlens_q", _I32, 1)
    _need_contiguous(cu_seqlens_q, "cu_seqlens_q")
    B = cu_seqlens_q.shape[0] - 1
    if B < 0:
        raise ValueError("cu_seqlens_q needs batch + 1 entries")
    paged = page_table is not None
    if paged:
        if k_fp4.dim() != 4 or tuple(k_fp4.shape[2:]) != (128, 64):
            raise ValueError("paged k_fp4 must be [num_pages, num_kv_heads, 128, 64]; got %s"
                             % (tuple(k_fp4.shape),))
        if not k_fp4[0].is_contiguous():
            raise ValueError("k_fp4: page contents must be contiguous")
        num_pages, hkv = k_fp4.shape[:2]
        page_stride = k_fp4.stride(0)
        _need_numel(k_scale, "k_scale", num_pages * hkv * 128 * 8)
        _need(page_table, "page_table", _I32, 2)
        if page_table.shape[0] < B:
            raise ValueError("page_table has %d rows; batch is %d" % (page_table.shape[0], B))
        pt_stride, pt_width = _rows_of(page_table)
        if seqused_k is None:
            raise ValueError("paged keys need seqused_k")
        _need(seqused_k, "seqused_k", _I32, 1)
        _need_numel(seqused_k, "seqused_k", B)
        _need_contiguous(seqused_k, "seqused_k")
        total_k = 0
        if max_k_tiles is None:
            max_k_tiles = pt_width
    else:
        if k_fp4.dim() != 3 or k_fp4.shape[2] != 64:
            raise ValueError("flat k_fp4 must be [total_k, num_kv_heads, 64]; got %s"
                             % (tuple(k_fp4.shape),))
        _need_contiguous(k_fp4, "k_fp4")
        total_k, hkv = k_fp4.shape[:2]
        _need_numel(k_scale, "k_scale", total_k * hkv * 8)
        if cu_seqlens_k is None:
            raise ValueError("flat keys need cu_seqlens_k")
        _need(cu_seqlens_k, "cu_seqlens_k", _I32, 1)
        _need_numel(cu_seqlens_k, "cu_seqlens_k", B + 1)
        _need_contiguous(cu_seqlens_k, "cu_seqlens_k")
        num_pages = page_stride = pt_stride = pt_width = 0
        if max_k_tiles is None:
            max_k_tiles = (total_k + 127) // 128
    if hq % hkv != 0:
        raise ValueError("num_qo_heads (%d) must be a multiple of num_kv_heads (%d)" % (hq, hkv))
    dev = _need_device([("q_fp4", q_fp4), ("k_fp4", k_fp4), ("q_scale", q_scale),
                        ("k_scale", k_scale), ("cu_seqlens_q", cu_seqlens_q),
                        ("cu_seqlens_k", cu_seqlens_k if not paged else None),
                        ("page_table", page_table), ("seqused_k", seqused_k if paged else None),
                        ("output", output),
                        ("q_offset", q_offset if isinstance(q_offset, torch.Tensor) else None)])
    if q_offset is not None and not isinstance(q_offset, torch.Tensor):
        q_offset = torch.full((max(B, 1),), int(q_offset), dtype=torch.int32, device=dev)
    if q_offset is not None:
        _need(q_offset, "q_offset", _I32, 1)
        _need_numel(q_offset, "q_offset", B)
        _need_contiguous(q_offset, "q_offset")
    hout = 1 if reduce_heads else hq
    if output is None:
        output = torch.empty((hout, max_k_tiles, total_q), dtype=torch.float32, device=dev)
    _need(output, "output", (torch.float32,), 3)
    _need_contiguous(output, "output")
    if tuple(output.shape) != (hout, max_k_tiles, total_q):
        raise ValueError("output has shape %s; expected %s" % (tuple(output.shape),
                                                                (hout, max_k_tiles, total_q)))
    args = (_ptr(q_fp4), _ptr(q_scale), total_q, hq, _ptr(k_fp4), _ptr(k_scale), hkv,
            page_stride, num_pages, total_k, float(q_global_scale), float(k_global_scale),
            _ptr(cu_seqlens_q), None if paged else _ptr(cu_seqlens_k),
            _ptr(page_table), pt_stride, pt_width, _ptr(seqused_k) if paged else None, B,
            int(bool(causal)), _ptr(q_offset), int(max_seqlen_q or 0), int(max_k_tiles),
            int(bool(reduce_heads)), _ptr(output), _stream(stream, dev))
    return output, args, (q_fp4, k_fp4, q_scale, k_scale, cu_seqlens_q, cu_seqlens_k,
                          page_table, seqused_k, q_offset)


def msa_proxy_score_fp4(q_fp4, k_fp4, q_scale, k_scale, q_global_scale, k_global_scale,
                        cu_seqlens_q, cu_seqlens_k=None, *, page_table=None, seqused_k=None,
                        causal=True, max_seqlen_q=None, max_k_tiles=None, output=None,
                        reduce_heads=False, q_offset=None, stream=None):
    """Per-KV-block max of the causally masked Q K^T logits with NVFP4 inputs.

    q_fp4 uint8 [total_q, Hq, 64] packed e2m1; q_scale e4m3 [total_q*Hq, 8];
    keys paged (k_fp4 [num_pages, Hkv, 128, 64], k_scale rows
    (page*Hkv + kv_head)*128 + token, with page_table [batch, width] and
    seqused_k [batch]) or flat (k_fp4 [total_k, Hkv, 64], k_scale rows
    token*Hkv + kv_head, with cu_seqlens_k [batch+1]).  q_offset: None (Lk -
    Lq per request), an int, or an int32 tensor [batch].  Returns float32
    [Hq or 1, max_k_tiles, total_q]; max_k_tiles defaults to the page-table
    width (paged) or ceil(total_k / 128) (flat)."""
    output, args, _ = _proxy_args(q_fp4, k_fp4, q_scale, k_scale, q_global_scale,
                                  k_global_scale, cu_seqlens_q, cu_seqlens_k, page_table,
                                  seqused_k, causal, max_seqlen_q, max_k_tiles, output,
                                  reduce_heads, q_offset, stream)
    _check(_lib.msa_proxy_score_fp4(*args), "msa_proxy_score_fp4")
    return output


def prepare_msa_proxy_score_fp4(q_fp4, k_fp4, q_scale, k_scale, q_global_scale, k_global_scale,
                                cu_seqlens_q, cu_seqlens_k=None, *, page_table=None,
                                seqused_k=None, causal=True, max_seqlen_q=None,
                                max_k_tiles=None, output=None, reduce_heads=False, q_offset=None,
                                stream=None):
    """msa_proxy_score_fp4 with its arguments marshalled once; returns a PreparedCall."""
    output, args, keep = _proxy_args(q_fp4, k_fp4, q_scale, k_scale, q_global_scale,
                                     k_global_scale, cu_seqlens_q, cu_seqlens_k, page_table,
                                     seqused_k, causal, max_seqlen_q, max_k_tiles, output,
                                     reduce_heads, q_offset, stream)
    return PreparedCall(_lib.msa_proxy_score_fp4, args, "msa_proxy_score_fp4", output, keep)


def prepare_indexer_scores(query, key_cache, block_table, context_lengths, *, requests, scores,
                           query_scales=None, key_scales=None, group_row_offsets=None,
                           stream=None):
    """indexer_scores with its arguments marshalled once; returns a PreparedCall."""
    fn, args, where = _indexer_args(query, key_cache, block_table, context_lengths, requests,
                                    scores, query_scales, key_scales, group_row_offsets, stream)
    return PreparedCall(fn, args, where, scores,
                        (query, key_cache, block_table, context_lengths, requests,
                         query_scales, key_scales, group_row_offsets))
