"""The Python binding rejects malformed tensors before any library call.

The C ABI receives raw device pointers and cannot check the sizes of the
buffers behind them, so the binding checks every tensor first: dtype, shape
and size, layout, and that it lives on the GPU.  These run on the CPU: every
case must raise ValueError (a valid CPU tensor set is rejected for its
device), so nothing is ever launched."""
import pytest
import torch

B, N, H, D, P, MAXC = 2, 1, 64, 128, 4, 128


@pytest.fixture(scope="module")
def pm():
    import os
    from paged_mqa_logits_02_amd import LIB_PATH
    if not os.path.exists(LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    import paged_mqa_logits_02_amd as m
    return m


def fp8_args(**over):
    a = dict(q=torch.zeros((B, N, H, D), dtype=torch.uint8),
             kv_fused=torch.zeros((P, 64 * (D + 4)), dtype=torch.uint8),
             weights=torch.zeros((B * N, H), dtype=torch.float32),
             seq_lens=torch.zeros(B, dtype=torch.int32),
             block_table=torch.zeros((B, MAXC // 64), dtype=torch.int32),
             out=torch.zeros((B * N, MAXC), dtype=torch.float32))
    a.update(over)
    return a


def mxfp4_args(**over):
    a = dict(q=torch.zeros((B, N, H, D // 2), dtype=torch.uint8),
             q_sf=torch.zeros((B, N, H, D // 32), dtype=torch.uint8),
             kv_fused=torch.zeros((P, 64 * (D // 2 + D // 32)), dtype=torch.uint8),
             weights=torch.zeros((B * N, H), dtype=torch.float32),
             seq_lens=torch.zeros(B, dtype=torch.int32),
             block_table=torch.zeros((B, MAXC // 64), dtype=torch.int32),
             out=torch.zeros((B * N, MAXC), dtype=torch.bfloat16))
    a.update(over)
    return a


def call_fp8(pm, a):
    pm.mqa_logits_fp8(a["q"], a["kv_fused"], a["weights"], a["seq_lens"], a["block_table"],
                      out=a["out"], schedule_meta=a.get("schedule_meta"))


def call_mxfp4(pm, a):
    pm.mqa_logits_mxfp4(a["q"], a["q_sf"], a["kv_fused"], a["weights"], a["seq_lens"],
                        a["block_table"], out=a["out"], sf_vec_size=a.get("sf_vec_size", 32),
                        is_kv_sf_interleaved=a.get("is_kv_sf_interleaved", False))


FP8_BAD = {
    "cpu tensors": {},
    "q bf16": dict(q=torch.zeros((B, N, H, D), dtype=torch.bfloat16)),
    "q 3-D": dict(q=torch.zeros((B, H, D), dtype=torch.uint8)),
    "q not contiguous": dict(q=torch.zeros((B, N, D, H), dtype=torch.uint8).transpose(2, 3)),
    "weights bf16": dict(weights=torch.zeros((B * N, H), dtype=torch.bfloat16)),
    "weights too short": dict(weights=torch.zeros((B * N, H - 1), dtype=torch.float32)),
    "weights not contiguous": dict(weights=torch.zeros((H, B * N), dtype=torch.float32).t()),
    "seq_lens int64": dict(seq_lens=torch.zeros(B, dtype=torch.int64)),
    "seq_lens too short": dict(seq_lens=torch.zeros(B - 1, dtype=torch.int32)),
    "block_table int64": dict(block_table=torch.zeros((B, 2), dtype=torch.int64)),
    "block_table too few rows": dict(block_table=torch.zeros((B - 1, 2), dtype=torch.int32)),
    "kv pages too small": dict(kv_fused=torch.zeros((P, 64 * D), dtype=torch.uint8)),
    "kv float32": dict(kv_fused=torch.zeros((P, 16 * (D + 4)), dtype=torch.float32)),
    "out int32": dict(out=torch.zeros((B * N, MAXC), dtype=torch.int32)),
    "out too few rows": dict(out=torch.zeros((B * N - 1, MAXC), dtype=torch.float32)),
    "schedule int64": dict(schedule_meta=torch.zeros(64, dtype=torch.int64)),
    "schedule too short": dict(schedule_meta=torch.zeros(3, dtype=torch.int32)),
}


@pytest.mark.parametrize("case", sorted(FP8_BAD))
def test_fp8_bad_argument_raises(pm, case):
    with pytest.raises(ValueError):
        call_fp8(pm, fp8_args(**FP8_BAD[case]))


MXFP4_BAD = {
    "cpu tensors": {},
    "q_sf wrong shape": dict(q_sf=torch.zeros((B, N, H, 2), dtype=torch.uint8)),
    "q_sf not contiguous": dict(q_sf=torch.zeros((B, N, D // 32, H), dtype=torch.uint8)
                                .transpose(2, 3)),
    "q rows too long": dict(q=torch.zeros((B, N, H, D), dtype=torch.uint8)),
    "kv pages too small": dict(kv_fused=torch.zeros((P, 64 * D // 2), dtype=torch.uint8)),
    "weights float64": dict(weights=torch.zeros((B * N, H), dtype=torch.float64)),
}


@pytest.mark.parametrize("case", sorted(MXFP4_BAD))
def test_mxfp4_bad_argument_raises(pm, case):
    with pytest.raises(ValueError):
        call_mxfp4(pm, mxfp4_args(**MXFP4_BAD[case]))


# (arguments, message): one code per 16 values needs 8 codes per query row and
# 64 * (64 + 8) bytes per page; other code sizes and flags are refused.
MXFP4_LAYOUT_BAD = {
    "sf_vec_size 8": (dict(sf_vec_size=8), "sf_vec_size"),
    "sf_vec_size 64": (dict(sf_vec_size=64), "sf_vec_size"),
    "interleaved 2": (dict(is_kv_sf_interleaved=2), "is_kv_sf_interleaved"),
    "sf16 with 4 codes a row": (dict(sf_vec_size=16), "q_sf"),
    "sf16 pages of sf32 size": (dict(sf_vec_size=16, q_sf=torch.zeros((B, N, H, 8),
                                                                        dtype=torch.uint8)),
                                "kv_fused"),
}


@pytest.mark.parametrize("case", sorted(MXFP4_LAYOUT_BAD))
def test_mxfp4_bad_layout_raises(pm, case):
    over, msg = MXFP4_LAYOUT_BAD[case]
    with pytest.raises(ValueError, match=msg):
        call_mxfp4(pm, mxfp4_args(**over))


def test_mxfp4_sf16_records_pass_host_checks(pm):
    """A well-formed sf_vec_size 16, interleaved call fails only on the device
    check (CPU tensors here)."""
    a = mxfp4_args(sf_vec_size=16, is_kv_sf_interleaved=True,
                   q_sf=torch.zeros((B, N, H, 8), dtype=torch.uint8),
                   kv_fused=torch.zeros((P, 64 * (D // 2 + D // 16)), dtype=torch.uint8))
    with pytest.raises(ValueError, match="GPU|device|cuda"):
        call_mxfp4(pm, a)


def indexer_args(**over):
    rows, groups = 4, 2
    a = dict(query=torch.zeros((rows, D), dtype=torch.bfloat16),
             key_cache=torch.zeros((P, 64, D), dtype=torch.bfloat16),
             block_table=torch.zeros((groups, MAXC // 64), dtype=torch.int32),
             context_lengths=torch.zeros(groups, dtype=torch.int32),
             requests=torch.zeros(groups, dtype=torch.int32),
             scores=torch.zeros((rows, MAXC), dtype=torch.float32))
    a.update(over)
    return a


INDEXER_BAD = {
    "cpu tensors": {},
    "query float32": dict(query=torch.zeros((4, D), dtype=torch.float32)),
    "keys float16": dict(key_cache=torch.zeros((P, 64, D), dtype=torch.float16)),
    "key pages too small": dict(key_cache=torch.zeros((P, 32, D), dtype=torch.bfloat16)),
    "requests too short": dict(requests=torch.zeros(1, dtype=torch.int32)),
    "lengths int64": dict(context_lengths=torch.zeros(2, dtype=torch.int64)),
    "scores bf16": dict(scores=torch.zeros((4, MAXC), dtype=torch.bfloat16)),
    "scores too few rows": dict(scores=torch.zeros((3, MAXC), dtype=torch.float32)),
    "offsets too short": dict(group_row_offsets=torch.zeros(2, dtype=torch.int32)),
    "nvfp4 without key scales": dict(query=torch.zeros((4, D // 2), dtype=torch.uint8),
                                     query_scales=torch.zeros((4, 8), dtype=torch.uint8)),
    "nvfp4 key scale pages too small": dict(
        query=torch.zeros((4, D // 2), dtype=torch.uint8),
        query_scales=torch.zeros((4, 8), dtype=torch.uint8),
        key_cache=torch.zeros((P, 64, D // 2), dtype=torch.uint8),
        key_scales=torch.zeros((P, 32, 8), dtype=torch.uint8)),
}


@pytest.mark.parametrize("case", sorted(INDEXER_BAD))
def test_indexer_bad_argument_raises(pm, case):
    a = indexer_args(**INDEXER_BAD[case])
    with pytest.raises(ValueError):
        pm.indexer_scores(a["query"], a["key_cache"], a["block_table"], a["context_lengths"],
                          requests=a["requests"], scores=a["scores"],
                          query_scales=a.get("query_scales"), key_scales=a.get("key_scales"),
                          group_row_offsets=a.get("group_row_offsets"))


def test_schedule_bad_argument_raises(pm):
    with pytest.raises(ValueError):
        pm.mqa_logits_schedule(torch.zeros(4, dtype=torch.int64), 1, max_context=128,
                               num_units=8)
    with pytest.raises(ValueError):
        pm.mqa_logits_schedule(torch.zeros(4, dtype=torch.int32), 1, max_context=128,
                               num_units=8)
