"""bench.py's accounting and its one-GPU contract, on the CPU.

The bench line's roofline figure is algorithmic bytes per launch over the
launch duration; these tests pin the per-position byte counts (key bytes, key
scale, one output per query slot), the split of a call into launches over
query slots, the refusal to run at more than one GPU, and the rule that
committed counter traffic is reported only for the kernel sources it was
taken on."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("variant,next_n,out_bytes,expect", [
    ("fp8", 1, 4, 128 + 4 + 4),      # decode: key row, s_p, one fp32 logit
    ("fp8", 4, 4, 128 + 4 + 16),     # verify: four slots
    ("fp8", 4, 2, 128 + 4 + 8),      # verify, bf16 out
    ("mxfp4", 2, 2, 64 + 4 + 4),     # packed e2m1 row, four e8m0 codes, two bf16 logits
    ("mxfp4", 4, 2, 64 + 4 + 8),
])
def test_algorithmic_bytes_per_position(variant, next_n, out_bytes, expect):
    assert bench.algorithmic_bytes_per_position(variant, next_n, out_bytes) == expect


def test_algorithmic_bytes_other_head_dim():
    assert bench.algorithmic_bytes_per_position("fp8", 2, 4, head_dim=256) == 256 + 4 + 8


@pytest.mark.parametrize("variant,next_n,heads,head_dim,slots", [
    ("fp8", 4, 64, 128, [4]),
    ("fp8", 8, 64, 128, [4, 4]),
    ("fp8", 6, 64, 128, [4, 2]),
    ("mxfp4", 5, 64, 128, [4, 1]),
    ("fp8", 2, 32, 128, [2]),          # 32 KB query slice: 8 slots of 32 heads x 128
    ("fp8", 5, 96, 192, [1] * 5),      # 96 heads x 2 planes of 128: one slot per launch
    ("fp8", 7, 20, 80, [7]),           # 20 heads padded to 32, one plane: 8 slots fit
])
def test_launch_slots(variant, next_n, heads, head_dim, slots):
    assert bench.launch_slots(variant, next_n, heads, head_dim) == slots
    assert sum(slots) == next_n


def test_launch_bytes_sum_over_launches():
    # every launch reads the keys again and writes its own slots
    assert bench.launch_bytes_per_position("fp8", 8, 4, 64, 128) == 2 * (132 + 16)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_counter_traffic_only_for_current_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda kernel="mqa_logits": "abc")
    path = prof / "mqa_logits_w_traffic.txt"
    assert bench.counter_traffic("w") is None
    path.write_text("# comment: x\nkernel_source_sha256: abc\ntraffic_bytes_per_launch: 1234\n")
    assert bench.counter_traffic("w") == 1234.0
    path.write_text("kernel_source_sha256: other\ntraffic_bytes_per_launch: 1234\n")
    assert bench.counter_traffic("w") is None


def test_committed_traffic_summaries_name_their_sources():
    """Every committed counter summary records the kernel sources' hash and
    its traffic per launch, so the bench can tell whether it is current."""
    prof = os.path.join(ROOT, "profiles")
    names = [n for n in os.listdir(prof) if n.endswith("_traffic.txt")]
    assert names
    for n in names:
        text = open(os.path.join(prof, n)).read()
        assert "kernel_source_sha256:" in text and "traffic_bytes_per_launch:" in text, n


def test_every_bench_workload_is_a_named_synthetic_config():
    import synth
    for name in bench.WORKLOADS:
        assert name in synth.SEEDS, name
    # the small ones build here; the rest share their code paths
    inp = synth.make_config("tiny_fp8")
    assert inp.batch == 2 and inp.next_n == 1
    ix = synth.make_config("indexer_bf16")
    assert ix.rows == 24
