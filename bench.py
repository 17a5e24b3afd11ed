"""Benchmark: FP8 paged MQA logits (H=64, d=128; other workloads by name) on one MI355X.

One step = one whole call of the hot path on the synthetic workload: the
work split (computed on the GPU, either inside the logits kernel or by the
schedule kernel), then the logits kernel (page gather, FP8 MFMA, per-head
rectifier, weighted head sum, s_p, store).  Inputs are resident in HBM before
the timed region.  The KV cache is replicated and rotated so that one step's
pages are never still in the 256 MB Infinity Cache from the previous one.

Each step is launched from the host with its arguments marshalled once
beforehand (prepared calls), so the host stays ahead of the GPU; the K timed
steps are bracketed by one pair of HIP events on the launch stream, and the
average launch duration is their interval over K.  --launch-events also
brackets every launch with its own events (which can include host submission
latency when launches are short); --graph captures the K steps into a HIP
graph and times one replay.

Prints one JSON line (rank 0, one GPU).  Usage:
  python bench.py [--steps K] [--warmup W] [--workload verify_fp8|decode_fp8|mxfp4|...]
                  [--mode in_call|schedule] [--graph|--launch-events] [--no-cpu-baseline]
  python bench.py --copy-calibration     # plain copy of known size (counter scale)
  python bench.py --read-calibration     # page-gather read rate (pages of 8448 / 4352 / 16384 B)
  python bench.py --gemm-calibration     # library bf16 GEMM (engine clock, matrix rate)
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC_FMT = "KV positions/sec and achieved HBM GB/s, %s paged MQA logits H=%d d=%d"
METRIC = METRIC_FMT % ("fp8", 64, 128)
METRIC_MXFP4 = METRIC_FMT % ("mxfp4", 64, 128)
METRIC_INDEXER = "KV positions/sec and achieved HBM GB/s, one-head bf16 indexer scores d=128"
METRIC_INDEXER_NVFP4 = ("KV positions/sec and achieved HBM GB/s, one-head nvfp4 indexer scores "
                        "d=128")
HBM_PEAK_GBS = 8000.0
# dense matrix peaks of MI355X, TFLOP/s
MFMA_PEAK_TFLOPS = {"fp8": 5000.0, "fp4": 10100.0, "f16": 2500.0}
MALL_BYTES = 256 << 20

WORKLOADS = {
    "verify_fp8": "B=128, next_n=4, H=64, d=128, page 64, seq_lens uniform 4K..64K, fp32 out",
    "decode_fp8": "B=64, next_n=1, H=64, d=128, page 64, seq_lens log-uniform 1K..32K, fp32 out",
    "mxfp4": "B=64, next_n=2, H=64, d=128, page 64, seq_lens uniform 16K..128K, bf16 out",
    "verify_fp8_n8": "B=64, next_n=8, H=64, d=128, page 64, seq_lens uniform 4K..64K, fp32 out",
    "verify_fp8_h32": "B=128, next_n=2, H=32, d=128, page 64, seq_lens uniform 4K..64K, "
                      "fp32 out",
    "verify_fp8_bf16": "B=128, next_n=4, H=64, d=128, page 64, seq_lens uniform 4K..64K, "
                       "bf16 out",
    "mxfp4_n4": "B=64, next_n=4, H=64, d=128, page 64, seq_lens uniform 16K..128K, bf16 out",
    "mxfp4_sf16": "mxfp4 with one e8m0 code per 16 values (8 per token)",
    "mxfp4_records": "mxfp4 with each token's codes after its packed bytes (68-byte records)",
    "mxfp4_sf16_records": "mxfp4 with 8 codes per token in 72-byte token records",
    "proxy_decode": "block-max proxy score: B=64 x 1 query token, 64 query heads over 8 KV "
                    "heads, d=128, paged NVFP4 keys (blocks of 128), key counts uniform "
                    "16K..128K, causal, 1024 blocks per row, fp32 out",
    "proxy_verify": "proxy_decode with 4 query tokens per request",
    "indexer_bf16": "24 query rows in groups of 1..8 over 6 requests, d=128, bf16 key pages of 64, "
                    "context lengths uniform 0..4096 (one 0), fp32 scores",
    "indexer_nvfp4": "as indexer_bf16 with NVFP4 query and keys (packed e2m1, e4m3 scale per "
                     "16 values, key scales paged like the keys)",
    "indexer_bf16_8k": "8192 query rows in groups of 1..8 over 512 requests, d=128, bf16 key "
                       "pages of 64 (64 per request), context lengths uniform 0..4096, fp32 "
                       "scores [8192, 4096]",
    "indexer_nvfp4_8k": "indexer_bf16_8k with NVFP4 query and keys",
}


def algorithmic_bytes_per_position(variant, next_n, out_bytes, head_dim=128, sf_vec_size=32):
    """Bytes the method must move per KV position (page-tail padding, query,
    weight and block-table reads excluded): the key, its scale(s), one output
    per query slot."""
    if variant == "fp8":
        return head_dim + 4 + next_n * out_bytes
    return head_dim // 2 + head_dim // sf_vec_size + next_n * out_bytes


def launch_slots(variant, next_n, num_heads, head_dim):
    """Query slots of each kernel launch of one call, as the library splits
    them: up to 4 per launch with 64 heads x 128; otherwise (FP8) as many as
    a 32 KB query slice of the heads padded to 32 holds."""
    if num_heads == 64 and head_dim == 128:
        per = 4
    else:
        per = 32768 // (-(-head_dim // 128) * 128 * (-(-num_heads // 32) * 32))
    return [min(per, next_n - s) for s in range(0, next_n, per)]


def launch_bytes_per_position(variant, next_n, out_bytes, num_heads, head_dim, sf_vec_size=32):
    """Algorithmic bytes per KV position summed over the launches of a call:
    every launch reads the key and its scale and writes its own slots."""
    return sum(algorithmic_bytes_per_position(variant, n, out_bytes, head_dim, sf_vec_size)
               for n in launch_slots(variant, next_n, num_heads, head_dim))


KERNEL_SOURCES = ["paged_mqa_logits_02_amd/csrc/mqa_logits.hip",
                  "paged_mqa_logits_02_amd/csrc/mqa_any.hip",
                  "paged_mqa_logits_02_amd/csrc/ring.hpp",
                  "paged_mqa_logits_02_amd/csrc/device.hpp",
                  "paged_mqa_logits_02_amd/csrc/pmqa_internal.h",
                  "paged_mqa_logits_02_amd/build.py"]


# the sources of the other kernels' profiles (proxy score, indexer)
KERNEL_SOURCES_OF = {
    "mqa_logits": KERNEL_SOURCES,
    "proxy": ["paged_mqa_logits_02_amd/csrc/proxy.hip", "paged_mqa_logits_02_amd/csrc/device.hpp",
              "paged_mqa_logits_02_amd/csrc/pmqa_internal.h", "paged_mqa_logits_02_amd/build.py"],
    "indexer": ["paged_mqa_logits_02_amd/csrc/indexer.hip",
                "paged_mqa_logits_02_amd/csrc/device.hpp",
                "paged_mqa_logits_02_amd/csrc/pmqa_internal.h",
                "paged_mqa_logits_02_amd/build.py"],
}


def kernel_source_hash(kernel="mqa_logits"):
    """sha256 over a kernel's sources and build flags."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES_OF[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_traffic(workload, kernel="mqa_logits"):
    """HBM bytes per launch from the committed rocprofv3 counter summary of this
    workload (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads
    for a plain copy of known size); None if there is none or it was taken on
    other kernel sources."""
    path = os.path.join(ROOT, "profiles", "%s_%s_traffic.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_hash(kernel):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp, target_s=12.0):
    """The oracle (float64, as it stands) on a bounded sample of the same
    workload: random KV positions, every query slot of each."""
    import oracle
    threads = oracle.default_threads()
    rng = np.random.default_rng(123)
    lens = np.minimum(np.maximum(inp.seq_lens, 0), inp.max_context).astype(np.int64)
    cum = np.concatenate([[0], np.cumsum(lens)])

    def sample(npos):
        f = rng.integers(0, cum[-1], npos)
        b = np.searchsorted(cum, f, side="right") - 1
        p = f - cum[b]
        rows = (b[:, None] * inp.next_n + np.arange(inp.next_n)[None, :]).ravel()
        cols = np.repeat(p, inp.next_n)
        return rows, cols

    done, spent = 0, 0.0
    npos = 256
    while spent < target_s:
        rows, cols = sample(npos)
        t0 = time.perf_counter()
        oracle.mqa_logits_points_for(inp, rows, cols, nthreads=threads)
        dt = time.perf_counter() - t0
        done += npos
        spent += dt
        rate = npos / max(dt, 1e-6)
        npos = int(min(max(rate * (target_s - spent), 256), 4_000_000))
        if target_s - spent < 0.5:
            break
    # the same oracle on one thread, on a short sample (about 3 s)
    done1, spent1, npos = 0, 0.0, 64
    while spent1 < 3.0:
        rows, cols = sample(npos)
        t0 = time.perf_counter()
        oracle.mqa_logits_points_for(inp, rows, cols, nthreads=1)
        dt = time.perf_counter() - t0
        done1 += npos
        spent1 += dt
        npos = int(min(max(npos / max(dt, 1e-6) * (3.0 - spent1), 64), 1_000_000))
        if 3.0 - spent1 < 0.2:
            break
    return {"value": done / spent, "unit": "KV positions/s", "cores": threads, "kind": "oracle",
            "sample": "%d random KV positions of the workload x all %d query slots, float64 "
                      "oracle at sampled cells, %.1f s" % (done, inp.next_n, spent),
            "single_thread_value": done1 / spent1,
            "single_thread_sample": "%d random KV positions, 1 thread, %.1f s" % (done1, spent1)}


def copy_calibration(steps):
    """A plain device-to-device copy of known size, for scaling the HBM byte
    counters (FETCH_SIZE / WRITE_SIZE) of a profiler run."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": dt * 1e3,
                      "gb_per_s": 2 * n / dt / 1e9}))


def read_calibration(steps):
    """The page-gather read rate of the GPU: whole pages of the logits and
    indexer kernels' sizes (FP8 8448 B, MXFP4 4352 B, BF16 indexer 16 KiB)
    read in a random order from a 2 GiB pool by a kernel that does nothing
    else (libpmqa_calib.so, a measurement tool), one JSON line per size."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "paged_mqa_logits_02_amd", "libpmqa_calib.so"))
    fn = lib.pmqa_calib_read_pages
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_void_p,
                   ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    dev = torch.device("cuda", 0)
    pool = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    pool.fill_(1)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(cus * 16 * 256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    gen = torch.Generator(device="cpu").manual_seed(0)
    for page_bytes, per_cu in [(b, g) for b in (8448, 4352, 16384) for g in (4, 16)]:
        grid = cus * per_cu  # workgroups resident at once, or queued behind them
        n = pool.numel() // page_bytes
        ids = torch.randperm(n, generator=gen).to(torch.int32).to(dev)

        def run():
            rc = fn(pool.data_ptr(), page_bytes, page_bytes, ids.data_ptr(), n, out.data_ptr(),
                    grid, ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError("pmqa_calib_read_pages failed (%d)" % rc)
        for _ in range(3):
            run()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(steps):
            run()
        ev[1].record(stream)
        torch.cuda.synchronize()
        dt = ev[0].elapsed_time(ev[1]) / 1e3 / steps
        print(json.dumps({"page_bytes": page_bytes, "pages": n, "grid": grid,
                          "ms": dt * 1e3, "gb_per_s": n * page_bytes / dt / 1e9}))


def gemm_calibration(steps):
    """A compute-bound library kernel (bf16 GEMM 8192^3 on the matrix cores),
    for reading the engine clock under matrix load from the profiler's
    cycle counters."""
    import torch
    n = 8192
    a = torch.randn((n, n), dtype=torch.bfloat16, device="cuda")
    b = torch.randn((n, n), dtype=torch.bfloat16, device="cuda")
    for _ in range(2):
        c = a @ b
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        c = a @ b
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"gemm_n": n, "ms": dt * 1e3, "tflops": 2 * n ** 3 / dt / 1e12,
                      "check": float(c[0, 0])}))


def run_indexer(args, torch, synth, pm, dev):
    """The one-head indexer workloads: one indexer_scores call per step."""
    nvfp4 = args.workload.startswith("indexer_nvfp4")
    inp = synth.make_config(args.workload)
    key_bytes = inp.key_cache.nbytes + (inp.key_scales.nbytes if nvfp4 else 0)
    R = args.replicas or max(2, -(-2 * MALL_BYTES // key_bytes))
    keys = [torch.from_numpy(inp.key_cache).to(dev) for _ in range(R)]
    kscales = [torch.from_numpy(inp.key_scales).to(dev) for _ in range(R)] if nvfp4 else [None]
    if nvfp4:
        qry = torch.from_numpy(inp.query).to(dev)
        qsc = torch.from_numpy(inp.query_scales).to(dev)
    else:
        qry = torch.from_numpy(inp.query.view(np.int16)).to(dev).view(torch.bfloat16)
        qsc = None
    bt = torch.from_numpy(inp.block_table).to(dev)
    lens = torch.from_numpy(inp.context_lengths).to(dev)
    reqs = torch.from_numpy(inp.requests).to(dev)
    offs = None if inp.group_row_offsets is None else torch.from_numpy(inp.group_row_offsets).to(dev)
    scores = [torch.empty((inp.rows, inp.max_context), dtype=torch.float32, device=dev)
              for _ in range(2)]
    stream = torch.cuda.current_stream(dev)
    import math
    L = R * 2 // math.gcd(R, 2)
    calls = [pm.prepare_indexer_scores(qry, keys[i % R], bt, lens, requests=reqs,
                                       scores=scores[i % 2], query_scales=qsc,
                                       key_scales=kscales[i % R] if nvfp4 else None,
                                       group_row_offsets=offs, stream=stream)
             for i in range(L)]
    t_ramp = time.time() + args.ramp
    i = 0
    while time.time() < t_ramp:
        calls[i % L]()
        i += 1
        if i % 50 == 0:
            torch.cuda.synchronize()
    for i in range(args.warmup):
        calls[i % L]()
    torch.cuda.synchronize()
    K = args.steps
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(K):
        calls[i % L]()
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    kern = total_ms / K
    lens_np = np.minimum(np.maximum(inp.context_lengths, 0), inp.max_context).astype(np.int64)
    sizes = np.diff(inp.row_offsets()).astype(np.int64)
    # per key and group: its packed values (and scales) + one fp32 score per row
    key_b = 64 + 8 if nvfp4 else 256
    alg = int((lens_np * (key_b + 4 * sizes)).sum())
    positions = int(lens_np.sum())
    achieved = alg / (kern * 1e-3) / 1e9
    traffic = counter_traffic(args.workload, "indexer")
    traffic_gbs = None if traffic is None else traffic / (kern * 1e-3) / 1e9
    line = {
        "metric": METRIC_INDEXER_NVFP4 if nvfp4 else METRIC_INDEXER,
        "value": positions * K / (total_ms * 1e-3),
        "unit": "KV positions/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": kern, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "nvfp4" if nvfp4 else "bf16", "data": "synthetic",
        "gb_per_s": achieved,
        "config": {"workload": args.workload, "shape": WORKLOADS[args.workload],
                   "rows": inp.rows, "groups": inp.groups, "max_context": inp.max_context,
                   "kv_positions": positions, "key_replicas": R, "kernel_ms_avg": kern,
                   "timing": "host launches of prepared calls, events around the %d launches" % K,
                   "algorithmic_bytes_per_launch": alg, "counter_bytes_per_launch": traffic},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_gbs},
    }
    print(json.dumps(line), flush=True)


METRIC_PROXY = ("KV positions/sec (keys of every KV head scored per second), block-max proxy "
                "score, nvfp4 paged keys, %d query heads over %d KV heads, d=128, MI355X")


def proxy_bytes_and_flops(inp):
    """Algorithmic bytes of one call (every key block scored, once per KV
    head: 64 packed bytes + 8 e4m3 scales per key; every output float once;
    the query rows once) and flops (2 * 128 per query head, token and key
    scored)."""
    L = inp.key_lengths()
    lq = np.diff(inp.cu_q).astype(np.int64)
    blocks = np.minimum((L + 127) // 128, inp.max_k_tiles)
    keys = blocks * 128  # per KV head, block-granular
    kb = int(keys.sum()) * inp.num_kv_heads * 72
    ob = inp.out_heads * inp.max_k_tiles * inp.total_q * 4
    qb = inp.total_q * inp.num_qo_heads * 72
    flops = 2.0 * 128 * inp.num_qo_heads * float((lq * keys).sum())
    return kb + ob + qb, flops, int(keys.sum()) * inp.num_kv_heads


def run_proxy(args, torch, synth, pm, dev):
    """The block-max proxy score workloads: one msa_proxy_score_fp4 call per step."""
    inp = synth.make_config(args.workload)
    t = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    raw = t(inp.k)
    H = inp.num_kv_heads
    k = raw.as_strided((raw.shape[0], H, 128, 64), (raw.shape[1], 128 * 64, 64, 1))
    q, qs, ks = t(inp.q), t(inp.q_scale), t(inp.k_scale)
    cu_q, pt, su = t(inp.cu_q), t(inp.page_table), t(inp.seqused_k)
    outs = [torch.empty((inp.out_heads, inp.max_k_tiles, inp.total_q), dtype=torch.float32,
                        device=dev) for _ in range(2)]
    stream = torch.cuda.current_stream(dev)
    maxq = int(np.max(np.diff(inp.cu_q)))
    calls = [pm.prepare_msa_proxy_score_fp4(q, k, qs, ks, inp.q_global_scale, inp.k_global_scale,
                                            cu_q, page_table=pt, seqused_k=su,
                                            causal=inp.causal, max_seqlen_q=maxq,
                                            max_k_tiles=inp.max_k_tiles, output=outs[i],
                                            reduce_heads=inp.reduce_heads, stream=stream)
             for i in range(2)]
    t_ramp = time.time() + args.ramp
    i = 0
    while time.time() < t_ramp:
        calls[i % 2]()
        i += 1
        if i % 20 == 0:
            torch.cuda.synchronize()
    for i in range(args.warmup):
        calls[i % 2]()
    torch.cuda.synchronize()
    K = args.steps
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(K):
        calls[i % 2]()
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    kern = total_ms / K
    alg, flops, positions = proxy_bytes_and_flops(inp)
    achieved = alg / (kern * 1e-3) / 1e9
    tflops = flops / (kern * 1e-3) / 1e12
    traffic = counter_traffic(args.workload, "proxy")
    traffic_gbs = None if traffic is None else traffic / (kern * 1e-3) / 1e9
    hbm = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_gbs}
    mfma = {"bound": "mfma", "achieved": tflops, "peak": MFMA_PEAK_TFLOPS["f16"],
            "unit": "TFLOP/s", "frac": tflops / MFMA_PEAK_TFLOPS["f16"], "traffic": traffic_gbs,
            "traffic_unit": "GB/s of HBM counter bytes"}
    hbm_s, mfma_s = alg / (HBM_PEAK_GBS * 1e9), flops / (MFMA_PEAK_TFLOPS["f16"] * 1e12)
    line = {
        "metric": METRIC_PROXY % (inp.num_qo_heads, inp.num_kv_heads),
        "value": positions * K / (total_ms * 1e-3),
        "unit": "KV positions/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": kern, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic", "gb_per_s": achieved,
        "config": {"workload": args.workload, "shape": WORKLOADS[args.workload],
                   "batch": inp.batch, "total_q": inp.total_q, "pages": inp.num_pages,
                   "kv_positions": positions, "kernel_ms_avg": kern,
                   "products": "f16 MFMA of exactly dequantised e2m1 x e4m3, fp32 sums",
                   "timing": "host launches of prepared calls, events around the %d launches" % K,
                   "algorithmic_bytes_per_launch": alg, "flops_per_launch": flops,
                   "counter_bytes_per_launch": traffic,
                   "hbm": dict(hbm, ideal_us=hbm_s * 1e6), "mfma": dict(mfma, ideal_us=mfma_s * 1e6)},
        "roofline": mfma if mfma_s > hbm_s else hbm,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="verify_fp8", choices=sorted(WORKLOADS))
    ap.add_argument("--mode", default="in_call", choices=["in_call", "schedule", "reuse"],
                    help="work split: inside the logits kernel; by the schedule kernel every "
                         "step; or one schedule computed before the timed steps and reused")
    ap.add_argument("--replicas", type=int, default=0)
    ap.add_argument("--ramp", type=float, default=1.0,
                    help="seconds of untimed launches to bring the clock up before warmup")
    ap.add_argument("--graph", action="store_true",
                    help="capture the timed steps into one HIP graph and time a replay")
    ap.add_argument("--launch-events", action="store_true",
                    help="also time every launch with its own pair of events")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workspace", action="store_true",
                    help="give the logits calls a workspace: a work counter with which the "
                         "workgroups that finish first take the call's last items in chunks")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--gemm-calibration", action="store_true")
    ap.add_argument("--read-calibration", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the paged MQA logits path has no multi-GPU "
              "mode here (every logit is independent; sharding by request or page range "
              "needs no collective).  Run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration(args.steps)
        return
    if args.gemm_calibration:
        gemm_calibration(args.steps)
        return
    if args.read_calibration:
        read_calibration(args.steps)
        return

    import synth
    import paged_mqa_logits_02_amd as pm

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pm.init(0)
    if args.workload.startswith("indexer_"):
        run_indexer(args, torch, synth, pm, dev)
        return
    if args.workload.startswith("proxy_"):
        run_proxy(args, torch, synth, pm, dev)
        return
    inp = synth.make_config(args.workload)
    variant = 0 if inp.variant == "fp8" else 1
    out_dtype = torch.float32 if inp.out_dtype == "f32" else torch.bfloat16
    out_bytes = 4 if out_dtype == torch.float32 else 2

    kv_bytes = inp.kv.nbytes
    R = args.replicas or max(2, -(-2 * MALL_BYTES // kv_bytes))
    kv = [torch.from_numpy(inp.kv).to(dev) for _ in range(R)]
    q = torch.from_numpy(inp.q).to(dev)
    q_sf = None if inp.q_sf is None else torch.from_numpy(inp.q_sf).to(dev)
    w = torch.from_numpy(inp.weights).to(dev)
    sl = torch.from_numpy(inp.seq_lens).to(dev)
    bt = torch.from_numpy(inp.block_table).to(dev)
    outs = [torch.empty((inp.rows, inp.max_context), dtype=out_dtype, device=dev)
            for _ in range(2)]
    U = pm.num_units(inp.next_n, variant)
    sched = torch.empty(pm.schedule_ints(U), dtype=torch.int32, device=dev)
    mx_layout = dict(sf_vec_size=inp.sf_vec_size, is_kv_sf_interleaved=inp.kv_sf_interleaved)
    # the work counter of the in-call split (caller workspace), if asked for
    ws = pm.workspace(dev) if args.workspace else None
    stream = torch.cuda.current_stream(dev)

    def step(i, st, ev0=None, ev1=None):
        s = sched if args.mode == "reuse" else None
        if args.mode == "schedule":
            pm.mqa_logits_schedule(sl, inp.next_n, variant, max_context=inp.max_context,
                                   num_units=U, out=sched, stream=st)
            s = sched
        if ev0 is not None:
            ev0.record(st)
        if variant == 0:
            pm.mqa_logits_fp8(q, kv[i % R], w, sl, bt, max_context=inp.max_context,
                              out=outs[i % 2], schedule_meta=s, stream=st, workspace=ws)
        else:
            pm.mqa_logits_mxfp4(q, q_sf, kv[i % R], w, sl, bt, max_context=inp.max_context,
                                out=outs[i % 2], schedule_meta=s, stream=st, workspace=ws,
                                **mx_layout)
        if ev1 is not None:
            ev1.record(st)

    # Prepared calls: the arguments of every distinct step are marshalled
    # once, outside the timed region.
    import math
    L = R * 2 // math.gcd(R, 2)
    sched_call = None
    if args.mode != "in_call":
        sched_call = pm.prepare_mqa_logits_schedule(sl, inp.next_n, variant,
                                                    max_context=inp.max_context, num_units=U,
                                                    out=sched, stream=stream)
        sched_call()  # the reused schedule; recomputed every step in "schedule" mode
    calls = []
    for i in range(L):
        s_meta = sched if args.mode != "in_call" else None
        if variant == 0:
            calls.append(pm.prepare_mqa_logits_fp8(q, kv[i % R], w, sl, bt,
                                                   max_context=inp.max_context, out=outs[i % 2],
                                                   schedule_meta=s_meta, stream=stream,
                                                   workspace=ws))
        else:
            calls.append(pm.prepare_mqa_logits_mxfp4(q, q_sf, kv[i % R], w, sl, bt,
                                                     max_context=inp.max_context,
                                                     out=outs[i % 2], schedule_meta=s_meta,
                                                     stream=stream, workspace=ws, **mx_layout))

    def fast_step(i, ev0=None, ev1=None):
        if args.mode == "schedule":
            sched_call()
        if ev0 is not None:
            ev0.record(stream)
        calls[i % L]()
        if ev1 is not None:
            ev1.record(stream)

    # Bring the engine clock up before the warmup steps (the first launches
    # after idle run at a lower clock); untimed.
    t_ramp = time.time() + args.ramp
    i = 0
    while time.time() < t_ramp:
        fast_step(i)
        i += 1
        if i % 20 == 0:
            torch.cuda.synchronize()
    for i in range(args.warmup):
        fast_step(i)
    torch.cuda.synchronize()

    K = args.steps
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    if not args.graph:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              if args.launch_events else (None, None) for _ in range(K)]
        torch.cuda.synchronize()
        t_begin.record(stream)
        for i in range(K):
            fast_step(i, *ev[i])
        t_end.record(stream)
        torch.cuda.synchronize()
        total_ms = t_begin.elapsed_time(t_end)
        kern_ms = ([a.elapsed_time(b) for a, b in ev] if args.launch_events else [total_ms / K])
    else:
        # the K steps as one graph, captured on a side stream (default
        # priority), replayed once untimed and once timed on the launch stream
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream(dev)
        cap.wait_stream(stream)
        with torch.cuda.graph(graph, stream=cap):
            for i in range(K):
                step(i, cap)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        t_begin.record(stream)
        graph.replay()
        t_end.record(stream)
        torch.cuda.synchronize()
        total_ms = t_begin.elapsed_time(t_end)
        kern_ms = [total_ms / K]
    kern_avg = float(np.mean(kern_ms))

    traffic = counter_traffic(args.workload)
    positions = inp.kv_positions()
    bpp = algorithmic_bytes_per_position(inp.variant, inp.next_n, out_bytes, inp.head_dim,
                                         inp.sf_vec_size)
    slots = launch_slots(inp.variant, inp.next_n, inp.num_heads, inp.head_dim)
    lbpp = launch_bytes_per_position(inp.variant, inp.next_n, out_bytes, inp.num_heads,
                                     inp.head_dim, inp.sf_vec_size)
    alg_bytes = positions * bpp
    # roofline of the logits kernel: algorithmic bytes of every launch of a
    # call (each launch reads the keys) over the call's duration, i.e. the
    # average over its launches (equal-size launches)
    achieved = positions * lbpp / (kern_avg * 1e-3) / 1e9
    value = positions * K / (total_ms * 1e-3)
    # matrix-core roofline: the method's 2*H*D*next_n flops per KV position,
    # against the dense peak of the products' type (FP8 multiplies exactly
    # widened f16 operands, MXFP4 its e2m1 operands)
    mfma_type = "f16" if inp.variant == "fp8" else "fp4"
    flops = positions * 2.0 * inp.num_heads * inp.head_dim * inp.next_n
    mfma_tflops = flops / (kern_avg * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[mfma_type]
    # the bound is the roofline with the longer ideal time per call
    hbm_s = positions * lbpp / (HBM_PEAK_GBS * 1e9)
    mfma_s = flops / (peak * 1e12)
    traffic_gbs = None if traffic is None else traffic * len(slots) / (kern_avg * 1e-3) / 1e9
    hbm_line = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_gbs}
    mfma_line = {"bound": "mfma", "achieved": mfma_tflops, "peak": peak, "unit": "TFLOP/s",
                 "frac": mfma_tflops / peak, "traffic": traffic_gbs,
                 "traffic_unit": "GB/s of HBM counter bytes"}

    line = {
        "metric": METRIC_FMT % (inp.variant, inp.num_heads, inp.head_dim),
        "value": value,
        "unit": "KV positions/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": total_ms / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if inp.variant == "fp8" else "fp4",
        "data": "synthetic",
        "gb_per_s": alg_bytes * K / (total_ms * 1e-3) / 1e9,
        "config": {
            "workload": args.workload,
            "shape": WORKLOADS[args.workload],
            "batch": inp.batch, "next_n": inp.next_n, "num_heads": inp.num_heads,
            "head_dim": inp.head_dim, "max_context": inp.max_context,
            "kv_positions": positions, "pages": int(inp.num_pages),
            "schedule": args.mode, "kv_replicas": R, "units": U,
            "work_counter": bool(args.workspace and args.mode == "in_call"),
            "products": ("f16 MFMA of exactly widened e4m3, fp32 sums" if inp.variant == "fp8"
                         else "scaled e2m1 MFMA, fp32 sums"),
            **({} if inp.variant == "fp8" else {
                "sf_vec_size": inp.sf_vec_size, "kv_sf_interleaved": inp.kv_sf_interleaved}),
            "timing": ("graph of the %d steps, events around one replay" % K if args.graph else
                       "host launches of prepared calls, " +
                       ("events around every launch" if args.launch_events else
                        "events around the %d launches" % K)),
            "kernel_ms_avg": kern_avg, "kernel_ms_min": float(np.min(kern_ms)),
            "algorithmic_bytes_per_position": bpp,
            "launch_slots": slots,
            "launch_bytes_per_position": lbpp,
            "algorithmic_bytes_per_launch": positions * lbpp / len(slots),
            "counter_bytes_per_launch": traffic,
            "mfma": dict(mfma_line, products=mfma_type, flops_per_call=flops,
                         ideal_us=mfma_s * 1e6),
            "hbm": dict(hbm_line, ideal_us=hbm_s * 1e6),
        },
        "roofline": mfma_line if mfma_s > hbm_s else hbm_line,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
