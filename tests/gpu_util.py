"""GPU-side helpers of the parity tests: move synthetic inputs to the device,
call the library through its binding with sentinel-filled outputs, and compare
with the oracle (written set exactly, values within the stated tolerance)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from fixtures_util import BF16_SENTINEL, F32_SENTINEL

DEV = torch.device("cuda:0")

# |gpu - ref| <= REL * A + ABS, A = s_p * sum_h |w| * relu(q.k)
TOL_F32 = (2e-3, 1e-5)
TOL_BF16 = (1e-2, 1e-5)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def pm():
    import paged_mqa_logits_02_amd as m
    return m


class DevMqa:
    """Device copies of a synth.MqaInputs."""

    def __init__(self, inp, kv=None):
        self.inp = inp
        t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
        self.q = t(inp.q)
        self.q_sf = t(inp.q_sf)
        self.kv = t(inp.kv) if kv is None else kv
        self.w = t(inp.weights)
        self.sl = t(inp.seq_lens)
        self.bt = t(inp.block_table)

    def new_out(self, dtype=None):
        inp = self.inp
        if dtype is None:
            dtype = torch.float32 if inp.out_dtype == "f32" else torch.bfloat16
        out = torch.empty((inp.rows, inp.max_context), dtype=dtype, device=DEV)
        if dtype == torch.float32:
            out.view(torch.int32).fill_(F32_SENTINEL)
        else:
            out.view(torch.int16).fill_(BF16_SENTINEL)
        return out

    def run(self, out=None, schedule=None, dtype=None, stream=None, workspace=None):
        if out is None:
            out = self.new_out(dtype)
        m = pm()
        if self.inp.variant == "fp8":
            m.mqa_logits_fp8(self.q, self.kv, self.w, self.sl, self.bt,
                             max_context=self.inp.max_context, out=out, schedule_meta=schedule,
                             stream=stream, workspace=workspace)
        else:
            m.mqa_logits_mxfp4(self.q, self.q_sf, self.kv, self.w, self.sl, self.bt,
                               sf_vec_size=self.inp.sf_vec_size,
                               is_kv_sf_interleaved=self.inp.kv_sf_interleaved,
                               max_context=self.inp.max_context, out=out,
                               schedule_meta=schedule, stream=stream, workspace=workspace)
        return out


def host_out(out):
    """(values float64, written mask) of a device output buffer."""
    torch.cuda.synchronize()
    o = out.cpu()
    if o.dtype == torch.float32:
        bits = o.view(torch.int32).numpy().view(np.uint32)
        wrote = bits != F32_SENTINEL
        vals = o.numpy().astype(np.float64)
    else:
        bits = o.view(torch.int16).numpy().view(np.uint16)
        wrote = bits != BF16_SENTINEL
        vals = o.float().numpy().astype(np.float64)
    return vals, wrote


def tol_for(dtype):
    return TOL_F32 if dtype == torch.float32 else TOL_BF16


def check_values(got, ref, amag, tol, what=""):
    rel, ab = tol
    err = np.abs(got - ref)
    lim = rel * amag + ab
    bad = ~(err <= lim)
    if bad.any():
        i = np.argmax(np.where(bad, err / lim, 0))
        raise AssertionError("%s: %d of %d values out of tolerance; worst got %r ref %r A %r" % (
            what, int(bad.sum()), bad.size, got.flat[i], ref.flat[i], amag.flat[i]))
    return float(np.max(err / lim)) if err.size else 0.0


def check_dense(dm, out, what=""):
    """Whole-output comparison against the dense oracle."""
    got, wrote = host_out(out)
    ref, amag, written = oracle.mqa_logits_for(dm.inp)
    assert np.array_equal(wrote, written), "%s: written set differs (%d vs %d cells)" % (
        what, int(wrote.sum()), int(written.sum()))
    return check_values(got[written], ref[written], amag[written], tol_for(out.dtype), what)


def sample_cells(inp, rng, per_request=24):
    """Cells the oracle evaluates one by one at full size: per request the first
    and last written columns, the meaningful limit of every slot and random
    columns; plus random cells anywhere."""
    rows, cols = [], []
    N = inp.next_n
    for b in range(inp.batch):
        L = int(inp.seq_lens[b])
        E = 0 if L <= 0 else min((L + 63) // 64 * 64, inp.max_context)
        for t in range(N):
            r = b * N + t
            picks = [0, max(E - 1, 0), min(max(L - N + t, 0), inp.max_context - 1)]
            picks += rng.integers(0, max(E, 1), per_request // N).tolist()
            rows += [r] * len(picks)
            cols += picks
    n = 256
    rows += rng.integers(0, inp.rows, n).tolist()
    cols += rng.integers(0, inp.max_context, n).tolist()
    return np.array(rows, np.int32), np.array(cols, np.int32)


def meaningful(inp, rows, cols):
    """Cells (row b*N+t, column p) with p <= seq_lens[b] - N + t: the columns a
    slot's logits are defined for (the rest of the written extent is padding)."""
    N = inp.next_n
    b, t = rows // N, rows % N
    return cols <= inp.seq_lens[b].astype(np.int64) - N + t


def check_sampled(dm, out, rng, what=""):
    """Full-size comparison: the complete written set, values at sampled cells.
    Returns the worst err/tol over the sampled written cells; the worst over
    the meaningful ones among them is printed beside it."""
    inp = dm.inp
    got, wrote = host_out(out)
    written = oracle.mqa_written(inp.seq_lens, inp.batch, inp.next_n, inp.max_context)
    assert np.array_equal(wrote, written), "%s: written set differs (%d vs %d cells)" % (
        what, int(wrote.sum()), int(written.sum()))
    rows, cols = sample_cells(inp, rng)
    ref, amag, w = oracle.mqa_logits_points_for(inp, rows, cols)
    assert np.array_equal(w, written[rows, cols])
    tol = tol_for(out.dtype)
    r = check_values(got[rows, cols][w], ref[w], amag[w], tol, what)
    m = w & meaningful(inp, rows, cols)
    if m.any():
        rm = check_values(got[rows, cols][m], ref[m], amag[m], tol, what + " (meaningful)")
        say("%s: max err/tol %.3g over %d sampled cells, %.3g over the %d meaningful ones" % (
            what, r, int(w.sum()), rm, int(m.sum())))
    return r


class DevIndexer:
    """Device copies of a synth.IndexerInputs (BF16 or NVFP4)."""

    def __init__(self, ix, key_cache=None, key_scales=None):
        self.ix = ix
        t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
        if getattr(ix, "fmt", "bf16") == "nvfp4":
            self.q = t(ix.query)
            self.qs = t(ix.query_scales)
            self.ks = t(ix.key_scales) if key_scales is None else key_scales
        else:
            self.q = t(ix.query.view(np.int16)).view(torch.bfloat16)
            self.qs = self.ks = None
        self.kc = t(ix.key_cache) if key_cache is None else key_cache
        self.bt = t(ix.block_table)
        self.lens = t(ix.context_lengths)
        self.reqs = t(ix.requests)
        self.offs = t(ix.group_row_offsets)

    def run(self):
        scores = torch.empty((self.ix.rows, self.ix.max_context), dtype=torch.float32, device=DEV)
        scores.view(torch.int32).fill_(F32_SENTINEL)
        pm().indexer_scores(self.q, self.kc, self.bt, self.lens, requests=self.reqs,
                            scores=scores, query_scales=self.qs, key_scales=self.ks,
                            group_row_offsets=self.offs)
        return scores


def check_indexer(di, scores, what=""):
    got, wrote = host_out(scores)
    ref, amag, written = oracle.indexer_scores_for(di.ix)
    assert np.array_equal(wrote, written), "%s: written set differs (%d vs %d)" % (
        what, int(wrote.sum()), int(written.sum()))
    # one head: A = |q.k| (weight 1, no rectifier, no s_p)
    return check_values(got[written], ref[written], np.abs(ref[written]), TOL_F32, what)


def page_edge_cells(inp):
    """The first and last column of every written page, for every row of
    every request (full-size checks)."""
    rows, cols = [], []
    N = inp.next_n
    for b in range(inp.batch):
        L = int(inp.seq_lens[b])
        T = 0 if L <= 0 else min((L + 63) // 64, inp.max_context // 64)
        c = np.concatenate([np.arange(T) * 64, np.arange(T) * 64 + 63])
        for t in range(N):
            rows.append(np.full(c.size, b * N + t))
            cols.append(c)
    if not rows:
        return np.zeros(0, np.int32), np.zeros(0, np.int32)
    return np.concatenate(rows).astype(np.int32), np.concatenate(cols).astype(np.int32)


def check_cells(dm, out, rows, cols, what=""):
    """Values at the given written cells against the oracle's point evaluation."""
    inp = dm.inp
    got, wrote = host_out(out)
    ref, amag, w = oracle.mqa_logits_points_for(inp, rows, cols)
    assert w.all(), "%s: a checked cell is outside the written set" % what
    assert wrote[rows, cols].all()
    return check_values(got[rows, cols], ref, amag, tol_for(out.dtype), what)
