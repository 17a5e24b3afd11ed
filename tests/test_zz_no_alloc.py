"""The entry point that allocates nothing (mqa_logits_fp8_no_alloc), through
the C ABI, against mqa_logits_fp8 on the same inputs: the same written set
and bit-identical values, on two calls in a row (the second smaller), for
the 64-head kernels with 1, 4 and 6 query slots (one or two launches, each
using the library's work counters) and for the general kernel."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import DevMqa, host_out, pm, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    pm().init()
    yield
    torch.cuda.synchronize()


def _no_alloc(dm, out):
    pm().mqa_logits_fp8_no_alloc(dm.q, dm.kv, dm.w, dm.sl, dm.bt,
                                 max_context=dm.inp.max_context, out=out)
    return out


@pytest.mark.parametrize("next_n,heads,head_dim", [(1, 64, 128), (4, 64, 128), (6, 64, 128),
                                                   (2, 32, 96)])
def test_no_alloc_matches_fp8_entry_point(next_n, heads, head_dim):
    calls = [  # (lengths, max_context): the second call is smaller
        (np.random.default_rng(340 + next_n).integers(0, 3000, 23), 3072),
        (np.array([700, 0, 65, 1]), 1024),
    ]
    for k, (lens, maxc) in enumerate(calls):
        inp = synth.make_mqa_inputs(lens, next_n, num_heads=heads, head_dim=head_dim,
                                    max_context=maxc, bt_width=maxc // 64, seed=350 + k)
        say("no-alloc call %d: N=%d H=%d D=%d B=%d" % (k, next_n, heads, head_dim, inp.batch))
        dm = DevMqa(inp)
        ref, wref = host_out(dm.run())
        got, wrote = host_out(_no_alloc(dm, dm.new_out()))
        assert np.array_equal(wrote, wref)
        assert np.array_equal(got.view(np.uint64), ref.view(np.uint64))
