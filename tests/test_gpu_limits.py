"""The largest shapes the stream plan takes in one call, against the oracle:
4096 sequences (the in-kernel prefix sum over context_lens holds one entry per
sequence in LDS) and 8192 wave ranges (the merge keeps one weight per range
in LDS), with ragged short rows, empty rows among them, and the widest GQA
group (g = 16) at d_h = 128.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from synth import BF16, FP8, INT8
from tests.helpers import make_case
from tests.gpu_helpers import TOL_16BIT, TOL_8BIT, assert_parity, max_err, run_case

pytestmark = pytest.mark.gpu

MAX_BATCH = 4096
MAX_WAVES = 8192


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("kv_dtype", [BF16, FP8, INT8])
@pytest.mark.parametrize("nw", [0, MAX_WAVES])
def test_largest_batch(kv_dtype, nw):
    r = np.random.default_rng(60_000 + kv_dtype + nw)
    ctx = r.integers(0, 60, size=MAX_BATCH)
    ctx[r.integers(0, MAX_BATCH, size=50)] = 0
    ctx[7] = 700                                  # one long row among short ones
    _say(f"largest batch kv={kv_dtype} nw={nw}")
    c = make_case(61_000 + kv_dtype + nw, ctx.tolist(), n_q=8, n_kv=2, d_h=64,
                  kv_dtype=kv_dtype)
    got, _ = run_case(c, num_partitions=nw, total_context=int(ctx.sum()))
    ref = c.oracle_out()
    empty = ctx == 0
    assert (got[empty] == 0).all()
    tol = TOL_8BIT if kv_dtype in (FP8, INT8) else TOL_16BIT
    assert_parity(max_err(got[~empty], ref[~empty]), tol)


def test_batch_above_the_limit_is_rejected():
    import decode_attention_paged_slot_amd as pda
    c = make_case(62_000, [3] * (MAX_BATCH + 1), n_q=4, n_kv=2, d_h=64)
    with pytest.raises(pda.PdaError):
        run_case(c)


@pytest.mark.parametrize("kv_dtype", [BF16, FP8])
def test_widest_group_most_waves(kv_dtype):
    """g = 16 query heads per KV head at d_h = 128, rows split over the most
    wave ranges the plan allows (more ranges than blocks: the kernel caps
    them at the block count)."""
    _say(f"widest group kv={kv_dtype}")
    c = make_case(63_000 + kv_dtype, [9000, 1, 4500], n_q=128, n_kv=8, d_h=128,
                  kv_dtype=kv_dtype)
    got, _ = run_case(c, num_partitions=MAX_WAVES)
    tol = TOL_8BIT if kv_dtype == FP8 else TOL_16BIT
    assert_parity(max_err(got, c.oracle_out()), tol)


def test_default_split_follows_the_device():
    """With a device current, the default plan takes one workgroup (four
    wave ranges) per compute unit for a 16-bit cache and two for an 8-bit
    one, when the work is large enough."""
    import torch
    import decode_attention_paged_slot_amd as pda
    torch.cuda.init()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    _say(f"default split on {cus} compute units")
    for kv, per_cu in ((BF16, 4), (FP8, 8)):
        d = pda.AttnDesc(8, 64, 8, 128, 16, 2048, 18205, kv, BF16, 0, 32768, 0, 8 * 32768, 0, 0,
                         0, BF16)
        assert pda.attn_plan(d)[0] == per_cu * cus
