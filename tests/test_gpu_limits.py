"""The largest shapes the stream plan takes in one call, against the oracle:
4096 sequences (the in-kernel prefix sum over context_lens holds one entry per
sequence in LDS) and 8192 wave ranges (the merge keeps one weight per range
in LDS), with ragged short rows, empty rows among them, and the widest GQA
group (g = 16) at d_h = 128; for the 16-bit, 8-bit and 4-bit caches.
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


@pytest.mark.parametrize("nw", [0, MAX_WAVES])
def test_largest_batch_int4(nw):
    """The 4-bit cache at the largest batch: ragged short rows (most shorter
    than a block, so that their residual window is their only piece), empty
    rows and one long row, against the oracle; then one fused step over a
    cache of the same shape against the append followed by the attention,
    bit for bit (outputs, codes, value scales, residual rows). At this batch
    the kernel's LDS holds one of its workgroups per compute unit instead of
    two, so the wave ranges run in more than one round."""
    import torch
    import decode_attention_paged_slot_amd as pda
    import oracle
    import synth
    from synth import F32
    from tests.gpu_helpers import to_dev
    from tests.test_gpu_int4 import _attend, _case, _desc, _dev
    n_q, n_kv, d_h, scale = 8, 2, 64, 0.125
    r = np.random.default_rng(64_000 + nw)
    ctx = r.integers(0, 60, size=MAX_BATCH).astype(np.int32)
    ctx[r.integers(0, MAX_BATCH, size=50)] = 0
    ctx[7] = 700                                  # one long row among short ones
    _say(f"largest batch int4 nw={nw}")
    dev = "cuda"
    st, ks, table, ctx, nb, mb = _case(65_000 + nw, ctx, n_q=n_q, n_kv=n_kv, d_h=d_h)
    st_d, ks_d = _dev(st, ks, dev)
    q_np = synth.gaussian((MAX_BATCH, n_q, d_h), BF16, r)
    q = to_dev(q_np, BF16, dev)
    got = _attend(st_d, ks_d, q, table, ctx, scale,
                  _desc(MAX_BATCH, n_q, n_kv, d_h, mb, nb, BF16, F32, ctx, nw))
    ref, _, _, bad = oracle.paged_attn_int4(q_np, st, ks, table, ctx, scale, n_q=n_q,
                                            n_kv=n_kv, q_dtype=BF16)
    assert bad == 0
    ref = ref.reshape(got.shape)
    empty = ctx == 0
    assert (got[empty] == 0).all()
    assert_parity(float(np.abs(got[~empty] - ref[~empty]).max()), TOL_8BIT)

    # one fused step: the same lengths now count the step's new token
    st, ks, table, ctx, nb, mb = _case(66_000 + nw, ctx, n_q=n_q, n_kv=n_kv, d_h=d_h,
                                       poison=False)
    a_d, ks_d = _dev(st, ks, dev)
    b_d, _ = _dev(st, ks, dev)
    bt = torch.from_numpy(table).to(dev)
    ct = torch.from_numpy(ctx).to(dev)
    kn = to_dev(synth.gaussian((MAX_BATCH, n_kv, d_h), BF16, r), BF16, dev)
    vn = to_dev(synth.gaussian((MAX_BATCH, n_kv, d_h), BF16, r), BF16, dev)
    desc = _desc(MAX_BATCH, n_q, n_kv, d_h, mb, nb, BF16, F32, ctx, nw)
    out_a = torch.full((MAX_BATCH, n_q, d_h), 7.0, device=dev)
    out_b = torch.full((MAX_BATCH, n_q, d_h), -7.0, device=dev)
    pda.kv_append_int4(kn, vn, bt, ct, a_d["k"], a_d["v"], ks_d, a_d["v_scale"], a_d["k_res"],
                       a_d["v_res"], desc=desc)
    pda.paged_decode_attn_int4(q, a_d["k"], a_d["v"], ks_d, a_d["v_scale"], a_d["k_res"],
                               a_d["v_res"], bt, ct, scale, out_a, desc=desc,
                               workspace=pda.workspace_for(desc, dev))
    pda.decode_step_int4(q, kn, vn, b_d["k"], b_d["v"], ks_d, b_d["v_scale"], b_d["k_res"],
                         b_d["v_res"], bt, ct, scale, out_b, desc=desc,
                         workspace=pda.workspace_for(desc, dev))
    torch.cuda.synchronize()

    def bits(x):
        return x.view(torch.int16 if x.element_size() == 2 else
                      (torch.uint8 if x.element_size() == 1 else torch.int32)).cpu().numpy()

    assert (bits(out_a) == bits(out_b)).all()
    for key in ("k", "v", "v_scale", "k_res", "v_res"):
        assert (bits(a_d[key]) == bits(b_d[key])).all(), key


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
