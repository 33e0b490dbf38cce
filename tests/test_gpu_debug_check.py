"""PDA_DEBUG=1: before launching, the host copies the lengths and table
entries back and rejects (EINVAL) any row the kernels would turn into NaN,
by the kernels' own lookup rule. A row is invalid when its length is outside
[0, max_blocks * 16] or a block it looks up is unmapped; blocks a sliding
window skips, a shared-prefix row's own entries below its prefix, and a
4-bit row's open block (held in the residual buffer) are not looked up, so
leaving them unmapped is accepted and the results are unchanged."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import synth
from synth import BF16, F32, FP8
from tests.helpers import make_case
from tests.gpu_helpers import TOL_16BIT, TOL_8BIT, assert_parity, max_err, run_case, to_dev
from tests import test_gpu_int4 as i4
from tests import test_gpu_prefix as pfx

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _rejects(fn):
    import decode_attention_paged_slot_amd as pda
    with pytest.raises(pda.PdaError) as e:
        fn()
    return e.value.status == pda.binding.EINVAL


def test_debug_rejects_unmapped_or_overlong_rows(monkeypatch):
    c = make_case(9901, [300, 70, 129], n_q=8, n_kv=2, d_h=128)
    monkeypatch.setenv("PDA_DEBUG", "1")
    _say("debug: plain rows")
    got, _ = run_case(c)
    assert_parity(max_err(got, c.oracle_out()), TOL_16BIT)
    t = c.table.copy()
    t[1, 2] = -1
    assert _rejects(lambda: run_case(c, table=t))
    t = c.table.copy()
    t[2, 8] = c.num_blocks          # the last block of a 129-token row
    assert _rejects(lambda: run_case(c, table=t))
    c.ctx = c.ctx.copy()
    c.ctx[0] = c.max_blocks * 16 + 1
    assert _rejects(lambda: run_case(c, max_context=300))


@pytest.mark.parametrize("kv_dtype", [BF16, FP8, F32])
@pytest.mark.parametrize("window,sinks", [(100, 4), (33, 0)])
def test_debug_accepts_blocks_a_window_skips(monkeypatch, kv_dtype, window, sinks):
    ctx = [700, 33, 2000, 0]
    c = make_case(9910 + window + kv_dtype, ctx, n_q=8, n_kv=2, d_h=128, kv_dtype=kv_dtype,
                  q_dtype=BF16 if kv_dtype != F32 else F32)
    table = c.table.copy()
    for b, n in enumerate(c.ctx):
        for blk in range((int(n) + 15) // 16):
            ts = range(16 * blk, min(int(n), 16 * blk + 16))
            if all(not (t < sinks or t >= n - window) for t in ts):
                table[b, blk] = -1
    assert (table == -1).sum() > (c.table == -1).sum()
    monkeypatch.setenv("PDA_DEBUG", "1")
    _say(f"debug: window {window} + {sinks} sinks, kv {kv_dtype}")
    got, _ = run_case(c, table=table, window=window, sinks=sinks)
    tol = TOL_8BIT if kv_dtype == FP8 else TOL_16BIT
    assert_parity(max_err(got, c.oracle_out(window=window, sinks=sinks)), tol)
    t2 = table.copy()
    t2[2, (2000 - 1) // 16] = -1    # the newest block is always attended
    assert _rejects(lambda: run_case(c, table=t2, window=window, sinks=sinks))


def test_debug_shared_prefix_rule(monkeypatch):
    n_shared = 21
    c = make_case(9920, pfx.CTX, n_q=8, n_kv=2, d_h=128, kv_dtype=FP8,
                  shared_prefix_blocks=n_shared)
    pl = pfx._prefix_lens(c, n_shared)
    monkeypatch.setenv("PDA_DEBUG", "1")
    _say("debug: shared prefix")
    # the rows' own entries below their prefix are unmapped (blank_prefix)
    got, _, _ = pfx._run(c, c.shared_ids, pl)
    ref, invalid, bad = pfx._oracle(c, c.shared_ids, pl)
    assert bad == 0 and not invalid.any()
    assert_parity(float(np.abs(got - ref).max()), TOL_8BIT)
    long_pl = pl.copy()
    b = int(np.argmax(pl))
    long_pl[b] = (int(c.ctx[b]) + 15) // 16     # reaches the row's newest block
    assert _rejects(lambda: pfx._run(c, c.shared_ids, long_pl))
    bad_ids = np.asarray(c.shared_ids, dtype=np.int32).copy()
    bad_ids[3] = -1
    assert _rejects(lambda: pfx._run(c, bad_ids, pl))


def test_debug_int4_open_block_not_looked_up(monkeypatch):
    import torch
    ctx = [300, 17, 40, 5, 64]
    st, ks, table, ctx, nb, mb = i4._case(9930, ctx, n_q=8, n_kv=2, d_h=128)
    r = np.random.default_rng(11)
    q_np = synth.gaussian((ctx.size, 8, 128), BF16, r)
    dev = "cuda"
    st_d, ks_d = i4._dev(st, ks, dev)
    q = to_dev(q_np, BF16, dev)
    ref, _, _, _ = oracle.paged_attn_int4(q_np, st, ks, table, ctx, 0.1, n_q=8, n_kv=2,
                                          q_dtype=BF16)
    ref = ref.reshape(ctx.size, 8, 128)
    t = table.copy()
    for b, n in enumerate(ctx):
        if n % 16:
            t[b, n // 16] = -1          # the open block lives in the residual buffer
    monkeypatch.setenv("PDA_DEBUG", "1")
    _say("debug: 4-bit open blocks")
    desc = i4._desc(ctx.size, 8, 2, 128, mb, nb, BF16, F32, ctx, 0)
    got = i4._attend(st_d, ks_d, q, t, ctx, 0.1, desc)
    assert_parity(float(np.abs(got - ref).max()), TOL_8BIT)
    t[0, 2] = -1                        # an encoded block of the 300-token row
    assert _rejects(lambda: i4._attend(st_d, ks_d, q, t, ctx, 0.1, desc))
    torch.cuda.synchronize()
