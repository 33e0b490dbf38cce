"""Seeded random configurations against the oracle: the attention call,
the fused decode step, the shared-prefix call and the 4-bit call.

The other parity tests walk grids of one or two parameters at a time; here
each case draws every parameter at once: head dimension, KV heads, group
factor, batch, cache and query dtypes, a ragged length mix with empty and
one-token rows, the split (default plan, unsplit, or a forced wave count,
sometimes far above the block count), the host hints (exact, unknown, or one
token short), and a sliding window with sink tokens. The draws come from a
seeded generator, so a failing case is named by its index and replays
exactly.
"""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest

from synth import F32, BF16, FP8, INT8
from tests.helpers import make_case
from tests.gpu_helpers import TOL_16BIT, TOL_8BIT, assert_parity, max_err, run_case

# PDA_RANDOM_SCALE=k multiplies every case count below (a wider sweep of the
# same seeded draws; the default run keeps k = 1)
_K = max(1, int(os.environ.get("PDA_RANDOM_SCALE", "1")))
N_CASES = 48 * _K


def _draw(i: int) -> dict:
    r = np.random.default_rng(77_000 + i)
    d_h = int(r.choice([64, 128]))
    n_kv = int(r.choice([1, 2, 4, 8]))
    g = int(r.choice([g for g in (1, 2, 3, 4, 5, 8, 16) if g * n_kv <= 64]))
    B = int(r.integers(1, 10))
    kv_dtype = int(r.choice([F32, BF16, FP8, INT8]))
    q_dtype = int(r.choice([F32, BF16]))
    ctx = []
    for _ in range(B):
        u = r.random()
        if u < 0.1:
            ctx.append(0)
        elif u < 0.2:
            ctx.append(1)
        elif u < 0.3:
            ctx.append(16 * int(r.integers(1, 120)))           # whole blocks
        else:
            ctx.append(int(r.integers(2, 3000)))
    if max(ctx) == 0:
        ctx[0] = int(r.integers(1, 500))
    nw = int(r.choice([0, 0, 1, int(r.integers(2, 65)), 300]))
    hint = str(r.choice(["exact", "unknown", "short"]))
    window = sinks = 0
    if r.random() < 0.25:
        window = int(r.integers(1, 600))
        sinks = int(r.choice([0, 0, 4, int(r.integers(1, 40))]))
    return dict(d_h=d_h, n_kv=n_kv, g=g, B=B, kv_dtype=kv_dtype, q_dtype=q_dtype, ctx=ctx,
                nw=nw, hint=hint, window=window, sinks=sinks)


def test_draws_cover_the_space():
    """The case list reaches every dtype, both head dims, the empty and
    one-token rows, windows, forced splits and every hint setting."""
    ds = [_draw(i) for i in range(N_CASES)]
    assert {d["kv_dtype"] for d in ds} == {F32, BF16, FP8, INT8}
    assert {d["q_dtype"] for d in ds} == {F32, BF16}
    assert {d["d_h"] for d in ds} == {64, 128}
    assert {d["hint"] for d in ds} == {"exact", "unknown", "short"}
    assert any(0 in d["ctx"] for d in ds) and any(1 in d["ctx"] for d in ds)
    assert any(d["window"] for d in ds) and any(d["nw"] == 300 for d in ds)
    assert any(d["nw"] == 0 for d in ds) and any(d["nw"] == 1 for d in ds)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_configuration(i):
    d = _draw(i)
    print(f"random case {i}: {d}", flush=True)
    sys.stdout.flush()
    n_max = max(d["ctx"])
    c = make_case(78_000 + i, d["ctx"], n_q=d["g"] * d["n_kv"], n_kv=d["n_kv"], d_h=d["d_h"],
                  kv_dtype=d["kv_dtype"], q_dtype=d["q_dtype"])
    mc = {"exact": n_max, "unknown": n_max, "short": max(n_max - 1, 0)}[d["hint"]]
    tc = {"exact": int(sum(d["ctx"])), "unknown": 0, "short": int(sum(d["ctx"]))}[d["hint"]]
    got, _ = run_case(c, max_context=mc, total_context=tc, num_partitions=d["nw"],
                      window=d["window"], sinks=d["sinks"])
    ref = c.oracle_out(window=d["window"], sinks=d["sinks"])
    empty = [b for b, n in enumerate(d["ctx"]) if n == 0]
    assert (got[empty] == 0).all()
    keep = [b for b, n in enumerate(d["ctx"]) if n > 0]
    tol = TOL_8BIT if d["kv_dtype"] in (FP8, INT8) else TOL_16BIT
    assert_parity(max_err(got[keep], ref[keep]), tol)


N_STEP_CASES = 16 * _K


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_STEP_CASES))
def test_random_fused_step(i):
    """The fused decode step (append each row's new K/V at position n - 1,
    then attend) on random configurations: the caches equal the oracle's
    append bit for bit, and the output the oracle's attention over them."""
    import torch
    import decode_attention_paged_slot_amd as pda
    import oracle
    import synth

    d = _draw(1000 + i)
    kv_dtype = (BF16, FP8, INT8)[i % 3]
    # a 16-bit cache takes new rows of its own dtype; an 8-bit one encodes
    # fp32 or bf16 rows
    new_dtype = BF16 if kv_dtype == BF16 else (BF16, F32)[(i // 3) % 2]
    print(f"random fused step {i}: kv={kv_dtype} new={new_dtype} {d}", flush=True)
    sys.stdout.flush()
    c = make_case(79_000 + i, d["ctx"], n_q=d["g"] * d["n_kv"], n_kv=d["n_kv"], d_h=d["d_h"],
                  kv_dtype=kv_dtype, q_dtype=d["q_dtype"])
    r = np.random.default_rng(80_000 + i)
    kn = synth.gaussian((c.B, c.n_kv, c.d_h), new_dtype, r)
    vn = synth.gaussian((c.B, c.n_kv, c.d_h), new_dtype, r)
    dev = "cuda"
    from tests.gpu_helpers import to_dev
    quant = kv_dtype in (FP8, INT8)
    q = to_dev(c.q, c.q_dtype, dev)
    k = to_dev(c.k, kv_dtype, dev)
    v = to_dev(c.v, kv_dtype, dev)
    bt = torch.from_numpy(c.table).to(dev)
    cl = torch.from_numpy(c.ctx).to(dev)
    dkn, dvn = to_dev(kn, new_dtype, dev), to_dev(vn, new_dtype, dev)
    n_max = int(c.ctx.max())
    desc = pda.AttnDesc(c.B, c.n_q, c.n_kv, c.d_h, c.bs, bt.shape[1], c.k.shape[0], kv_dtype,
                        c.q_dtype, F32, n_max, d["nw"], int(c.ctx.sum()), 0, d["window"],
                        d["sinks"], new_dtype)
    ws = pda.workspace_for(desc, dev)
    out = torch.full((c.B, c.n_q, c.d_h), float("nan"), device=dev)
    if quant:
        ks = torch.from_numpy(c.k_scale).to(dev)
        vs = torch.from_numpy(c.v_scale).to(dev)
        pda.decode_step_quant(q, dkn, dvn, k, v, ks, vs, bt, cl, c.scale, out, desc=desc,
                              workspace=ws)
    else:
        pda.decode_step(q, dkn, dvn, k, v, bt, cl, c.scale, out, desc=desc, workspace=ws)
    torch.cuda.synchronize()
    kf = oracle.decode(kn, new_dtype).astype(np.float32)
    vf = oracle.decode(vn, new_dtype).astype(np.float32)
    if quant:
        k2 = oracle.kv_append_quant(c.k, c.k_scale, kf, c.slots, kv_dtype)
        v2 = oracle.kv_append_quant(c.v, c.v_scale, vf, c.slots, kv_dtype)
    else:
        k2 = oracle.kv_append(c.k, kn, c.slots)
        v2 = oracle.kv_append(c.v, vn, c.slots)
    assert (k.view(torch.uint8).cpu().numpy().reshape(-1) ==
            np.ascontiguousarray(k2).view(np.uint8).reshape(-1)).all()
    assert (v.view(torch.uint8).cpu().numpy().reshape(-1) ==
            np.ascontiguousarray(v2).view(np.uint8).reshape(-1)).all()
    ref, _, _, bad = oracle.paged_attn(c.q, k2, v2, c.table, c.ctx, c.scale, n_q=c.n_q,
                                       n_kv=c.n_kv, q_dtype=c.q_dtype, kv_dtype=kv_dtype,
                                       k_scale=c.k_scale, v_scale=c.v_scale,
                                       window=d["window"], sinks=d["sinks"])
    assert bad == 0
    got = out.cpu().numpy().reshape(-1, c.d_h)
    keep = np.repeat(c.ctx > 0, c.n_q)
    assert (got[~keep] == 0).all()
    assert_parity(max_err(got[keep], ref[keep]), (TOL_8BIT if quant else TOL_16BIT))


N_PREFIX_CASES = 16 * _K


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_PREFIX_CASES))
def test_random_shared_prefix(i):
    """The shared-prefix call on random configurations: a random number of
    shared blocks (one chunk or several, with a partial last chunk), each
    row's prefix length drawn up to its own limit (zero included), the rows'
    own prefix entries unmapped, against the oracle over the prefix table."""
    from tests import test_gpu_prefix as pfx

    d = _draw(2000 + i)
    r = np.random.default_rng(81_000 + i)
    kv_dtype = (BF16, FP8, INT8)[i % 3]
    n_shared = int(r.integers(1, 60))
    ctx = [max(n, 1) for n in d["ctx"]]
    ctx[0] = max(ctx[0], 16 * n_shared + 1)          # one row can hold the whole prefix
    print(f"random shared prefix {i}: kv={kv_dtype} shared={n_shared} {d}", flush=True)
    sys.stdout.flush()
    c = make_case(82_000 + i, ctx, n_q=d["g"] * d["n_kv"], n_kv=d["n_kv"], d_h=d["d_h"],
                  kv_dtype=kv_dtype, q_dtype=d["q_dtype"], shared_prefix_blocks=n_shared)
    top = pfx._prefix_lens(c, n_shared)
    pl = np.array([int(r.integers(0, t + 1)) for t in top], dtype=np.int32)
    pl[0] = top[0]
    got, _, _ = pfx._run(c, c.shared_ids, pl, nw=d["nw"])
    ref, invalid, bad = pfx._oracle(c, c.shared_ids, pl)
    assert bad == 0 and not invalid.any()
    tol = TOL_8BIT if kv_dtype in (FP8, INT8) else TOL_16BIT
    assert_parity(max_err(got, ref), tol)


N_INT4_CASES = 12 * _K


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_INT4_CASES))
def test_random_int4_attention(i):
    """4-bit attention (encoded blocks plus each row's residual window) on
    random configurations, with NaN-poisoned blocks and residual slots that
    must not be read, against the oracle."""
    import oracle
    import synth
    from tests import test_gpu_int4 as i4
    from tests.gpu_helpers import to_dev

    d = _draw(3000 + i)
    print(f"random 4-bit {i}: {d}", flush=True)
    sys.stdout.flush()
    n_q = d["g"] * d["n_kv"]
    st, ks, table, ctx, nb, mb = i4._case(83_000 + i, d["ctx"], n_q=n_q, n_kv=d["n_kv"],
                                          d_h=d["d_h"])
    r = np.random.default_rng(84_000 + i)
    q_np = synth.gaussian((ctx.size, n_q, d["d_h"]), d["q_dtype"], r)
    st_d, ks_d = i4._dev(st, ks, "cuda")
    q = to_dev(q_np, d["q_dtype"], "cuda")
    scale = 1.0 / np.sqrt(d["d_h"])
    got = i4._attend(st_d, ks_d, q, table, ctx, scale,
                     i4._desc(ctx.size, n_q, d["n_kv"], d["d_h"], mb, nb, d["q_dtype"], F32,
                              ctx, d["nw"]))
    ref, _, _, bad = oracle.paged_attn_int4(q_np, st, ks, table, ctx, scale, n_q=n_q,
                                            n_kv=d["n_kv"], q_dtype=d["q_dtype"])
    assert bad == 0
    ref = ref.reshape(got.shape)
    empty = ctx == 0
    assert (got[empty] == 0).all()
    assert_parity(max_err(got[~empty], ref[~empty]), TOL_8BIT)


N_INT4_STEP_CASES = 8 * _K


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_INT4_STEP_CASES))
def test_random_int4_fused_step(i):
    """The fused 4-bit decode step on random configurations (a third of the
    rows complete a block this step): output, codes, value scales and
    residual buffers bit for bit against the append followed by the
    attention call, and the output against the oracle."""
    import torch
    import oracle
    import synth
    import decode_attention_paged_slot_amd as pda
    from oracle import int4
    from tests import test_gpu_int4 as i4
    from tests.gpu_helpers import to_dev

    d = _draw(5000 + i)
    ctx = [(c + 15) // 16 * 16 if k % 3 == 0 and c > 0 else c for k, c in enumerate(d["ctx"])]
    print(f"random fused 4-bit {i}: {d} lengths {ctx}", flush=True)
    sys.stdout.flush()
    n_q, n_kv, d_h = d["g"] * d["n_kv"], d["n_kv"], d["d_h"]
    st, ks, table, ctx, nb, mb = i4._case(85_000 + i, ctx, n_q=n_q, n_kv=n_kv, d_h=d_h,
                                          poison=False)
    r = np.random.default_rng(86_000 + i)
    dev = "cuda"
    q_np = synth.gaussian((ctx.size, n_q, d_h), d["q_dtype"], r)
    kn_np = synth.gaussian((ctx.size, n_kv, d_h), BF16, r)
    vn_np = synth.gaussian((ctx.size, n_kv, d_h), BF16, r)
    a_d, ks_d = i4._dev(st, ks, dev)
    b_d, _ = i4._dev(st, ks, dev)
    q = to_dev(q_np, d["q_dtype"], dev)
    kn, vn = to_dev(kn_np, BF16, dev), to_dev(vn_np, BF16, dev)
    bt, ct = torch.from_numpy(table).to(dev), torch.from_numpy(ctx).to(dev)
    desc = i4._desc(ctx.size, n_q, n_kv, d_h, mb, nb, d["q_dtype"], F32, ctx, d["nw"])
    scale = 1.0 / np.sqrt(d_h)
    out_a = torch.full((ctx.size, n_q, d_h), 7.0, device=dev)
    out_b = torch.full((ctx.size, n_q, d_h), -7.0, device=dev)
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
        return x.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[x.element_size()]).cpu().numpy()

    assert (bits(out_a) == bits(out_b)).all()
    for key in ("k", "v", "v_scale", "k_res", "v_res"):
        assert (bits(a_d[key]) == bits(b_d[key])).all(), key
    st = int4.kv_append_int4(st, kn_np, vn_np, table, ctx, ks)
    ref, _, _, bad = oracle.paged_attn_int4(q_np, st, ks, table, ctx, scale, n_q=n_q, n_kv=n_kv,
                                            q_dtype=d["q_dtype"])
    assert bad == 0
    got = out_b.cpu().numpy()
    ref = ref.reshape(got.shape)
    empty = ctx == 0
    assert (got[empty] == 0).all()
    assert_parity(max_err(got[~empty], ref[~empty]), TOL_8BIT)
