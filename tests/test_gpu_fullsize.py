"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark uses (library-chosen split, total context passed for the plan).

For each workload: inputs are drawn on the device by the seeded generators,
the library's block pool and the oracle's pool model build the tables from
the same free-list order (they must agree bit for bit), the step's new K/V are
appended by the HIP kernel (checked bit for bit against the oracle's append at
every appended slot), and the attention output of sampled rows is compared
with the fp64 oracle computed on the host copy of the drawn inputs. The
sample always includes the first and last row and every query head of one
KV group, so that all group positions and both ends of the batch are seen.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import TOL_16BIT, TOL_8BIT, assert_parity

pytestmark = pytest.mark.gpu

FULL = ["tiny_mha", "llama3_8b_layer", "llama3_70b_layer_b8_32k", "long_context_131k_sinks",
        "quant_prefix_fp8", "quant_prefix_int8", "llama3_70b_layer_b8_32k_window4k_sinks4",
        # the shared-prefix workloads again through the fused shared-prefix step
        # (each shared block read once), the benchmark's launch for them
        "quant_prefix_fp8:prefix", "quant_prefix_int8:prefix",
        "llama3_70b_layer_b8_32k_int4"]


def _raw(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _sample_rows(w, r, n=40):
    total = w.B * w.n_q
    if total <= n:
        return np.arange(total, dtype=np.int64)
    grp = [(w.B - 1) * w.n_q + h for h in range(w.n_q - w.g, w.n_q)]   # last row's last group
    pick = set([0, total - 1, *grp])
    pick.update(int(x) for x in r.choice(total, size=n - len(pick), replace=False))
    return np.array(sorted(pick), dtype=np.int64)


@pytest.mark.parametrize("name", FULL)
def test_full_size_workload(name):
    import torch
    import decode_attention_paged_slot_amd as pda

    wname, _, mode = name.partition(":")
    w = synth.WORKLOADS[wname]
    cascade = mode == "prefix"
    print(f"full-size parity: {name}", flush=True)
    sys.stdout.flush()
    dev = "cuda"
    inp = synth.make_device_inputs(w, dev)
    bs = w.block_size
    mb = int(synth.blocks_needed(inp.ctx, bs).max())

    # block tables: product pool vs the oracle's pool model, same free order
    lpool = pda.Pool(inp.num_blocks, inp.free_order)
    lsh = lpool.alloc(inp.shared_ids_count) if inp.shared_ids_count else np.empty(0, np.int32)
    ltable, lslots = lpool.build_block_table(inp.ctx, bs, mb, lsh)
    opool = oracle.OraclePool(inp.num_blocks, inp.free_order)
    osh = opool.alloc(inp.shared_ids_count) if inp.shared_ids_count else []
    table, slots = opool.build_block_table(inp.ctx, bs, mb, osh)
    assert (ltable == table).all() and (lslots == slots).all()
    assert [int(x) for x in lsh] == list(osh)

    synth.apply_sinks_device(w, inp, table)
    synth.poison_unowned_device(w, inp, table)
    torch.cuda.synchronize()
    if w.kv_dtype == synth.INT4:
        _full_size_int4(w, inp, table)
        return
    q_h, k_h, v_h = _raw(inp.q), _raw(inp.k_cache), _raw(inp.v_cache)
    kn_h, vn_h = _raw(inp.k_new), _raw(inp.v_new)
    quant = w.kv_dtype in (synth.FP8, synth.INT8)
    ks_h = vs_h = None
    if quant:
        ks_h, vs_h = inp.k_scale.cpu().numpy(), inp.v_scale.cpu().numpy()

    # the step on the GPU: append, then attend
    bt = torch.from_numpy(table).to(dev)
    cl = torch.from_numpy(inp.ctx).to(dev)
    sl = torch.from_numpy(slots).to(dev)
    out = torch.full((w.B, w.n_q, w.d_h), float("nan"), device=dev)
    desc = pda.attn_desc(inp.q, inp.k_cache, bt, max_context=int(inp.ctx.max()),
                         kv_dtype=w.kv_dtype, total_context=int(inp.ctx.sum()),
                         reuse_prefix_blocks=w.shared_prefix_tokens // w.block_size,
                         window=w.attn_window, sink_tokens=w.attn_sinks)
    if cascade:
        n_sh = inp.shared_ids_count
        nblk = synth.blocks_needed(inp.ctx, bs)
        plen = np.minimum(n_sh, np.maximum(nblk - 1, 0)).astype(np.int32)
        desc.prefix_blocks = n_sh
        desc.reuse_prefix_blocks = 0
        desc.new_dtype = synth.BF16
        ws = pda.workspace_for(desc, dev)
        pt = torch.from_numpy(np.asarray(osh, dtype=np.int32)).to(dev)
        pls = torch.from_numpy(plen).to(dev)
        pda.decode_step_prefix(inp.q, inp.k_new, inp.v_new, inp.k_cache, inp.v_cache,
                               inp.k_scale, inp.v_scale, bt, cl, pt, pls, w.softmax_scale, out,
                               desc=desc, workspace=ws)
    elif quant:
        ws = pda.workspace_for(desc, dev)
        pda.kv_append_quant(inp.k_new, inp.v_new, sl, inp.k_cache, inp.v_cache, inp.k_scale,
                            inp.v_scale, cache_dtype=w.kv_dtype)
        pda.paged_decode_attn_quant(inp.q, inp.k_cache, inp.v_cache, inp.k_scale, inp.v_scale,
                                    bt, cl, w.softmax_scale, out, desc=desc, workspace=ws)
    else:
        ws = pda.workspace_for(desc, dev)
        pda.kv_append(inp.k_new, inp.v_new, sl, inp.k_cache, inp.v_cache)
        pda.paged_decode_attn(inp.q, inp.k_cache, inp.v_cache, bt, cl, w.softmax_scale, out,
                              desc=desc, workspace=ws)
    torch.cuda.synchronize()

    # oracle append on the host copy; the appended rows must match bit for bit
    if quant:
        k2 = oracle.kv_append_quant(k_h, ks_h, synth.bf16_bits_to_f32(kn_h), slots, w.kv_dtype)
        v2 = oracle.kv_append_quant(v_h, vs_h, synth.bf16_bits_to_f32(vn_h), slots, w.kv_dtype)
    else:
        k2 = oracle.kv_append(k_h, kn_h, slots)
        v2 = oracle.kv_append(v_h, vn_h, slots)
    live = slots >= 0
    pbs = torch.from_numpy(slots[live] // bs).to(dev)
    offs = torch.from_numpy(slots[live] % bs).to(dev)
    got_k = _raw(inp.k_cache[pbs, :, offs, :])
    got_v = _raw(inp.v_cache[pbs, :, offs, :])
    sp, so = slots[live] // bs, slots[live] % bs
    assert (got_k == k2[sp, :, so, :]).all()
    assert (got_v == v2[sp, :, so, :]).all()

    rows = _sample_rows(w, np.random.default_rng(w.seed + 100))
    ref, _, _, bad = oracle.paged_attn(q_h, k2, v2, table, inp.ctx, w.softmax_scale, n_q=w.n_q,
                                       n_kv=w.n_kv, q_dtype=w.q_dtype, kv_dtype=w.kv_dtype,
                                       k_scale=ks_h, v_scale=vs_h, rows=rows,
                                       window=w.attn_window, sinks=w.attn_sinks)
    assert bad == 0
    got = out.reshape(w.B * w.n_q, w.d_h)[torch.from_numpy(rows).to(dev)].cpu().numpy()
    assert np.isfinite(got).all()
    err = float(np.abs(got.astype(np.float64) - ref).max())
    tol = TOL_8BIT if quant else TOL_16BIT
    print(f"  {name}: rows={rows.size} max-abs={err:.3g} (tol {tol}) "
          f"plan={pda.attn_plan(desc)}", flush=True)
    assert_parity(err, tol)


def _full_size_int4(w, inp, table):
    """4-bit cache: the residual-window append (state bit for bit against the
    oracle's append), then attention on sampled rows against the oracle."""
    import torch
    import decode_attention_paged_slot_amd as pda
    from oracle import int4
    dev = inp.q.device
    st = {"k": _raw(inp.k_cache), "v": _raw(inp.v_cache), "v_scale": inp.v_scale.cpu().numpy(),
          "k_res": _raw(inp.k_res), "v_res": _raw(inp.v_res)}
    ks = inp.k_scale.cpu().numpy()
    q_h, kn_h, vn_h = _raw(inp.q), _raw(inp.k_new), _raw(inp.v_new)
    bt = torch.from_numpy(table).to(dev)
    cl = torch.from_numpy(inp.ctx).to(dev)
    desc = pda.attn_desc(inp.q, inp.k_cache, bt, max_context=int(inp.ctx.max()),
                         kv_dtype=synth.INT4, total_context=int(inp.ctx.sum()),
                         new_dtype=synth.BF16)
    pda.kv_append_int4(inp.k_new, inp.v_new, bt, cl, inp.k_cache, inp.v_cache, inp.k_scale,
                       inp.v_scale, inp.k_res, inp.v_res, desc=desc)
    out = torch.full((w.B, w.n_q, w.d_h), float("nan"), device=dev)
    pda.paged_decode_attn_int4(inp.q, inp.k_cache, inp.v_cache, inp.k_scale, inp.v_scale,
                               inp.k_res, inp.v_res, bt, cl, w.softmax_scale, out, desc=desc,
                               workspace=pda.workspace_for(desc, dev))
    torch.cuda.synchronize()
    st2 = int4.kv_append_int4(st, kn_h, vn_h, table, inp.ctx, ks)
    assert (_raw(inp.k_res) == st2["k_res"]).all() and (_raw(inp.v_res) == st2["v_res"]).all()
    filled = [int(table[b, (int(n) - 1) // 16]) for b, n in enumerate(inp.ctx) if n % 16 == 0]
    print(f"  int4: {len(filled)} rows filled a block this step", flush=True)
    got_vs = inp.v_scale.cpu().numpy()
    for pb in filled:
        assert (_raw(inp.k_cache[pb]) == st2["k"][pb]).all()
        assert (_raw(inp.v_cache[pb]) == st2["v"][pb]).all()
        assert (got_vs[pb].view(np.uint32) == st2["v_scale"][pb].view(np.uint32)).all()
    rows = _sample_rows(w, np.random.default_rng(w.seed + 100))
    ref, _, _, bad = oracle.paged_attn_int4(q_h, st2, ks, table, inp.ctx, w.softmax_scale,
                                            n_q=w.n_q, n_kv=w.n_kv, q_dtype=w.q_dtype, rows=rows)
    assert bad == 0
    got = out.reshape(w.B * w.n_q, w.d_h)[torch.from_numpy(rows).to(dev)].cpu().numpy()
    assert np.isfinite(got).all()
    err = float(np.abs(got.astype(np.float64) - ref).max())
    print(f"  {w.name}: rows={rows.size} max-abs={err:.3g} (tol {TOL_8BIT}) "
          f"plan={pda.attn_plan(desc)}", flush=True)
    assert_parity(err, TOL_8BIT)
