#!/usr/bin/env python3
"""Decode-step benchmark for paged single-token decode attention on MI355X.

One step = one decode step of one attention layer over a whole batch: the
step's new K/V rows are appended into their mapped cache slots, then every
sequence's query attends over its paged cache (split-KV partitions and their
log-sum-exp merge included). By default the step is one fused
pda_decode_step call; --two-calls runs pda_kv_append then
pda_paged_decode_attn, with bit-identical results. Inputs are seeded
synthetic tensors drawn in HBM before the timed region; nothing is copied
between host and device inside it. Every library call is bound once (its
arguments marshalled up front), so a launch costs one ctypes call.

Default workload: the Llama-3-70B layer shape on one GPU -- batch 8, 64 query
heads over 8 KV heads (GQA g = 8), d_h 128, bf16 cache, every context 32,768
tokens, block size 16, physical blocks placed at random in a pool with 10%
free (NaN-poisoned) blocks. The default run also measures the long-context
row (batch 1, 131,072 tokens, four sink keys x8) the same way and reports it
under "long_context". The byte counts follow the SoK paper's appendix A.1
accounting (cache read once, no score spill) in decimal units (appendix C.2).

Timing: K steps, each after a 1 GiB write that evicts the L2s and the 256 MB
Infinity Cache, with HIP events on the launch stream around the step only;
value, ms_per_step and the roofline use the median (p10 / p90 beside it).
The same calls back to back ("warm") are reported as secondary figures.

Printed: one JSON line with the metric (KV GB/s of the step), ms/step, the
roofline object (algorithmic bytes per step over the median step against
8 TB/s), the HBM read probes of this device (sequential, and this
workload's own K/V tiles in the kernel's order), and the CPU baseline (the
fp64 oracle on the host's cores over the same workload). The oracle output
is also compared with the GPU output row by row (parity at full size).

    python bench.py [--gpus 1] [--steps 60] [--warmup 20] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor figure (decimal GB/s)
DEFAULT_WORKLOAD = "llama3_70b_layer_b8_32k"


def _say(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def _pct(xs, q):
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q))


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60,
                    help="timed steps, each after a 1 GiB cache-evicting write")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle", type=float, default=0.1,
                    help="seconds of untimed steps before the warmup (clock ramp)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-oracle", action="store_true",
                    help="skip the CPU oracle leg (parity + cpu_baseline)")
    ap.add_argument("--no-probe", action="store_true", help="skip the HBM read probes")
    ap.add_argument("--no-long", action="store_true",
                    help="default workload only: skip the long-context (131k) measurement")
    ap.add_argument("--num-partitions", type=int, default=0,
                    help="split-KV partitions (0 = the library's choice)")
    ap.add_argument("--two-calls", dest="fused", action="store_false", default=True,
                    help="pda_kv_append + pda_paged_decode_attn per step instead of one fused "
                         "pda_decode_step launch (the default; identical results)")
    ap.add_argument("--no-prefix-pass", dest="prefix_pass", action="store_false", default=True,
                    help="shared-prefix workloads: every row reads the shared blocks itself "
                         "(with the cache-retaining hint) instead of the *_prefix calls that "
                         "read each shared block once for all rows")
    ap.add_argument("--graph", dest="graph", action="store_true", default=False,
                    help="replay the step from a captured HIP graph (eager launches by "
                         "default: on this stack a replay adds ~6 us per step)")
    ap.add_argument("--sweep", action="store_true", default=False,
                    help="also time the attention call at 1/4, 1/2 and 2x the workload's "
                         "context lengths and fit us = fixed + bytes / rate: the kernel's "
                         "steady streaming rate apart from its fixed per-call cost (workloads "
                         "whose bytes scale with context: no window, shared prefix or 4-bit)")
    return ap.parse_args(argv)


def build_inputs(w, dev):
    """Seeded device inputs, the product's block table, poison and sinks."""
    import torch  # noqa: F401
    import synth
    import decode_attention_paged_slot_amd as pda

    inp = synth.make_device_inputs(w, dev)
    bs = w.block_size
    max_blocks = int(synth.blocks_needed(inp.ctx, bs).max())
    pool = pda.Pool(inp.num_blocks, inp.free_order)
    shared = pool.alloc(inp.shared_ids_count) if inp.shared_ids_count else np.empty(0, np.int32)
    table, slots = pool.build_block_table(inp.ctx, bs, max_blocks, shared)
    synth.apply_sinks_device(w, inp, table)
    synth.poison_unowned_device(w, inp, table)
    return inp, pool, shared, table, slots


def context_sweep(w, dev, reps, factors=(0.25, 0.5, 2.0)):
    """Attention-call time at scaled context lengths of workload `w` (same
    shape, seed and structure otherwise): [(factor, attention bytes, us)].
    Each point is the median of 5 runs of `reps` back-to-back calls between
    two HIP events on the launch stream."""
    import torch
    import synth
    import decode_attention_paged_slot_amd as pda
    from decode_attention_paged_slot_amd import accounting as acc

    pts = []
    for f in factors:
        w2 = w.with_(ctx_lo=max(1, int(round(w.ctx_lo * f))), ctx_hi=max(1, int(round(w.ctx_hi * f))))
        inp, pool, _, table, _ = build_inputs(w2, dev)
        bt = torch.from_numpy(table).to(dev)
        cl = torch.from_numpy(inp.ctx).to(dev)
        out = torch.empty((w2.B, w2.n_q, w2.d_h), dtype=torch.float32, device=dev)
        desc = pda.attn_desc(inp.q, inp.k_cache, bt, max_context=int(inp.ctx.max()),
                             kv_dtype=w2.kv_dtype, total_context=int(inp.ctx.sum()))
        ws = pda.workspace_for(desc, dev)
        if w2.kv_dtype in (synth.FP8, synth.INT8):
            def call():
                pda.paged_decode_attn_quant(inp.q, inp.k_cache, inp.v_cache, inp.k_scale,
                                            inp.v_scale, bt, cl, w2.softmax_scale, out,
                                            desc=desc, workspace=ws)
        else:
            def call():
                pda.paged_decode_attn(inp.q, inp.k_cache, inp.v_cache, bt, cl,
                                      w2.softmax_scale, out, desc=desc, workspace=ws)
        for _ in range(20):
            call()
        torch.cuda.synchronize()
        per = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                call()
            b.record()
            torch.cuda.synchronize()
            per.append(a.elapsed_time(b) * 1e3 / reps)
        nbytes = acc.step_bytes(inp.ctx, n_q=w2.n_q, n_kv=w2.n_kv, d_h=w2.d_h,
                                block_size=w2.block_size, kv_dtype=w2.kv_dtype,
                                q_dtype=w2.q_dtype, new_dtype=synth.BF16).attention
        pts.append((f, int(nbytes), float(np.median(per))))
        _say(f"[bench] sweep x{f}: {nbytes / 1e9:.3f} GB in {pts[-1][2]:.2f} us")
        pool.close()
        del inp, bt, cl, out, ws
        torch.cuda.empty_cache()
    return pts


def oracle_leg(w, inp, table, slots, shared, host):
    """fp64 oracle over the whole workload on the host cores.

    The oracle's inputs are the seeded cache as drawn (copied to the host
    before any library kernel touched it), the step's new rows placed by the
    oracle's own append, and block tables from the oracle's own pool model
    (checked equal to the library's). Returns (timing dict, oracle out)."""
    import oracle
    import synth

    opool = oracle.OraclePool(inp.num_blocks, inp.free_order)
    osh = opool.alloc(inp.shared_ids_count) if inp.shared_ids_count else []
    otable, oslots = opool.build_block_table(inp.ctx, w.block_size, table.shape[1], osh)
    tables_equal = bool((otable == table).all() and (oslots == slots).all()
                        and list(osh) == [int(x) for x in shared])
    if w.kv_dtype == 4:
        # 4-bit cache: the oracle's residual-window append, then attention
        from oracle import int4
        st = int4.kv_append_int4({"k": host["k"], "v": host["v"], "v_scale": host["vs"],
                                  "k_res": host["k_res"], "v_res": host["v_res"]},
                                 host["kn_raw"], host["vn_raw"], otable, inp.ctx, host["ks"])
        t0 = time.perf_counter()
        out, _, _, bad = oracle.paged_attn_int4(host["q"], st, host["ks"], otable, inp.ctx,
                                                w.softmax_scale, n_q=w.n_q, n_kv=w.n_kv,
                                                q_dtype=w.q_dtype)
        secs = time.perf_counter() - t0
        return {"secs": secs, "threads": oracle.num_threads(), "bad_rows": bad,
                "tables_equal": tables_equal}, out
    k = oracle.kv_append(host["k"], host["kn_raw"], oslots) if w.kv_dtype in (0, 1) else \
        oracle.kv_append_quant(host["k"], host["ks"], host["kn_f32"], oslots, w.kv_dtype)
    v = oracle.kv_append(host["v"], host["vn_raw"], oslots) if w.kv_dtype in (0, 1) else \
        oracle.kv_append_quant(host["v"], host["vs"], host["vn_f32"], oslots, w.kv_dtype)
    t0 = time.perf_counter()
    out, _, _, bad = oracle.paged_attn(host["q"], k, v, otable, inp.ctx, w.softmax_scale,
                                       n_q=w.n_q, n_kv=w.n_kv, q_dtype=w.q_dtype,
                                       kv_dtype=w.kv_dtype, k_scale=host.get("ks"),
                                       v_scale=host.get("vs"), window=w.attn_window,
                                       sinks=w.attn_sinks)
    secs = time.perf_counter() - t0
    del k, v
    return {"secs": secs, "threads": oracle.num_threads(), "bad_rows": bad,
            "tables_equal": tables_equal}, out


def host_snapshot(w, inp):
    """Host copies of the drawn inputs (raw storage) for the oracle leg."""
    import torch
    import synth

    def raw(t):
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()

    h = {"q": raw(inp.q), "k": raw(inp.k_cache), "v": raw(inp.v_cache)}
    kn, vn = raw(inp.k_new), raw(inp.v_new)
    h["kn_raw"], h["vn_raw"] = kn, vn
    if w.kv_dtype in (2, 3, 4):
        h["ks"], h["vs"] = inp.k_scale.cpu().numpy(), inp.v_scale.cpu().numpy()
        h["kn_f32"] = synth.bf16_bits_to_f32(kn)
        h["vn_f32"] = synth.bf16_bits_to_f32(vn)
    if w.kv_dtype == 4:
        h["k_res"], h["v_res"] = raw(inp.k_res), raw(inp.v_res)
    return h


def _events(n):
    import torch
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n)]


def read_probe(dev, table, ctx, w, scratch, reps=10, sequential=True):
    """Read-only HBM probes (pda_hbm_read_probe), GB/s: a sequential walk of
    2 GiB (2048 waves), and the (block, head) K and V tiles of this workload
    read in the attention kernel's order (segment by segment, K then V per
    block, four tiles in flight, with the kernel's wave count: 1024 for bf16
    caches, 2048 for 8-bit and 4-bit ones), from a buffer laid out like the
    two caches (the 4-bit value scales are not read). A tile several rows
    share (a shared prefix) is read once, where it first appears, so the
    probe moves the unique bytes the steps are rated on. Each figure is the
    median of 5 runs of `reps` back-to-back launches between two HIP
    events; the tile probe is also timed as the steps are, each run after a
    1 GiB write of `scratch` (median of 20, `kv_tiles_flushed_*`)."""
    import torch
    import synth
    import decode_attention_paged_slot_amd as pda

    def timed(call):
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        per = []
        for _ in range(5):
            (a, b), = _events(1)
            a.record()
            for _ in range(reps):
                call()
            b.record()
            torch.cuda.synchronize()
            per.append(a.elapsed_time(b) / reps)
        return float(np.median(per))

    out = {}
    if sequential:
        seq_bytes = 2 << 30
        buf = torch.empty(seq_bytes // 4, dtype=torch.int32, device=dev).fill_(1)
        sink = torch.empty(2048 * 64, dtype=torch.int32, device=dev)
        ms = timed(pda.hbm_read_probe(buf, sink, waves=2048, bind=True))
        out["sequential_GBps"] = round(seq_bytes / (ms * 1e-3) / 1e9, 1)
        del buf
    if w.kv_dtype in (synth.BF16, synth.FP8, synth.INT8, synth.INT4) and not w.attn_window:
        eb = synth.ELEM_BYTES[w.kv_dtype]
        waves = 1024 if w.kv_dtype == synth.BF16 else 2048
        tile = int(16 * w.d_h * eb)                    # one (block, head) tile
        blk = w.n_kv * tile                            # one physical block, all heads
        nblk = synth.blocks_needed(ctx, w.block_size)
        nb_pool = int(table.max()) + 1
        offs = []
        seen = np.zeros(nb_pool, bool)
        for b in range(w.B):
            ids = table[b, :nblk[b]].astype(np.int64)
            ids = ids[ids >= 0]
            ids = ids[~seen[ids]]
            seen[ids] = True
            for j in range(w.n_kv):
                k = ids * blk + j * tile
                offs.append(np.stack([k, k + nb_pool * blk], 1).reshape(-1))
        offs = np.concatenate(offs)
        buf = torch.empty(2 * nb_pool * blk // 4, dtype=torch.int32, device=dev).fill_(1)
        t_off = torch.from_numpy(offs).to(dev)
        sink = torch.empty(waves * 64, dtype=torch.int32, device=dev)
        call = pda.hbm_read_probe(buf, sink, tile_offsets=t_off, tile_bytes=tile, waves=waves,
                                  bind=True)
        ms = timed(call)
        out["kv_tiles_GBps"] = round(offs.size * tile / (ms * 1e-3) / 1e9, 1)
        out["kv_tiles_us"] = round(ms * 1e3, 2)
        ms_f = float(np.median(flushed_calls(call, 20, scratch)))
        out["kv_tiles_flushed_GBps"] = round(offs.size * tile / (ms_f * 1e-3) / 1e9, 1)
        out["kv_tiles_flushed_us"] = round(ms_f * 1e3, 2)
        out["kv_tiles_bytes"] = int(offs.size * tile)
        del buf, t_off
    torch.cuda.empty_cache()
    return out


# Sources whose code decides what the attention call moves; a counter summary
# under profiles/ is only used while they hash to the value it records.
ATTN_SOURCES = ("attn_mfma.hip", "attn_prefix.hip", "attn_f32.hip", "merge.hip",
                "append_int4.hip", "device_common.h", "pda_internal.h", "api.cpp")


def code_tokens(text: str) -> str:
    """C / C++ source with comments removed and whitespace runs collapsed, so
    that the hash below follows the code, not its comments or layout. String
    and character literals are kept as written."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def attn_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in ATTN_SOURCES:
        with open(os.path.join(ROOT, "decode_attention_paged_slot_amd", "csrc", name)) as f:
            h.update(name.encode() + b"\0" + code_tokens(f.read()).encode())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per attention call from the committed rocprofv3 counter
    summary of this workload (FETCH_SIZE and WRITE_SIZE passes, calibrated),
    or None when there is none or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", f"paged_decode_attn__{workload}__pmc.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    try:
        if fields.get("source_sha256") != attn_source_hash():
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


LONG_WORKLOAD = "long_context_131k_sinks"


def setup_calls(w, args, dev, inp, shared, table, slots):
    """The workload's step, append and attention calls, each bound once
    (arguments marshalled up front, so a launch costs one ctypes call)."""
    import torch
    import synth
    import decode_attention_paged_slot_amd as pda

    quant = w.kv_dtype in (synth.FP8, synth.INT8)
    int4 = w.kv_dtype == synth.INT4
    bt = torch.from_numpy(table).to(dev)
    cl = torch.from_numpy(inp.ctx).to(dev)
    sl = torch.from_numpy(slots).to(dev)
    out = torch.empty((w.B, w.n_q, w.d_h), dtype=torch.float32, device=dev)
    # shared prompt prefix: by default the *_prefix calls read each shared
    # block once for all rows; otherwise every row reads them, hinted to stay
    # in cache after the first read
    n_sh = int(inp.shared_ids_count)
    cascade = args.prefix_pass and n_sh > 0
    reuse = 0 if cascade else w.shared_prefix_tokens // w.block_size
    new_dtype = synth.F32 if w.kv_dtype == synth.F32 else synth.BF16
    desc = pda.attn_desc(inp.q, inp.k_cache, bt, max_context=int(inp.ctx.max()),
                         kv_dtype=w.kv_dtype, num_partitions=args.num_partitions,
                         total_context=int(inp.ctx.sum()), reuse_prefix_blocks=reuse,
                         window=w.attn_window, sink_tokens=w.attn_sinks,
                         prefix_blocks=n_sh if cascade else 0, new_dtype=new_dtype)
    pt = pls = None
    if cascade:
        nblk = synth.blocks_needed(inp.ctx, w.block_size)
        pt = torch.from_numpy(np.asarray(shared, dtype=np.int32)).to(dev)
        pls = torch.from_numpy(np.minimum(n_sh, np.maximum(nblk - 1, 0)).astype(np.int32)).to(dev)
    ws = pda.workspace_for(desc, dev)
    scale = w.softmax_scale
    kc, vc, ks, vs = inp.k_cache, inp.v_cache, inp.k_scale, inp.v_scale
    if int4:
        append = pda.kv_append_int4(inp.k_new, inp.v_new, bt, cl, kc, vc, ks, vs, inp.k_res,
                                    inp.v_res, desc=desc, bind=True)
        attend = pda.paged_decode_attn_int4(inp.q, kc, vc, ks, vs, inp.k_res, inp.v_res, bt, cl,
                                            scale, out, desc=desc, workspace=ws, bind=True)
    else:
        if quant:
            append = pda.kv_append_quant(inp.k_new, inp.v_new, sl, kc, vc, ks, vs,
                                         cache_dtype=w.kv_dtype, bind=True)
        else:
            append = pda.kv_append(inp.k_new, inp.v_new, sl, kc, vc, bind=True)
        if cascade:
            attend = pda.paged_decode_attn_prefix(inp.q, kc, vc, ks, vs, bt, cl, pt, pls, scale,
                                                  out, desc=desc, workspace=ws, bind=True)
        elif quant:
            attend = pda.paged_decode_attn_quant(inp.q, kc, vc, ks, vs, bt, cl, scale, out,
                                                 desc=desc, workspace=ws, bind=True)
        else:
            attend = pda.paged_decode_attn(inp.q, kc, vc, bt, cl, scale, out, desc=desc,
                                           workspace=ws, bind=True)
    fused = args.fused
    if fused:
        # one launch: each row's new K/V land at position n - 1, then attention
        # (4-bit: the attention launch also does the append, then the merge)
        if int4:
            step1 = pda.decode_step_int4(inp.q, inp.k_new, inp.v_new, kc, vc, ks, vs, inp.k_res,
                                         inp.v_res, bt, cl, scale, out, desc=desc, workspace=ws,
                                         bind=True)
        elif cascade:
            step1 = pda.decode_step_prefix(inp.q, inp.k_new, inp.v_new, kc, vc, ks, vs, bt, cl,
                                           pt, pls, scale, out, desc=desc, workspace=ws,
                                           bind=True)
        elif quant:
            step1 = pda.decode_step_quant(inp.q, inp.k_new, inp.v_new, kc, vc, ks, vs, bt, cl,
                                          scale, out, desc=desc, workspace=ws, bind=True)
        else:
            step1 = pda.decode_step(inp.q, inp.k_new, inp.v_new, kc, vc, bt, cl, scale, out,
                                    desc=desc, workspace=ws, bind=True)
        step = step1
    else:
        def step():
            append()
            attend()
    P, bpp = pda.attn_plan(desc)
    return {"step": step, "append": append, "attend": attend, "out": out, "fused": fused,
            "cascade": cascade, "reuse": reuse, "n_sh": n_sh, "P": P, "bpp": bpp,
            "keep": (bt, cl, sl, ws, pt, pls, desc)}


def timed_b2b(fn, reps):
    """Average duration of `reps` back-to-back calls between two HIP events on
    the launch stream, repeated 5 times: [ms per call]."""
    import torch
    per = []
    for _ in range(5):
        (a, b), = _events(1)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b) / reps)
    return per


def flushed_calls(fn, iters, scratch):
    """`iters` calls, each after a 1 GiB write of `scratch` that evicts the
    L2s and the 256 MB Infinity Cache; HIP events around each call only (the
    flush is outside them). Everything is queued without host waits, so the
    events see the GPU's own time. [ms per call]"""
    import torch
    ev = _events(iters)
    for a, b in ev:
        scratch.fill_(1.0)
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def settle(fn, seconds, warmup):
    """Clock settle (untimed): MI355X takes ~15-20 ms of sustained work to
    reach its steady clocks; the first calls of a cold GPU run up to 1.5x
    slower. Calls run until `seconds` have passed, then `warmup` more."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()


def step_bytes_of(w, inp):
    import synth
    from decode_attention_paged_slot_amd import accounting as acc
    return acc.step_bytes(inp.ctx, n_q=w.n_q, n_kv=w.n_kv, d_h=w.d_h, block_size=w.block_size,
                          kv_dtype=w.kv_dtype, q_dtype=w.q_dtype,
                          new_dtype=synth.BF16 if w.kv_dtype != synth.F32 else synth.F32,
                          shared_prefix_blocks=inp.shared_ids_count, window=w.attn_window,
                          sinks=w.attn_sinks)


def _cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def parity_and_cpu(w, inp, table, slots, shared, host, out, att_bytes):
    """Full-size parity of this run's output against the fp64 oracle, and the
    oracle's own rate on the host cores (the CPU baseline)."""
    import torch
    import synth
    quant = w.kv_dtype in (synth.FP8, synth.INT8, synth.INT4)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(w.B * w.n_q, w.d_h).astype(np.float64)
    info, ref = oracle_leg(w, inp, table, slots, shared, host)
    tol = 3e-2 if quant else 5e-3
    err = float(np.abs(got - ref).max()) if np.isfinite(got).all() else float("inf")
    parity = {"rows": int(ref.shape[0]), "max_abs_err": err, "tol": tol,
              "pass": bool(err < tol and info["bad_rows"] == 0 and info["tables_equal"]),
              "block_tables_identical": info["tables_equal"]}
    cpu = {"value": round(att_bytes / info["secs"] / 1e9, 4), "unit": "GB/s",
           "cores": int(info["threads"]), "kind": "oracle", "cpu_model": _cpu_model(),
           "sample": (f"whole workload {w.name} ({w.B} sequences x {w.n_q} query heads, "
                      f"{int(inp.ctx.sum())} cached tokens"
                      + (f", window {w.attn_window} + {w.attn_sinks} sinks"
                         if w.attn_window else "")
                      + f"); fp64 two-pass oracle, "
                      f"{info['secs']:.2f} s wall on {info['threads']} threads")}
    _say(f"[bench] {w.name}: parity max-abs {err:.3g} (tol {tol}); oracle {info['secs']:.2f} s")
    return parity, cpu


def measure(w, args, dev, K, scratch, with_oracle):
    """Build the workload, time it and check it. Returns a dict of figures."""
    import torch
    import synth

    _say(f"[bench] workload {w.name}: drawing inputs")
    inp, pool, shared, table, slots = build_inputs(w, dev)
    host = host_snapshot(w, inp) if with_oracle else None
    c = setup_calls(w, args, dev, inp, shared, table, slots)
    _say(f"[bench] {w.name}: plan P={c['P']} blocks/partition={c['bpp']}; settle "
         f"{args.settle} s, warmup {args.warmup}")
    settle(c["step"], args.settle, args.warmup)

    graph = None
    if args.graph:
        # one decode step captured as a HIP graph and replayed: the launches
        # are issued by the GPU's command processor without a host round trip
        s_cap = torch.cuda.Stream()
        s_cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s_cap):
            c["step"]()
        torch.cuda.current_stream().wait_stream(s_cap)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            c["step"]()
        torch.cuda.synchronize()
        for _ in range(max(args.warmup, 1)):
            graph.replay()
        torch.cuda.synchronize()
    run_step = graph.replay if graph is not None else c["step"]

    # the timed steps: each after a cache-evicting flush, HIP events around
    # the step itself
    _say(f"[bench] {w.name}: timing {K} flushed steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step_ms = flushed_calls(run_step, K, scratch)
    wall = time.perf_counter() - t0
    # secondary figures: the same calls back to back (caches warm), the
    # attention call alone (flushed and warm), the append alone
    warm_step = timed_b2b(run_step, K)
    att_cold = flushed_calls(c["attend"], K, scratch)
    att_warm = timed_b2b(c["attend"], K)
    app_warm = timed_b2b(c["append"], K)

    sb = step_bytes_of(w, inp)
    # the bytes the method moves: with the prefix pass each shared block is
    # read once, so the shared prefix counts once (the logical figure, every
    # row's prefix counted, is reported beside it)
    att_bytes = sb.attention_unique if c["cascade"] else sb.attention
    step_b = att_bytes + sb.step - sb.attention
    med = _pct(step_ms, 50)
    r = {
        "w": w, "inp_ctx": inp.ctx, "c": c, "sb": sb, "att_bytes": att_bytes,
        "step_bytes": step_b, "wall_s": wall, "step_ms": step_ms,
        "us": {"step_median": round(med * 1e3, 2), "step_p10": round(_pct(step_ms, 10) * 1e3, 2),
               "step_p90": round(_pct(step_ms, 90) * 1e3, 2),
               "step_warm": round(_pct(warm_step, 50) * 1e3, 2),
               "attention_median": round(_pct(att_cold, 50) * 1e3, 2),
               "attention_p10": round(_pct(att_cold, 10) * 1e3, 2),
               "attention_p90": round(_pct(att_cold, 90) * 1e3, 2),
               "attention_warm": round(_pct(att_warm, 50) * 1e3, 2),
               "append_warm": round(_pct(app_warm, 50) * 1e3, 2)},
        "GBps": round(step_b / (med * 1e-3) / 1e9, 1),
        "attention_GBps": round(att_bytes / (med * 1e-3) / 1e9, 1),
        "warm_GBps": round(att_bytes / (_pct(att_warm, 50) * 1e-3) / 1e9, 1),
        "logical_GBps": round(sb.attention / (med * 1e-3) / 1e9, 1),
        "graph": graph is not None,
    }
    _say(f"[bench] {w.name}: step median {med * 1e3:.1f} us -> {r['GBps']:.0f} GB/s "
         f"(warm {r['us']['step_warm']:.1f} us, attention warm {r['us']['attention_warm']:.1f} us)")

    r["parity"], r["cpu"] = (None, None)
    if with_oracle:
        # the output of the last timed call is the step's result
        r["parity"], r["cpu"] = parity_and_cpu(w, inp, table, slots, shared, host, c["out"],
                                               att_bytes)

    if args.sweep and not (w.kv_dtype == synth.INT4 or w.attn_window or inp.shared_ids_count):
        pts = context_sweep(w, dev, K) + [(1.0, int(sb.attention),
                                           _pct(att_warm, 50) * 1e3)]
        pts.sort()
        x = np.array([p[1] for p in pts], dtype=np.float64) / 1e9
        y = np.array([p[2] for p in pts], dtype=np.float64)
        slope, icpt = np.polyfit(x, y, 1)   # us per GB, us
        r["steady_state"] = {
            "GBps": round(1e6 / slope, 1), "frac": round(1e6 / slope / HBM_PEAK_GBPS, 4),
            "fixed_us": round(float(icpt), 2),
            "points": [{"context_scale": f, "bytes": b, "us": round(u, 2)} for f, b, u in pts],
            "fit": "least squares us = fixed_us + bytes / GBps over warm back-to-back calls"}
        _say(f"[bench] sweep fit: steady {1e6 / slope:.0f} GB/s, fixed {icpt:.2f} us per call")

    r["table"] = table
    pool.close()
    del inp, host
    return r


def main(argv=None) -> int:
    args = parse_args(argv)
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the decode path "
                          "shards over sequences / KV heads with no exchange, and one GPU's "
                          "throughput is the figure reported (--gpus 1)"}), flush=True)
        return 2

    import torch
    import synth

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        return 2
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.workload not in synth.WORKLOADS:
        print(json.dumps({"error": f"unknown workload {args.workload}",
                          "known": sorted(synth.WORKLOADS)}), flush=True)
        return 2
    w = synth.WORKLOADS[args.workload]
    K = args.steps
    scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB flush buffer

    r = measure(w, args, dev, K, scratch, not args.no_oracle)
    # the long-context row is the benchmark spec's second configuration: the
    # default run measures it too, the same way, beside the headline
    extra = None
    if args.workload == DEFAULT_WORKLOAD and not args.no_long:
        torch.cuda.empty_cache()
        extra = measure(synth.WORKLOADS[LONG_WORKLOAD], args, dev, K, scratch,
                        not args.no_oracle)
    probe = None if args.no_probe else read_probe(dev, r["table"], r["inp_ctx"], w, scratch)
    probe_long = (None if args.no_probe or extra is None else
                  read_probe(dev, extra["table"], extra["inp_ctx"], extra["w"], scratch,
                             sequential=False))
    del scratch
    torch.cuda.empty_cache()

    c = r["c"]
    med_ms = r["us"]["step_median"] * 1e-3
    achieved = r["att_bytes"] / (med_ms * 1e-3) / 1e9
    value = r["step_bytes"] / (med_ms * 1e-3) / 1e9

    def probe_pct(pr, rate):
        """The step's rate against the tile probe's, back to back and flushed."""
        if pr is None or "kv_tiles_GBps" not in pr:
            return {}
        return {"pct_of_kv_tiles": round(100.0 * rate / pr["kv_tiles_GBps"], 2),
                "pct_of_kv_tiles_flushed": round(100.0 * rate / pr["kv_tiles_flushed_GBps"], 2)}

    def summary(x, pr):
        wx = x["w"]
        return {"workload": wx.name, "us": x["us"], "GBps": x["GBps"],
                "attention_GBps": x["attention_GBps"],
                "frac": round(x["attention_GBps"] / HBM_PEAK_GBPS, 4),
                "warm_attention_frac": round(x["warm_GBps"] / HBM_PEAK_GBPS, 4),
                "bytes_attention": x["att_bytes"], "parity": x["parity"],
                "traffic": measured_traffic(wx.name),
                **({} if pr is None else
                   {"read_probe": {**pr, **probe_pct(pr, x["attention_GBps"])}})}

    cfg = {"workload": w.name, "B": w.B, "n_q": w.n_q, "n_kv": w.n_kv, "d_h": w.d_h,
           "block_size": w.block_size, "kv_dtype": synth.DTYPE_NAMES[w.kv_dtype],
           "context_min": int(r["inp_ctx"].min()), "context_max": int(r["inp_ctx"].max()),
           "total_context": int(r["inp_ctx"].sum()), "num_partitions": c["P"],
           "blocks_per_partition": c["bpp"], "reuse_prefix_blocks": c["reuse"],
           "window": w.attn_window, "sink_tokens": w.attn_sinks,
           "shared_prefix_blocks": c["n_sh"], "prefix_pass": c["cascade"],
           "parallelism": "none (1 GPU)"}
    res = {
        "metric": "decode-attn KV GB/s (% MI355X HBM peak) + us/step, 70B-shape batch 8x32k",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(med_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.kv_dtype == synth.BF16 else synth.DTYPE_NAMES[w.kv_dtype],
        "data": "synthetic (seeded N(0,1) q/K/V in HBM, random block placement)",
        "config": cfg,
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "us_per_step": r["us"],
        "timing": (("fused decode step" if c["fused"] else "append + attention calls") +
                   ("; graph replay" if r["graph"] else "; eager launches of bound calls") +
                   f"; {K} steps, each after a 1 GiB cache-evicting write, HIP events around "
                   "the step: median / p10 / p90 (value, ms_per_step, roofline); warm = the "
                   "same calls back to back"),
        "timed_region_wall_s": round(r["wall_s"], 4),
        "bytes_per_step": {"counted": r["att_bytes"], "attention": r["sb"].attention,
                           "attention_unique": r["sb"].attention_unique,
                           "step": r["step_bytes"], "kv_read": r["sb"].kv_read},
        "logical_GBps": r["logical_GBps"],
        "roofline": {"bound": "hbm",
                     "kernel": ("paged_decode_attn_prefix (prefix pass + attention + merge)"
                                if c["cascade"] else "k_attn_mfma (fused decode step)"),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "warm_frac": round(r["warm_GBps"] / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(w.name)},
        **({} if probe is None else {
            "read_probe": {**probe,
                           "pct_of_sequential": round(100.0 * achieved / probe["sequential_GBps"], 2),
                           **probe_pct(probe, achieved)}}),
        **({} if "steady_state" not in r else {"steady_state": r["steady_state"]}),
        **({} if extra is None else {"long_context": summary(extra, probe_long)}),
        "parity": r["parity"],
        "cpu_baseline": r["cpu"],
    }
    print(json.dumps(res), flush=True)
    ok = all(x is None or x["parity"] is None or x["parity"]["pass"] for x in (r, extra))
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
