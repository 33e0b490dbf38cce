"""Scores that jump inside a piece: the lazy rescale path on the GPU against
the oracle.

The kernels keep each head's reference maximum until a block's scores
exceed it by more than 8 (log2 units), then rescale the running sums. With
N(0,1) inputs that only happens at a piece's first block, so these cases
scale the keys of chosen blocks up by powers of two (exact in every cache
format: bf16 values, 8-bit block scales) or, for the 4-bit cache, draw the
codes of later blocks with growing spread, so that the reference has to move
several times in the middle of a wave's range, in either block of a 4-bit
pair, and just before a piece ends.

Patterns per row (per logical block of the row, exponent e of the factor
2^e on its keys):
- grow:  e rises from 0 to 4 along the row;
- spike: e = 4 on one block two thirds along the row, 0 elsewhere;
- last:  e = 4 on the row's last block only;
- fall:  e = 4 on the first block, then 0 (the reference never moves).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from oracle import int4 as oint4
import synth
from synth import BF16, FP8, INT8, F32
from tests.helpers import make_case
from tests.gpu_helpers import TOL_16BIT, TOL_8BIT, assert_parity, max_err, run_case

pytestmark = pytest.mark.gpu

PATTERNS = ("grow", "spike", "last", "fall")
CTX = [700, 2063, 33, 4096, 17, 1500]


def _exponents(pattern: str, nblk: int) -> np.ndarray:
    e = np.zeros(nblk, np.int64)
    if nblk == 0:
        return e
    if pattern == "grow":
        e = (np.arange(nblk) * 5) // max(nblk, 1)
    elif pattern == "spike":
        e[(2 * nblk) // 3] = 4
    elif pattern == "last":
        e[nblk - 1] = 4
    elif pattern == "fall":
        e[0] = 4
    return e


def _scale_keys(case, pattern):
    """Multiply the keys of each row's logical block by 2^e (bf16: the values
    themselves, exact; 8-bit: the block's K scale)."""
    k = case.k.copy()
    ks = None if case.k_scale is None else case.k_scale.copy()
    for b, n in enumerate(case.ctx):
        nblk = (int(n) + case.bs - 1) // case.bs
        for lb, ex in enumerate(_exponents(pattern, nblk)):
            pb = int(case.table[b, lb])
            if ex == 0 or pb < 0:
                continue
            if case.kv_dtype == BF16:
                vals = synth.bf16_bits_to_f32(k[pb]) * np.float32(2.0 ** ex)
                k[pb] = synth.bf16_bits_from_f32(vals)
            else:
                ks[pb] = ks[pb] * np.float32(2.0 ** ex)
    case.k = k
    case.k_scale = ks
    return case


@pytest.mark.parametrize("kv", [BF16, FP8, INT8])
@pytest.mark.parametrize("pattern", PATTERNS)
@pytest.mark.parametrize("nw", [0, 1, 9])
def test_scores_jump_inside_a_piece(kv, pattern, nw):
    print(f"rescale kv={kv} pattern={pattern} nw={nw}", flush=True)
    sys.stdout.flush()
    case = make_case(7100 + 10 * kv + nw, CTX, n_q=8, n_kv=2, d_h=128, kv_dtype=kv)
    # every row's blocks are owned (no unmapped entries), so all scales are finite
    assert not case.shared_ids
    case = _scale_keys(case, pattern)
    got, _ = run_case(case, num_partitions=nw)
    ref = case.oracle_out()
    assert np.isfinite(got).all()
    err = max_err(got, ref)
    print(f"  max-abs error {err:.2e}", flush=True)
    assert_parity(err, TOL_16BIT if kv == BF16 else TOL_8BIT)


def _int4_case(seed, ctx, pattern, *, n_q=8, n_kv=2, d_h=128):
    """4-bit cache whose codes grow in spread along each row (the per-channel
    key scales are fixed, so the keys' size is set by the codes): block
    spread 7 * 2^(e - 4) for the pattern's exponent e, codes rounded from
    N(0,1) draws and clamped to [-7, 7]."""
    r = np.random.default_rng(seed)
    ctx = np.asarray(ctx, np.int32)
    B = ctx.size
    nblk = (ctx.astype(np.int64) + 15) // 16
    nb = int(nblk.sum()) + 2
    mb = max(int(nblk.max()), 1)
    pool = oracle.OraclePool(nb, list(r.permutation(nb)))
    table, _ = pool.build_block_table(ctx, 16, mb)
    codes = np.clip(np.rint(0.4 * r.standard_normal((nb, n_kv, 16, d_h))), -7, 7)
    for b, n in enumerate(ctx):
        full = int(n) // 16
        ex = _exponents(pattern, full)
        for lb in range(full):
            z = r.standard_normal((n_kv, 16, d_h))
            codes[table[b, lb]] = np.clip(np.rint(z * 7.0 * 2.0 ** (int(ex[lb]) - 4)), -7, 7)
    vcodes = np.clip(np.rint(2.0 * r.standard_normal((nb, n_kv, 16, d_h))), -7, 7)
    st = {"k": oint4.pack_int4(codes.astype(np.int8)),
          "v": oint4.pack_int4(vcodes.astype(np.int8)),
          "v_scale": r.uniform(0.1, 0.5, size=(nb, n_kv, 16)).astype(np.float32),
          "k_res": synth.gaussian((B, n_kv, 16, d_h), BF16, r),
          "v_res": synth.gaussian((B, n_kv, 16, d_h), BF16, r)}
    ks = r.uniform(0.15, 0.3, size=(n_kv, d_h)).astype(np.float32)
    return st, ks, table, ctx, nb, mb


@pytest.mark.parametrize("pattern", PATTERNS)
@pytest.mark.parametrize("nw", [0, 1, 9])
@pytest.mark.parametrize("qd", [BF16, F32])
def test_int4_scores_jump_inside_a_piece(pattern, nw, qd):
    """The 4-bit scores start from the reference maximum itself, so a move of
    the reference also shifts the step's scores; the pairs see the jump in
    their first or second block. Queries x8 put the top scores near 20 (in
    units of the softmax), where the 2^-16 split of the scaled query weighs
    more (measured up to 1.8e-4 of an output): the bound here is the
    contract bar plus 1e-3."""
    from tests.test_gpu_int4 import _attend, _desc, _dev
    print(f"int4 rescale pattern={pattern} nw={nw} q={qd}", flush=True)
    sys.stdout.flush()
    n_q, n_kv, d_h = 8, 2, 128
    st, ks, table, ctx, nb, mb = _int4_case(7300 + nw + 3 * PATTERNS.index(pattern), CTX,
                                            pattern, n_q=n_q, n_kv=n_kv, d_h=d_h)
    r = np.random.default_rng(11)
    q_np = synth.gaussian((ctx.size, n_q, d_h), qd, r)
    if qd == BF16:   # x8 is exact in bf16
        q_np = synth.bf16_bits_from_f32(synth.bf16_bits_to_f32(q_np) * np.float32(8.0))
    else:
        q_np = (q_np * np.float32(8.0)).astype(np.float32)
    from tests.gpu_helpers import to_dev
    dev = "cuda"
    st_d, ks_d = _dev(st, ks, dev)
    q = to_dev(q_np, qd, dev)
    scale = 1.0 / np.sqrt(d_h)
    got = _attend(st_d, ks_d, q, table, ctx, scale,
                  _desc(ctx.size, n_q, n_kv, d_h, mb, nb, qd, F32, ctx, nw))
    ref, _, _, bad = oracle.paged_attn_int4(q_np, st, ks, table, ctx, scale, n_q=n_q, n_kv=n_kv,
                                            q_dtype=qd)
    assert bad == 0
    ref = ref.reshape(got.shape)
    assert np.isfinite(got).all()
    err = float(np.abs(got - ref).max())
    print(f"  max-abs error {err:.2e}", flush=True)
    assert_parity(err, TOL_8BIT, regression=1e-3)
