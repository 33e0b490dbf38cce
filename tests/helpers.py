"""Small paged decode-attention cases for the tests.

Random numbers come from the `synth` generators; block tables and slots come
from the oracle's pool model (never from the GPU library), so every input the
oracle sees is independent of the code under test.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

import oracle
import synth
from synth import F32, BF16, FP8, INT8


@dataclasses.dataclass
class Case:
    B: int
    n_q: int
    n_kv: int
    d_h: int
    bs: int
    kv_dtype: int
    q_dtype: int
    ctx: np.ndarray            # [B] int32
    num_blocks: int
    max_blocks: int
    table: np.ndarray          # [B, max_blocks] int32, -1 = unmapped
    slots: np.ndarray          # [B] int64 slot of each row's newest token
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    k_scale: Optional[np.ndarray]
    v_scale: Optional[np.ndarray]
    scale: float
    shared_ids: Sequence[int] = ()

    @property
    def g(self) -> int:
        return self.n_q // self.n_kv

    def oracle(self, **kw):
        return oracle.paged_attn(self.q, self.k, self.v, self.table, self.ctx, self.scale,
                                 n_q=self.n_q, n_kv=self.n_kv, q_dtype=self.q_dtype,
                                 kv_dtype=self.kv_dtype, k_scale=self.k_scale,
                                 v_scale=self.v_scale, **kw)

    def oracle_out(self, **kw) -> np.ndarray:
        out, _, _, bad = self.oracle(**kw)
        assert bad == 0
        return out.reshape(self.B, self.n_q, self.d_h) if "rows" not in kw else out


def make_case(seed: int, ctx: Sequence[int], *, n_q=4, n_kv=2, d_h=64, bs=16,
              kv_dtype=BF16, q_dtype=BF16, extra_blocks=3, max_blocks=None,
              shared_prefix_blocks=0, scale=None, poison=True) -> Case:
    r = np.random.default_rng(seed)
    ctx = np.asarray(ctx, dtype=np.int32)
    B = ctx.size
    nblk = synth.blocks_needed(ctx, bs)
    if shared_prefix_blocks:
        sh = np.minimum(shared_prefix_blocks, np.maximum(nblk - 1, 0))
        need = shared_prefix_blocks + int((nblk - sh).sum())
    else:
        need = int(nblk.sum())
    nb = need + extra_blocks
    mb = int(max(1, nblk.max() if B else 1)) if max_blocks is None else max_blocks
    order = synth.free_order(nb, r)
    pool = oracle.OraclePool(nb, order)
    shared = pool.alloc(shared_prefix_blocks) if shared_prefix_blocks else []
    table, slots = pool.build_block_table(ctx, bs, mb, shared)
    q = synth.gaussian((B, n_q, d_h), q_dtype, r)
    shape = (nb, n_kv, bs, d_h)
    ks = vs = None
    if kv_dtype in (F32, BF16):
        k = synth.gaussian(shape, kv_dtype, r)
        v = synth.gaussian(shape, kv_dtype, r)
    else:
        k, ks = synth.quantized_gaussian(shape, kv_dtype, r)
        v, vs = synth.quantized_gaussian(shape, kv_dtype, r)
    w = synth.Workload("case", seed, B=B, n_q=n_q, n_kv=n_kv, d_h=d_h, block_size=bs,
                       kv_dtype=kv_dtype, q_dtype=q_dtype, ctx_lo=0, ctx_hi=0)
    if poison:
        synth.poison_unowned(w, k, v, table, ctx, ks, vs)
    sc = (1.0 / np.sqrt(d_h)) if scale is None else scale
    return Case(B, n_q, n_kv, d_h, bs, kv_dtype, q_dtype, ctx, nb, mb, table, slots, q, k, v,
                ks, vs, float(sc), list(shared))


def permute_physical(case: Case, seed: int) -> Case:
    """Same logical content, physical blocks renumbered by a random permutation
    (cache rows moved, table rewritten)."""
    r = np.random.default_rng(seed)
    perm = r.permutation(case.num_blocks)           # old id -> new id
    inv = np.argsort(perm)                          # new id -> old id
    table = np.where(case.table >= 0, perm[np.maximum(case.table, 0)], -1).astype(np.int32)
    k = case.k[inv].copy()
    v = case.v[inv].copy()
    ks = case.k_scale[inv].copy() if case.k_scale is not None else None
    vs = case.v_scale[inv].copy() if case.v_scale is not None else None
    return dataclasses.replace(case, table=table, k=k, v=v, k_scale=ks, v_scale=vs)


def unshare(case: Case) -> Case:
    """Replace every shared physical block by private copies with the same
    bytes (one copy per extra row that references it)."""
    table = case.table.copy()
    k, v = [case.k], [case.v]
    ks = [case.k_scale] if case.k_scale is not None else None
    vs = [case.v_scale] if case.v_scale is not None else None
    nb = case.num_blocks
    seen = set()
    for b in range(case.B):
        for jb in range(table.shape[1]):
            pb = int(table[b, jb])
            if pb < 0:
                continue
            if pb in seen:
                table[b, jb] = nb
                nb += 1
                k.append(case.k[pb:pb + 1])
                v.append(case.v[pb:pb + 1])
                if ks is not None:
                    ks.append(case.k_scale[pb:pb + 1])
                    vs.append(case.v_scale[pb:pb + 1])
            else:
                seen.add(pb)
    return dataclasses.replace(
        case, table=table, k=np.concatenate(k), v=np.concatenate(v), num_blocks=nb,
        k_scale=np.concatenate(ks) if ks is not None else None,
        v_scale=np.concatenate(vs) if vs is not None else None)
