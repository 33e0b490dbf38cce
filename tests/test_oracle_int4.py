"""Pins of the 4-bit cache oracle (oracle/int4.py) to things other than itself.

* the packing and offset, on a hand-worked group of 8 channels;
* the quantizer's rounding (half to even) and clamping at its edges;
* the scale axes: per channel for keys, per token for values (a value scale
  applied per channel, or a key scale per token, fails the error bounds);
* the residual-window policy: 15 appends leave the block untouched, the 16th
  encodes it from the residual buffer;
* attention through the stored cache: with no full block it is plain bf16
  attention over the residual rows, and in general it agrees with the
  independent brute-force gather of the decoded values.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle import int4
import synth
from synth import BF16


def test_pack_worked_group():
    # channels 0..7 = -7..0 -> nibbles 1..8; byte i = ch i (low) | ch i+4 (high)
    assert int4.pack_int4(np.array([-7, -6, -5, -4, -3, -2, -1, 0])).tolist() == \
        [0x51, 0x62, 0x73, 0x84]
    assert int4.unpack_int4(np.array([0x51, 0x62, 0x73, 0x84], np.uint8)).tolist() == \
        [-7, -6, -5, -4, -3, -2, -1, 0]


def test_pack_round_trip():
    r = np.random.default_rng(0)
    c = r.integers(-7, 8, size=(3, 5, 16, 128)).astype(np.int8)
    p = int4.pack_int4(c)
    assert p.shape == (3, 5, 16, 64) and p.dtype == np.uint8
    assert (int4.unpack_int4(p) == c).all()
    assert ((p & 0x0F) != 0).all() and ((p >> 4) != 0).all()   # nibble 0 (code -8) never used


def test_quantizer_rounding_and_clamp():
    y = np.array([0.5, 1.5, 2.5, -0.5, -2.5, 6.5, 7.49, 7.5, 9.0, -100.0, np.nan], np.float32)
    assert int4.quantize_int4(y).tolist() == [0, 2, 2, 0, -2, 6, 7, 7, 7, -7, 0]


def test_token_scale():
    v = np.zeros((2, 128), np.float32)
    v[0, 5] = -3.5
    v[0, 9] = 1.0
    s = int4.token_scale(v)
    assert s[0] == np.float32(0.5) and s[1] == np.float32(1.0)


def test_encode_block_error_bounds_and_axes():
    """Keys: one scale per channel, so a channel's error is within half its own
    step even when channels differ 16x in size; values: one scale per token,
    every token reaches code +-7 at its largest element."""
    r = np.random.default_rng(1)
    n_kv, d_h = 2, 128
    mag = np.where(np.arange(d_h) % 16 == 3, 16.0, 1.0).astype(np.float32)  # outlier channels
    k = (r.standard_normal((n_kv, 16, d_h)) * mag).astype(np.float32)
    v = r.standard_normal((n_kv, 16, d_h)).astype(np.float32) * \
        r.uniform(0.1, 10.0, size=(n_kv, 16, 1)).astype(np.float32)
    ks = (np.abs(k).max(axis=1) / 7.0).astype(np.float32)      # per channel, no saturation
    kq, vq, vs = int4.encode_block(k, v, ks)
    kd = int4.unpack_int4(kq) * ks[:, None, :].astype(np.float64)
    assert (np.abs(kd - k) <= ks[:, None, :] * (0.5 + 1e-6)).all()
    vc = int4.unpack_int4(vq)
    vd = vc * vs[..., None].astype(np.float64)
    assert (np.abs(vd - v) <= vs[..., None] * (0.5 + 1e-6)).all()
    assert (np.abs(vc).max(axis=-1) == 7).all()
    assert np.allclose(vs, np.abs(v).max(axis=-1) / 7.0, rtol=1e-6)


def _state(NB, B, n_kv, d_h):
    return {"k": np.zeros((NB, n_kv, 16, d_h // 2), np.uint8),
            "v": np.zeros((NB, n_kv, 16, d_h // 2), np.uint8),
            "v_scale": np.ones((NB, n_kv, 16), np.float32),
            "k_res": np.zeros((B, n_kv, 16, d_h), np.uint16),
            "v_res": np.zeros((B, n_kv, 16, d_h), np.uint16)}


def test_fill_policy():
    r = np.random.default_rng(2)
    n_kv, d_h = 2, 64
    st = _state(4, 1, n_kv, d_h)
    table = np.array([[2, 0, -1, -1]], np.int32)
    ks = np.full((n_kv, d_h), 0.5, np.float32)
    rows = [synth.gaussian((1, n_kv, d_h), BF16, r) for _ in range(2 * 16)]
    vrows = [synth.gaussian((1, n_kv, d_h), BF16, r) for _ in range(2 * 16)]
    for t in range(15):
        st = int4.kv_append_int4(st, rows[t], vrows[t], table, [t + 1], ks)
        assert (st["k"] == 0).all() and (st["v_scale"] == 1).all()   # nothing encoded yet
        assert (st["k_res"][0, :, t, :] == rows[t][0]).all()
    st = int4.kv_append_int4(st, rows[15], vrows[15], table, [16], ks)
    res_k = np.stack([rows[t][0] for t in range(16)], axis=1)
    res_v = np.stack([vrows[t][0] for t in range(16)], axis=1)
    kq, vq, vs = int4.encode_block(synth.bf16_bits_to_f32(res_k), synth.bf16_bits_to_f32(res_v),
                                   ks)
    assert (st["k"][2] == kq).all() and (st["v"][2] == vq).all() and (st["v_scale"][2] == vs).all()
    assert (st["k"][[0, 1, 3]] == 0).all()
    # the next token opens block 0 (logical 1) in the residual buffer, slot 0
    st = int4.kv_append_int4(st, rows[16], vrows[16], table, [17], ks)
    assert (st["k_res"][0, :, 0, :] == rows[16][0]).all() and (st["k"][0] == 0).all()


def _random_state(r, NB, B, n_kv, d_h):
    st = _state(NB, B, n_kv, d_h)
    st["k"] = r.integers(0x11, 0xFF, size=st["k"].shape).astype(np.uint8) | 0x11
    st["v"] = r.integers(0x11, 0xFF, size=st["v"].shape).astype(np.uint8) | 0x11
    st["v_scale"] = r.uniform(0.05, 2.0, size=st["v_scale"].shape).astype(np.float32)
    st["k_res"] = synth.gaussian(st["k_res"].shape, BF16, r)
    st["v_res"] = synth.gaussian(st["v_res"].shape, BF16, r)
    return st


def test_attention_residual_only_is_bf16_attention():
    """Rows shorter than one block are attended from their residual rows
    alone: the same as plain attention on a bf16 cache holding them."""
    r = np.random.default_rng(3)
    B, n_q, n_kv, d_h = 3, 8, 2, 64
    st = _random_state(r, 6, B, n_kv, d_h)
    ks = r.uniform(0.1, 1.0, size=(n_kv, d_h)).astype(np.float32)
    ctx = np.array([1, 7, 15], np.int32)
    table = np.array([[4], [0], [5]], np.int32)
    q = synth.gaussian((B, n_q, d_h), BF16, r)
    got, _, _, bad = oracle.paged_attn_int4(q, st, ks, table, ctx, 0.125, n_q=n_q, n_kv=n_kv,
                                            q_dtype=BF16)
    assert bad == 0
    ref, _, _, _ = oracle.paged_attn(q, st["k_res"], st["v_res"], np.arange(B)[:, None], ctx,
                                     0.125, n_q=n_q, n_kv=n_kv, q_dtype=BF16, kv_dtype=BF16)
    assert np.abs(got - ref).max() < 1e-12


def test_attention_matches_brute_force_on_decoded_values():
    r = np.random.default_rng(4)
    B, n_q, n_kv, d_h = 4, 8, 2, 128
    ctx = np.array([16, 40, 3, 33], np.int32)
    NB = 12
    table = np.array([[7, -1, -1], [1, 9, 3], [11, -1, -1], [0, 2, 5]], np.int32)
    st = _random_state(r, NB, B, n_kv, d_h)
    ks = r.uniform(0.1, 1.0, size=(n_kv, d_h)).astype(np.float32)
    q = synth.gaussian((B, n_q, d_h), BF16, r)
    got, _, _, bad = oracle.paged_attn_int4(q, st, ks, table, ctx, 0.1, n_q=n_q, n_kv=n_kv,
                                            q_dtype=BF16)
    assert bad == 0
    # independent gather: position t of row b is block t // 16 (full blocks
    # decoded by hand here, the open block from the residual buffer)
    qf = synth.bf16_bits_to_f32(q).astype(np.float64)
    kcode = int4.unpack_int4(st["k"]).astype(np.float64)
    vcode = int4.unpack_int4(st["v"]).astype(np.float64)
    kres = synth.bf16_bits_to_f32(st["k_res"]).astype(np.float64)
    vres = synth.bf16_bits_to_f32(st["v_res"]).astype(np.float64)
    g = n_q // n_kv
    for b in range(B):
        n = int(ctx[b])
        for h in range(n_q):
            j = h // g
            K, V = [], []
            for t in range(n):
                if t // 16 < n // 16:
                    pb = table[b, t // 16]
                    K.append(ks[j] * kcode[pb, j, t % 16])
                    V.append(st["v_scale"][pb, j, t % 16] * vcode[pb, j, t % 16])
                else:
                    K.append(kres[b, j, t % 16])
                    V.append(vres[b, j, t % 16])
            sc = np.array(K) @ qf[b, h] * 0.1
            p = np.exp(sc - sc.max())
            ref = (p @ np.array(V)) / p.sum()
            assert np.abs(got[b * n_q + h] - ref).max() < 1e-12
