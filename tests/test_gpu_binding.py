"""The Python binding's argument checks on device tensors: every tensor's
dtype, shape or element count, and contiguity are checked before the C call,
so a mistaken argument raises instead of handing a kernel a buffer of the
wrong size or layout. Nothing is launched in these cases."""
from __future__ import annotations

import sys

import pytest

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _append_args(torch, dev):
    k = torch.zeros((8, 2, 16, 64), dtype=torch.bfloat16, device=dev)
    kn = torch.zeros((3, 2, 64), dtype=torch.bfloat16, device=dev)
    slots = torch.tensor([0, 17, 40], dtype=torch.int64, device=dev)
    return kn, kn.clone(), slots, k, k.clone()


def test_append_binding_refusals():
    import torch
    import decode_attention_paged_slot_amd as pda
    _say("binding refusals: append")
    dev = "cuda"
    kn, vn, slots, k, v = _append_args(torch, dev)
    # an int32 slot mapping would be read as 8-byte entries from a 4-byte array
    with pytest.raises(TypeError, match="slot_mapping"):
        pda.kv_append(kn, vn, slots.to(torch.int32), k, v)
    with pytest.raises(TypeError, match="v_new"):
        pda.kv_append(kn, vn.float(), slots, k, v)
    with pytest.raises(ValueError, match="slot_mapping"):
        pda.kv_append(kn, vn, slots[:2], k, v)
    with pytest.raises(ValueError, match="v_cache"):
        pda.kv_append(kn, vn, slots, k, v[:4])
    with pytest.raises(ValueError, match="contiguous"):
        pda.kv_append(kn.transpose(0, 1).contiguous().transpose(0, 1), vn, slots, k, v)
    torch.cuda.synchronize()
    # the caches are untouched
    assert int(k.abs().sum().item()) == 0


def test_attention_binding_refusals():
    import torch
    import decode_attention_paged_slot_amd as pda
    _say("binding refusals: attention")
    dev = "cuda"
    B, n_q, n_kv, d_h, mb, nb = 2, 8, 2, 64, 4, 8
    q = torch.zeros((B, n_q, d_h), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((nb, n_kv, 16, d_h), dtype=torch.bfloat16, device=dev)
    bt = torch.zeros((B, mb), dtype=torch.int32, device=dev)
    cl = torch.full((B,), 20, dtype=torch.int32, device=dev)
    out = torch.full((B, n_q, d_h), 5.0, device=dev)
    with pytest.raises(TypeError, match="block_table"):
        pda.paged_decode_attn(q, k, k.clone(), bt.long(), cl, 0.1, out, max_context=20)
    with pytest.raises(TypeError, match="context_lens"):
        pda.paged_decode_attn(q, k, k.clone(), bt, cl.long(), 0.1, out, max_context=20)
    with pytest.raises(ValueError, match="context_lens"):
        pda.paged_decode_attn(q, k, k.clone(), bt, cl[:1], 0.1, out, max_context=20)
    with pytest.raises(ValueError):
        pda.paged_decode_attn(q, k, k.clone(), bt, cl, 0.1, out[:, :4], max_context=20)
    with pytest.raises(ValueError, match="contiguous"):
        pda.paged_decode_attn(q, k, k.clone(), bt.t().contiguous().t(), cl, 0.1, out,
                              max_context=20)
    torch.cuda.synchronize()
    assert bool((out == 5.0).all())   # nothing was written
