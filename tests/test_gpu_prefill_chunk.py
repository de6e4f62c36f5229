"""gqa_prefill_chunk (a block of Sq new tokens after a cached prefix of
S - Sq tokens) on the GPU: against the oracle's rows S - Sq .. S - 1 of the
whole sequence's attention, and against gqa_prefill over the whole sequence
(bit for bit where the block starts on a workgroup's token boundary, so that
both runs tile every row's keys the same way)."""

import numpy as np
import pytest
import torch

import gpu_helpers as H
from oracle import reference as orc
from workloads import draw_cu_docs, draw_positions, draw_prefill_inputs

pytestmark = pytest.mark.gpu

BASE = 500000.0


def _dev(x):
    return x.to(torch.device("cuda"))


def _cu(cu, B):
    return None if cu is None else _dev(torch.as_tensor(np.asarray(cu), dtype=torch.int32).reshape(B, -1))


def _chunk(q_blk, kr, v, cu, positions=None, rope_base=BASE):
    """gqa_prefill_chunk on device tensors; O and LSE on the CPU."""
    import gqa_attention_rope_02_amd as la
    B, Sq, Hq, _ = q_blk.shape
    o = torch.full_like(q_blk, float("nan"))
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=q_blk.device)
    pos = None if positions is None else _dev(torch.as_tensor(np.asarray(positions), dtype=torch.int32))
    la.gqa_prefill_chunk(q_blk, kr, v, o, lse, _cu(cu, B), 0.0, positions=pos, rope_base=rope_base)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _rot_keys(k, positions=None):
    import gqa_attention_rope_02_amd as la
    kd = _dev(k)
    kr = torch.full_like(kd, float("nan"))
    pos = None if positions is None else _dev(torch.as_tensor(np.asarray(positions), dtype=torch.int32))
    la.rope_qk(None, None, kd, kr, positions=pos, rope_base=BASE)
    return kr


@pytest.mark.parametrize("B,S,Sq,Hq,Hkv,D,dtype,seed,nd", [
    (1, 700, 190, 32, 8, 128, "bf16", 81, 3),    # 8B heads; documents across the block start
    (1, 517, 517, 32, 8, 128, "bf16", 82, 2),    # the whole sequence
    (1, 400, 1, 16, 1, 128, "bf16", 83, 2),      # one new token
    (1, 333, 77, 16, 1, 128, "bf16", 84, 1),     # g=16, ragged block
    (2, 300, 64, 8, 8, 64, "bf16", 85, 3),       # g=1, D=64, two sequences
    (1, 260, 100, 32, 2, 128, "fp32", 86, 2),    # fp32 inputs
])
def test_prefill_chunk_matches_oracle(B, S, Sq, Hq, Hkv, D, dtype, seed, nd):
    H.say("prefill_chunk", dict(B=B, S=S, Sq=Sq, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, seed=seed))
    q, k, v = draw_prefill_inputs(B, S, Hq, Hkv, D, dtype, seed)
    cus = [draw_cu_docs(S, seed + 100 * b, nd, 6) for b in range(B)]
    width = max(c.size for c in cus)
    cu = np.stack([np.concatenate([c, np.full(width - c.size, S, dtype=np.int32)]) for c in cus])
    kr = _rot_keys(k)
    O, L = _chunk(_dev(q[:, S - Sq:].contiguous()), kr, _dev(v), cu)
    rows = np.arange(S - Sq, S)
    for b in range(B):
        Ow, Lw = orc.rope_attention(q[b:b + 1], k[b:b + 1], v[b:b + 1], cu[b], BASE, rows=rows)
        H.assert_close(O[b:b + 1], Ow)
        H.assert_lse_close(L[b:b + 1], Lw, "LSE")


def test_prefill_chunk_with_positions_matches_oracle():
    """Explicit positions (large, as deep in a 128K context) for the keys and
    the block's queries."""
    B, S, Sq, Hq, Hkv, D, seed = 1, 300, 120, 16, 2, 128, 87
    H.say("prefill_chunk positions")
    q, k, v = draw_prefill_inputs(B, S, Hq, Hkv, D, "bf16", seed)
    cu = draw_cu_docs(S, seed, 3, 1)
    pos = draw_positions(B, S, 131071 - S, seed)
    kr = _rot_keys(k, pos)
    O, L = _chunk(_dev(q[:, S - Sq:].contiguous()), kr, _dev(v), cu, positions=pos[:, S - Sq:])
    Ow, Lw = orc.rope_attention(q, k, v, cu, BASE, pos, rows=np.arange(S - Sq, S))
    H.assert_close(O, Ow)
    H.assert_lse_close(L, Lw, "LSE")


@pytest.mark.parametrize("Hq,Hkv,S,Sq", [(32, 8, 640, 192), (16, 1, 500, 52), (8, 8, 800, 544)])
def test_prefill_chunk_equals_whole_prefill_rows(Hq, Hkv, S, Sq):
    """Pre-rotated queries (rope_base 0): with the block starting on a
    multiple of the workgroup's 256 / g tokens, the chunk's outputs and LSE are
    the whole-sequence prefill's rows S - Sq .. S - 1, bit for bit."""
    import gqa_attention_rope_02_amd as la
    assert (S - Sq) % (256 // (Hq // Hkv)) == 0
    H.say("prefill_chunk vs gqa_prefill", dict(Hq=Hq, Hkv=Hkv, S=S, Sq=Sq))
    q, k, v = draw_prefill_inputs(1, S, Hq, Hkv, 128, "bf16", 88)
    cu = draw_cu_docs(S, 88, 4, 1)
    qd, kd, vd = _dev(q), _dev(k), _dev(v)
    qr, kr = torch.empty_like(qd), torch.empty_like(kd)
    la.rope_qk(qd, qr, kd, kr)
    o = torch.empty_like(qd)
    lse = torch.empty((1, Hq, S), dtype=torch.float32, device=qd.device)
    la.gqa_prefill(qr, kr, vd, o, lse, _cu(cu, 1))
    Oc, Lc = _chunk(qr[:, S - Sq:].contiguous(), kr, vd, cu, rope_base=0.0)
    assert torch.equal(Oc, o[:, S - Sq:].cpu())
    assert torch.equal(Lc, lse[:, :, S - Sq:].cpu())


def test_prefill_chunk_fused_rope_equals_gqa_prefill_rope_rows():
    """rope_base > 0: the block's queries rotated in the kernel at their
    positions S - Sq + i give gqa_prefill_rope's rows bit for bit (aligned
    block)."""
    import gqa_attention_rope_02_amd as la
    Hq, Hkv, S, Sq = 32, 8, 704, 320
    H.say("prefill_chunk fused rope vs gqa_prefill_rope")
    q, k, v = draw_prefill_inputs(1, S, Hq, Hkv, 128, "bf16", 89)
    cu = draw_cu_docs(S, 89, 5, 1)
    qd, vd = _dev(q), _dev(v)
    kr = _rot_keys(k)
    o = torch.empty_like(qd)
    la.gqa_prefill_rope(qd, kr, vd, o, None, _cu(cu, 1))
    Oc, _ = _chunk(qd[:, S - Sq:].contiguous(), kr, vd, cu)
    assert torch.equal(Oc, o[:, S - Sq:].cpu())


def test_prefill_chunk_document_probe_is_exact():
    """q = 0 and a V channel that holds each key's document index (small
    integers, exact in bf16): every block row averages its visible keys, all
    of one document, so that channel must come out as the row's document
    index exactly, and exp(LSE) as its count of visible keys."""
    B, S, Sq, Hq, Hkv, D = 1, 450, 200, 32, 8, 128
    H.say("prefill_chunk document probe")
    cu = np.array([0, 37, 250, 251, 333, S], dtype=np.int32)
    doc = orc.document_of(cu, S)
    q = torch.zeros(B, Sq, Hq, D, dtype=torch.bfloat16)
    k = torch.randn(B, S, Hkv, D, generator=torch.Generator().manual_seed(90)).to(torch.bfloat16)
    v = torch.zeros(B, S, Hkv, D, dtype=torch.bfloat16)
    v[0, :, :, 5] = torch.as_tensor(doc, dtype=torch.bfloat16)[:, None]
    O, L = _chunk(_dev(q), _dev(k), _dev(v), cu, rope_base=0.0)
    rows = np.arange(S - Sq, S)
    want = np.broadcast_to(doc[rows][:, None], (Sq, Hq)).astype(np.float32)
    assert np.array_equal(O[0, :, :, 5].float().numpy(), want)
    count = rows - cu[doc[rows]] + 1
    got = np.rint(np.exp(L[0].double().numpy()))
    assert np.array_equal(got, np.broadcast_to(count, (Hq, Sq)))
