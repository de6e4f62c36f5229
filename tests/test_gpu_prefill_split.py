"""gqa_prefill_split (query tiles' key ranges cut into pieces handled by
separate workgroups, partials merged by log-sum-exp weight) on the GPU:
against the oracle, against the unsplit gqa_prefill_chunk, and exact probes
where pieces hold no visible key for some rows."""

import numpy as np
import pytest
import torch

import gpu_helpers as H
from oracle import reference as orc
from workloads import draw_cu_docs, draw_prefill_inputs

pytestmark = pytest.mark.gpu

BASE = 500000.0


def _dev(x):
    return x.to(torch.device("cuda"))


def _cu(cu, B):
    return None if cu is None else _dev(torch.as_tensor(np.asarray(cu), dtype=torch.int32).reshape(B, -1))


def _split(q_blk, kr, v, cu, split_tiles, rope_base=BASE, fill=float("nan")):
    """gqa_prefill_split on device tensors (workspace filled with `fill` so
    that a slot read without being written shows up); O and LSE on the CPU."""
    import gqa_attention_rope_02_amd as la
    B, Sq, Hq, D = q_blk.shape
    S = kr.shape[1]
    o = torch.full_like(q_blk, float("nan"))
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=q_blk.device)
    op, lp = la.prefill_split_workspace(B, Sq, S, Hq, D, split_tiles, q_blk.device)
    op.fill_(fill)
    lp.fill_(fill)
    la.gqa_prefill_split(q_blk, kr, v, o, split_tiles, op, lp, lse, _cu(cu, B), rope_base=rope_base)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _chunk(q_blk, kr, v, cu, rope_base=BASE):
    import gqa_attention_rope_02_amd as la
    B, Sq, Hq, _ = q_blk.shape
    o = torch.full_like(q_blk, float("nan"))
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=q_blk.device)
    la.gqa_prefill_chunk(q_blk, kr, v, o, lse, _cu(cu, B), rope_base=rope_base)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _rot_keys(k):
    import gqa_attention_rope_02_amd as la
    kd = _dev(k)
    kr = torch.full_like(kd, float("nan"))
    la.rope_qk(None, None, kd, kr, rope_base=BASE)
    return kr


@pytest.mark.parametrize("B,S,Sq,Hq,Hkv,D,dtype,seed,nd,split", [
    (1, 900, 256, 32, 8, 128, "bf16", 91, 2, 2),    # long document before the block, 2-tile pieces
    (1, 700, 700, 32, 8, 128, "bf16", 92, 3, 3),    # whole sequence
    (1, 600, 33, 16, 1, 128, "bf16", 93, 1, 1),     # g=16, one-tile pieces, ragged block
    (2, 500, 120, 8, 8, 64, "bf16", 94, 3, 2),      # g=1, D=64, two sequences
    (1, 400, 150, 32, 2, 128, "fp32", 95, 2, 2),    # fp32 inputs
])
def test_prefill_split_matches_oracle(B, S, Sq, Hq, Hkv, D, dtype, seed, nd, split):
    H.say("prefill_split", dict(B=B, S=S, Sq=Sq, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, seed=seed, split=split))
    q, k, v = draw_prefill_inputs(B, S, Hq, Hkv, D, dtype, seed)
    cus = [draw_cu_docs(S, seed + 100 * b, nd, 6) for b in range(B)]
    width = max(c.size for c in cus)
    cu = np.stack([np.concatenate([c, np.full(width - c.size, S, dtype=np.int32)]) for c in cus])
    kr = _rot_keys(k)
    O, L = _split(_dev(q[:, S - Sq:].contiguous()), kr, _dev(v), cu, split)
    rows = np.arange(S - Sq, S)
    for b in range(B):
        Ow, Lw = orc.rope_attention(q[b:b + 1], k[b:b + 1], v[b:b + 1], cu[b], BASE, rows=rows)
        H.assert_close(O[b:b + 1], Ow)
        H.assert_lse_close(L[b:b + 1], Lw, "LSE")


@pytest.mark.parametrize("split", [1, 4, 16])
def test_prefill_split_agrees_with_unsplit(split):
    """The merge only regroups the softmax: outputs stay within a few bf16
    roundings of the unsplit chunk's; with pieces longer than every key range
    nothing is split and the result is the same bit for bit."""
    S, Sq, Hq, Hkv = 1100, 300, 32, 8
    H.say("prefill_split vs chunk", dict(split=split))
    q, k, v = draw_prefill_inputs(1, S, Hq, Hkv, 128, "bf16", 96)
    cu = draw_cu_docs(S, 96, 3, 1)
    kr = _rot_keys(k)
    qb, vd = _dev(q[:, S - Sq:].contiguous()), _dev(v)
    O1, L1 = _chunk(qb, kr, vd, cu)
    O2, L2 = _split(qb, kr, vd, cu, split)
    d = (O1.float() - O2.float()).abs()
    assert d.max().item() <= 8e-3 and d.mean().item() <= 2e-4, (d.max().item(), d.mean().item())
    assert (L1 - L2).abs().max().item() <= 2e-3
    O3, L3 = _split(qb, kr, vd, cu, 64)   # 64 tiles of 64 keys > S: never split
    assert torch.equal(O3, O1) and torch.equal(L3, L1)


def test_prefill_split_document_probe_is_exact():
    """q = 0 and a V channel holding each key's document index, with one-tile
    pieces: many pieces see none of a row's keys (document or causal edge) and
    must carry no weight; the merged channel is the row's document index and
    exp(LSE) its count of visible keys, exactly."""
    B, S, Sq, Hq, Hkv, D = 1, 520, 260, 32, 8, 128
    H.say("prefill_split document probe")
    cu = np.array([0, 100, 101, 380, S], dtype=np.int32)
    doc = orc.document_of(cu, S)
    q = torch.zeros(B, Sq, Hq, D, dtype=torch.bfloat16)
    k = torch.randn(B, S, Hkv, D, generator=torch.Generator().manual_seed(97)).to(torch.bfloat16)
    v = torch.zeros(B, S, Hkv, D, dtype=torch.bfloat16)
    v[0, :, :, 9] = torch.as_tensor(doc, dtype=torch.bfloat16)[:, None]
    O, L = _split(_dev(q), _dev(k), _dev(v), cu, 1, rope_base=0.0)
    rows = np.arange(S - Sq, S)
    want = np.broadcast_to(doc[rows][:, None], (Sq, Hq)).astype(np.float32)
    assert np.array_equal(O[0, :, :, 9].float().numpy(), want)
    count = rows - cu[doc[rows]] + 1
    assert np.array_equal(np.rint(np.exp(L[0].double().numpy())), np.broadcast_to(count, (Hq, Sq)))
    assert torch.isfinite(O).all()
