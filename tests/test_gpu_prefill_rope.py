"""gqa_prefill_rope (queries rotated inside the attention kernel, keys by
rope_qk) against the fp64 oracle, and against the two-call path rope_qk +
gqa_prefill on the same inputs, on the GPU."""

import numpy as np
import pytest
import torch

import gpu_helpers as H
from oracle import reference as orc
from workloads import draw_cu_docs, draw_positions, draw_prefill_inputs

pytestmark = pytest.mark.gpu


def _fused(q, k, v, cu, positions=None, rope_base=500000.0, softmax_scale=0.0, pairing="adjacent"):
    """rope_qk on k only, then gqa_prefill_rope on the raw q; CPU outputs."""
    import gqa_attention_rope_02_amd as la
    dev = torch.device("cuda")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    B, S, Hq, D = q.shape
    kr = torch.full_like(kd, float("nan"))
    pos = None if positions is None else torch.as_tensor(np.asarray(positions), dtype=torch.int32).to(dev)
    la.rope_qk(None, None, kd, kr, positions=pos, rope_base=rope_base, rope_pairing=pairing)
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, Hq, S), float("nan"), dtype=torch.float32, device=dev)
    cud = None if cu is None else torch.as_tensor(np.asarray(cu), dtype=torch.int32).reshape(B, -1).to(dev)
    la.gqa_prefill_rope(qd, kr, vd, o, lse, cud, softmax_scale, positions=pos, rope_base=rope_base,
                        rope_pairing=pairing)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


@pytest.mark.parametrize("B,S,Hq,Hkv,D,dtype,seed,nd,positions", [
    (1, 517, 32, 8, 128, "bf16", 71, None, False),   # the 8B head layout, g=4
    (1, 333, 16, 1, 128, "bf16", 72, None, True),    # g=16, positions up to 128K
    (1, 300, 8, 8, 64, "bf16", 73, 3, False),        # g=1, D=64
    (2, 190, 32, 2, 128, "bf16", 74, None, True),    # two sequences
    (1, 200, 32, 2, 128, "fp32", 75, None, False),   # fp32 inputs
])
def test_prefill_rope_matches_oracle(B, S, Hq, Hkv, D, dtype, seed, nd, positions):
    H.say("prefill_rope", dict(B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, seed=seed))
    q, k, v = draw_prefill_inputs(B, S, Hq, Hkv, D, dtype, seed)
    cus = [draw_cu_docs(S, seed + 100 * b, nd, 6) for b in range(B)]
    width = max(c.size for c in cus)   # rows of equal width: pad with empty documents
    cu = np.stack([np.concatenate([c, np.full(width - c.size, S, dtype=np.int32)]) for c in cus])
    pos = draw_positions(B, S, 131071 - S, seed) if positions else None
    O, L = _fused(q, k, v, cu, pos)
    Ow = np.zeros((B, S, Hq, D))
    Lw = np.zeros((B, Hq, S))
    for b in range(B):
        pb = None if pos is None else pos[b:b + 1]
        Ow[b:b + 1], Lw[b:b + 1] = orc.rope_attention(q[b:b + 1], k[b:b + 1], v[b:b + 1], cu[b],
                                                      500000.0, pb)
    H.assert_close(O, Ow)
    H.assert_lse_close(L, Lw, "LSE")


def test_prefill_rope_agrees_with_the_two_call_path():
    """Same inputs through rope_qk + gqa_prefill and through rope_qk(k) +
    gqa_prefill_rope. The kernel's query operand is q * scale * log2(e)
    rounded to bf16: the fused path rounds it once from the fp32 rotation,
    the two-call path from the bf16 query rope_qk stored, so the operands
    differ by up to one bf16 ulp in many elements, like two independent
    roundings. Each path is within the parity bar of the oracle (other
    tests); here the two agree within that same bar, and the LSE rows within
    the LSE bar."""
    B, S, Hq, Hkv, D = 1, 600, 32, 8, 128
    H.say("prefill_rope vs two-call path")
    q, k, v = draw_prefill_inputs(B, S, Hq, Hkv, D, "bf16", 76)
    cu = draw_cu_docs(S, 76, 4, 1)
    O1, L1, _, _ = H.run_prefill(q, k, v, cu)
    O2, L2 = _fused(q, k, v, cu)
    H.assert_close(O1.double().numpy(), O2.double().numpy(), what="O two-call vs fused")
    H.assert_lse_close(L1.double().numpy(), L2.double().numpy(), "LSE two-call vs fused")


def test_prefill_rope_position_zero_leaves_queries_unrotated():
    """At position 0 every angle is 0: with all positions 0 the fused path
    equals gqa_prefill on the unrotated queries given in fp32, bit for bit.
    (Both round q * scale * log2(e) once to bf16 from the same fp32 value; the
    fp32 call rounds K and V to bf16 on their way into LDS, exactly here since
    they are bf16 values, and writes O in fp32, which rounds to the bf16 O.)"""
    import gqa_attention_rope_02_amd as la
    B, S, Hq, Hkv, D = 1, 130, 16, 2, 128
    H.say("prefill_rope position 0")
    q, k, v = draw_prefill_inputs(B, S, Hq, Hkv, D, "bf16", 77)
    dev = torch.device("cuda")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    pos = torch.zeros(B, S, dtype=torch.int32, device=dev)
    o1 = torch.empty(B, S, Hq, D, dtype=torch.float32, device=dev)
    o2 = torch.empty_like(qd)
    la.gqa_prefill(qd.float(), kd.float(), vd.float(), o1)
    la.gqa_prefill_rope(qd, kd, vd, o2, positions=pos)
    torch.cuda.synchronize()
    assert torch.equal(o1.bfloat16(), o2)


@pytest.mark.parametrize("B,S,Hq,Hkv,D,seed,positions", [
    (1, 400, 32, 8, 128, 78, False),    # g=4: the shared angle table
    (1, 300, 8, 4, 128, 79, True),      # g=2: angles per lane
    (1, 260, 16, 1, 64, 80, True),      # g=16, D=64
])
def test_prefill_rope_half_pairing_matches_oracle(B, S, Hq, Hkv, D, seed, positions):
    """Half-split pairing through the fused path (keys by rope_qk, queries in
    the kernel) against the oracle's half layout."""
    H.say("prefill_rope half", dict(B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, seed=seed))
    q, k, v = draw_prefill_inputs(B, S, Hq, Hkv, D, "bf16", seed)
    cu = draw_cu_docs(S, seed, 3, 1)
    pos = draw_positions(B, S, 131071 - S, seed) if positions else None
    O, L = _fused(q, k, v, cu, pos, pairing="half")
    Ow, Lw = orc.rope_attention(q, k, v, cu, 500000.0, pos, pairing="half")
    H.assert_close(O, Ow)
    H.assert_lse_close(L, Lw, "LSE")
