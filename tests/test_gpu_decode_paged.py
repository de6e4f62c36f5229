"""gqa_decode_paged on the GPU: the same logical caches as gqa_decode, stored
as pages of a shared pool in a scrambled order with a block table per
sequence. The partials and the merged output must equal the contiguous
call's bit for bit (only the addresses differ), and the oracle's within
tolerance."""

import numpy as np
import pytest
import torch

import gpu_helpers as H
from oracle import reference as orc
from test_gpu_decode import build_cache, oracle_inputs, run_decode
from workloads import draw_decode_inputs

pytestmark = pytest.mark.gpu


def page_cache(kc, vc, lens, page_size, seed, layout="slot_head"):
    """Pools [n_pages, page_size, Hkv, D] (or [n_pages, Hkv, page_size, D]
    for layout "head_slot") holding each sequence's slots 0..L_b-1 in
    randomly chosen pages, unused pages and slots NaN; block table [B, n]."""
    B, Hkv, Lmax, D = kc.shape
    need = [-(-int(L) // page_size) for L in lens]
    n_pages = sum(need) + 3                          # a few pages nobody uses
    rng = np.random.default_rng(seed)
    order = rng.permutation(n_pages)
    bt_stride = -(-Lmax // page_size)
    table = np.zeros((B, bt_stride), dtype=np.int32)
    shape = (n_pages, page_size, Hkv, D) if layout == "slot_head" else (n_pages, Hkv, page_size, D)
    kp = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    vp = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    nxt = 0
    for b, L in enumerate(lens):
        for j in range(need[b]):
            pg = int(order[nxt])
            nxt += 1
            table[b, j] = pg
            lo, hi = j * page_size, min((j + 1) * page_size, int(L))
            src_k = kc[b, :, lo:hi].permute(1, 0, 2)     # [slots, Hkv, D]
            src_v = vc[b, :, lo:hi].permute(1, 0, 2)
            if layout == "slot_head":
                kp[pg, :hi - lo] = src_k
                vp[pg, :hi - lo] = src_v
            else:
                kp[pg, :, :hi - lo] = src_k.permute(1, 0, 2)
                vp[pg, :, :hi - lo] = src_v.permute(1, 0, 2)
    if layout == "head_slot":   # the binding takes [n_pages, page_size, Hkv, D]; pass a view
        kp, vp = kp.permute(0, 2, 1, 3), vp.permute(0, 2, 1, 3)
    return kp, vp, torch.as_tensor(table).cuda()


def run_paged(qr, kp, vp, table, lens, kv_chunk, Lmax):
    import gqa_attention_rope_02_amd as la
    B, Hq, D = qr.shape
    max_splits = -(-Lmax // kv_chunk)
    sl = torch.as_tensor(np.asarray(lens), dtype=torch.int32).cuda()
    op = torch.full((B, Hq, max_splits, D), float("nan"), device="cuda")
    lp = torch.full((B, Hq, max_splits), float("nan"), device="cuda")
    la.gqa_decode_paged(qr, kp, vp, table, sl, kv_chunk, op, lp, Lmax)
    o = torch.full((B, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, Hq), float("nan"), device="cuda")
    la.gqa_decode_combine(op, lp, sl, kv_chunk, o, lse)
    torch.cuda.synchronize()
    return op.cpu(), lp.cpu(), o.cpu(), lse.cpu()


@pytest.mark.parametrize("B,Hq,Hkv,D,lens,Lmax,chunk,page,layout", [
    (3, 16, 1, 128, [1, 700, 1234], 1300, 256, 16, "slot_head"),
    (4, 32, 8, 128, [64, 65, 999, 2048], 2048, 128, 64, "slot_head"),
    (2, 128, 8, 128, [3000, 517], 3072, 512, 256, "head_slot"),
    (3, 8, 2, 64, [17, 300, 777], 800, 64, 32, "slot_head"),
])
def test_paged_decode_equals_contiguous_and_oracle(B, Hq, Hkv, D, lens, Lmax, chunk, page, layout):
    H.say("decode paged", dict(B=B, Hq=Hq, Hkv=Hkv, D=D, lens=lens, chunk=chunk, page=page, layout=layout))
    q, ks, vs = draw_decode_inputs(B, Hq, Hkv, D, lens, "bf16", 31)
    qr, kc, vc = build_cache(q, ks, vs, lens, Lmax)
    ref = run_decode(qr, kc, vc, lens, chunk)
    kp, vp, table = page_cache(kc, vc, lens, page, 31, layout)
    got = run_paged(qr, kp, vp, table, lens, chunk, Lmax)
    # the slots the contiguous call writes hold the same bits (NaN where unwritten)
    for g, r in zip(got, ref):
        assert torch.equal(torch.nan_to_num(g, nan=7.0), torch.nan_to_num(r, nan=7.0))
    q_rot, k_rot = oracle_inputs(q, ks, lens)
    Ow, Lw = orc.decode(q_rot, k_rot, vs, lens)
    H.assert_close(got[2], Ow)
    H.assert_lse_close(got[3], Lw, "LSE")
