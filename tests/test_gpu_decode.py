"""gqa_decode + gqa_decode_combine against the fp64 oracle, on the GPU."""

import numpy as np
import pytest
import torch

import gpu_helpers as H
from oracle import reference as orc
from workloads import draw_decode_inputs

pytestmark = pytest.mark.gpu


def build_cache(q_raw, ks, vs, lens, Lmax, fill=float("nan")):
    """Device cache [B,Hkv,Lmax,D]: keys rotated at their slots by rope_qk,
    slots past each sequence's length filled with NaN (any read of them would
    poison the output); the new token's query rotated at position L_b - 1."""
    import gqa_attention_rope_02_amd as la
    B, Hq, D = q_raw.shape
    Hkv = ks[0].shape[0]
    kc = torch.full((B, Hkv, Lmax, D), fill, dtype=torch.bfloat16, device="cuda")
    vc = torch.full((B, Hkv, Lmax, D), fill, dtype=torch.bfloat16, device="cuda")
    for b in range(B):
        L = int(lens[b])
        kc[b, :, :L] = ks[b].cuda()
        vc[b, :, :L] = vs[b].cuda()
    # rotate the whole cache in place, viewed as [B, S=Lmax, H=Hkv, D]
    kview = kc.permute(0, 2, 1, 3)
    la.rope_qk(None, None, kview, kview)
    qd = q_raw.cuda().reshape(B, 1, Hq, D).contiguous()
    pos = torch.as_tensor(np.asarray(lens) - 1, dtype=torch.int32).reshape(B, 1).cuda()
    la.rope_qk(qd, qd, None, None, positions=pos)
    return qd.reshape(B, Hq, D), kc, vc


def run_decode(qr, kc, vc, lens, kv_chunk, out_dtype=torch.bfloat16):
    import gqa_attention_rope_02_amd as la
    B, Hq, D = qr.shape
    Lmax = kc.shape[2]
    max_splits = -(-Lmax // kv_chunk)
    sl = torch.as_tensor(np.asarray(lens), dtype=torch.int32).cuda()
    op = torch.full((B, Hq, max_splits, D), float("nan"), device="cuda")
    lp = torch.full((B, Hq, max_splits), float("nan"), device="cuda")
    la.gqa_decode(qr, kc, vc, sl, kv_chunk, op, lp)
    o = torch.full((B, Hq, D), float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full((B, Hq), float("nan"), device="cuda")
    la.gqa_decode_combine(op, lp, sl, kv_chunk, o, lse)
    torch.cuda.synchronize()
    return op.cpu(), lp.cpu(), o.cpu(), lse.cpu()


def oracle_inputs(q_raw, ks, lens):
    q_rot = np.stack([orc.rope(q_raw[b][None, None], np.array([[lens[b] - 1]]))[0, 0]
                      for b in range(q_raw.shape[0])])
    k_rot = [orc.rope(kb.transpose(0, 1)[None], np.arange(kb.shape[1])[None])[0].transpose(1, 0, 2)
             for kb in ks]
    return q_rot, k_rot


@pytest.mark.parametrize("B,Hq,Hkv,D,lens,Lmax,chunks", [
    (3, 16, 1, 128, (5, 700, 2100), 2200, (64, 256, 1024, 2240)),
    (4, 32, 8, 128, (1, 64, 65, 1500), 1600, (64, 512)),
    (2, 8, 8, 64, (333, 1000), 1024, (128,)),
    (2, 128, 8, 128, (900, 4097), 4100, (1024,)),
    (2, 16, 1, 128, (40000, 60001), 60064, (64, 128)),   # several splits per run
])
def test_decode_matches_oracle(B, Hq, Hkv, D, lens, Lmax, chunks):
    lens = np.asarray(lens, dtype=np.int32)
    q_raw, ks, vs = draw_decode_inputs(B, Hq, Hkv, D, lens, "bf16", 61)
    qr, kc, vc = build_cache(q_raw, ks, vs, lens, Lmax)
    q_rot, k_rot = oracle_inputs(q_raw, ks, lens)
    Ow, Lw = orc.decode(q_rot, k_rot, vs, lens)
    for chunk in chunks:
        H.say("decode", B, Hq, Hkv, D, tuple(lens), "chunk", chunk)
        op, lp, o, lse = run_decode(qr, kc, vc, lens, chunk)
        max_splits = op.shape[2]
        n_runs = H.check_partials(op, lp, q_rot, k_rot, vs, lens, chunk)
        H.say("  runs", n_runs, "of splits", Hq * int(sum(-(-int(L) // chunk) for L in lens)))
        H.assert_close(o, Ow)
        H.assert_lse_close(lse, Lw, "LSE")



def test_decode_equals_last_row_of_gpu_prefill():
    """Decode at length L == the last row of a one-document prefill of L tokens."""
    B, Hq, Hkv, D, L = 1, 16, 1, 128, 777
    H.say("decode vs prefill last row")
    lens = np.array([L], dtype=np.int32)
    q_raw, ks, vs = draw_decode_inputs(B, Hq, Hkv, D, lens, "bf16", 62)
    qr, kc, vc = build_cache(q_raw, ks, vs, lens, L)
    _, _, o, lse = run_decode(qr, kc, vc, lens, 256)
    qp = torch.zeros(1, L, Hq, D, dtype=torch.bfloat16)
    qp[0, -1] = q_raw[0]
    kp = ks[0].transpose(0, 1)[None].contiguous()
    vp = vs[0].transpose(0, 1)[None].contiguous()
    Op, Lp, _, _ = H.run_prefill(qp, kp, vp, None)
    H.assert_close(o[0], Op[0, -1].double().numpy(), what="decode vs prefill O")
    H.assert_lse_close(lse[0], Lp[0, :, -1].double().numpy(), "LSE")


def test_combine_invariant_over_chunk_sizes():
    B, Hq, Hkv, D = 2, 16, 1, 128
    lens = np.array([1234, 3000], dtype=np.int32)
    H.say("combine invariance")
    q_raw, ks, vs = draw_decode_inputs(B, Hq, Hkv, D, lens, "bf16", 63)
    qr, kc, vc = build_cache(q_raw, ks, vs, lens, 3072)
    outs = [run_decode(qr, kc, vc, lens, c)[2].double().numpy() for c in (64, 192, 1024, 3072)]
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 1e-2


def test_decode_fp32_output_and_uniform_probe():
    """q = 0: every visible slot weighs 1, so lse = ln L and, with one split, a V
    channel holding the KV-head index comes back exactly as h // g."""
    B, Hq, Hkv, D = 3, 32, 8, 128
    lens = np.array([1, 100, 1300], dtype=np.int32)
    H.say("decode uniform probe")
    _, ks, vs = draw_decode_inputs(B, Hq, Hkv, D, lens, "bf16", 64)
    for b in range(B):
        vs[b][:, :, 0] = torch.arange(Hkv, dtype=torch.bfloat16)[:, None]
    q0 = torch.zeros(B, Hq, D, dtype=torch.bfloat16)
    qr, kc, vc = build_cache(q0, ks, vs, lens, 1300)
    _, _, o, lse = run_decode(qr, kc, vc, lens, 1344, out_dtype=torch.float32)
    assert np.array_equal(np.rint(np.exp(lse.double().numpy())), np.broadcast_to(lens[:, None], (B, Hq)))
    assert np.array_equal(o[:, :, 0].numpy(), np.broadcast_to(np.arange(Hq) // 4, (B, Hq)).astype(np.float32))
