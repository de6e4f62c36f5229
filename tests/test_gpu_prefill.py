"""gqa_prefill (with rope_qk in front) against the fp64 oracle, on the GPU.

Sizes here are ones the oracle finishes in seconds yet span several 64-key
tiles, several workgroups per KV head and a ragged tail; the full-size
workloads are covered on sampled rows in ``test_gpu_fullsize.py``.
"""

import numpy as np
import pytest
import torch

import gpu_helpers as H
from oracle import reference as orc
from workloads import CONFIGS, draw_cu_docs, draw_positions, draw_prefill_inputs

pytestmark = pytest.mark.gpu


def _check_case(B, S, Hq, Hkv, D, dtype, seed, n_docs=None, n_docs_max=1, positions=False):
    H.say("prefill", dict(B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, seed=seed, n_docs=n_docs))
    q, k, v = draw_prefill_inputs(B, S, Hq, Hkv, D, dtype, seed)
    cus = [draw_cu_docs(S, seed + 100 * b, n_docs, n_docs_max) for b in range(B)]
    width = max(c.size for c in cus)
    # rows of equal width: pad shorter rows by repeating S (empty documents)
    cu = np.stack([np.concatenate([c, np.full(width - c.size, S, dtype=np.int32)]) for c in cus])
    pos = draw_positions(B, S, 131071 - S, seed) if positions else None
    O, L, _, _ = H.run_prefill(q, k, v, cu, pos)
    Ow = np.zeros((B, S, Hq, D))
    Lw = np.zeros((B, Hq, S))
    for b in range(B):
        pb = None if pos is None else pos[b:b + 1]
        Ow[b:b + 1], Lw[b:b + 1] = orc.rope_attention(q[b:b + 1], k[b:b + 1], v[b:b + 1], cu[b],
                                                      500000.0, pb)
    H.assert_close(O, Ow)
    H.assert_lse_close(L, Lw, "LSE")
    return O, L


def test_tiny_config_fp32():
    w = CONFIGS["tiny"]
    _check_case(w.B, w.S, w.Hq, w.Hkv, w.D, w.dtype, w.seed, n_docs=1)


@pytest.mark.parametrize("B,S,Hq,Hkv,D,seed,nd,ndmax", [
    (1, 333, 16, 1, 128, 31, None, 4),      # g=16, ragged tail, several docs
    (1, 517, 32, 8, 128, 32, None, 8),      # the 8B head layout, g=4
    (1, 300, 8, 8, 64, 33, 3, 1),           # g=1, D=64
    (1, 700, 16, 8, 128, 34, 9, 1),         # g=2, many documents
    (1, 257, 64, 8, 128, 35, 2, 1),         # g=8
    (2, 190, 32, 2, 128, 36, None, 6),      # two sequences, their own documents
    (1, 129, 16, 1, 64, 37, 1, 1),          # g=16, D=64
])
def test_prefill_bf16_matches_oracle(B, S, Hq, Hkv, D, seed, nd, ndmax):
    _check_case(B, S, Hq, Hkv, D, "bf16", seed, nd, ndmax)


def test_prefill_fp32_g16():
    _check_case(1, 200, 32, 2, 128, "fp32", 38, None, 5)


def test_prefill_with_large_positions():
    _check_case(1, 400, 16, 1, 128, "bf16", 39, 2, 1, positions=True)


@pytest.mark.parametrize("S", [1, 2, 63, 64, 65])
def test_prefill_tiny_lengths(S):
    _check_case(1, S, 16, 1, 128, "bf16", 40 + S, 1, 1)


def test_all_documents_of_length_one():
    """Every token its own document: O_i = v_i exactly, LSE = score_ii."""
    S, Hq, Hkv, D = 70, 8, 2, 128
    H.say("prefill length-1 documents")
    q, k, v = draw_prefill_inputs(1, S, Hq, Hkv, D, "bf16", 41)
    cu = np.arange(S + 1, dtype=np.int32)
    O, L, _, _ = H.run_prefill(q, k, v, cu)
    want = v.repeat_interleave(Hq // Hkv, dim=2)
    assert torch.equal(O, want)


# ------------------------------------------------------------- exact probes

def _probe_inputs(S, Hq, Hkv, D, cu, seed):
    """q = 0 (uniform attention over the visible keys) and V channels that
    carry the document index, the KV head index and the key position."""
    _, k, v = draw_prefill_inputs(1, S, Hq, Hkv, D, "bf16", seed)
    q = torch.zeros(1, S, Hq, D, dtype=torch.bfloat16)
    doc = orc.document_of(cu, S)
    v = v.clone()
    v[0, :, :, 0] = torch.as_tensor(doc, dtype=torch.bfloat16)[:, None]
    v[0, :, :, 1] = torch.arange(Hkv, dtype=torch.bfloat16)[None, :]
    v[0, :, :, 2] = torch.arange(S, dtype=torch.bfloat16)[:, None] if S <= 256 else 0
    return q, k, v, doc


@pytest.mark.parametrize("S,Hq,Hkv,D,cu", [
    (250, 16, 1, 128, [0, 1, 2, 90, 91, 200, 250]),
    (256, 32, 8, 128, [0, 64, 65, 127, 256]),
    (200, 8, 2, 64, [0, 200]),
    (1000, 16, 8, 128, [0, 17, 333, 334, 999, 1000]),
])
def test_exact_mask_and_index_probes(S, Hq, Hkv, D, cu):
    H.say("probes", S, Hq, Hkv, D, cu)
    cu = np.asarray(cu, dtype=np.int32)
    q, k, v, doc = _probe_inputs(S, Hq, Hkv, D, cu, 50)
    O, L, _, _ = H.run_prefill(q, k, v, cu)
    g = Hq // Hkv
    start = cu[doc]
    count = np.arange(S) - start + 1
    # causal + document count, exactly: exp(LSE) is the number of visible keys
    assert np.array_equal(np.rint(np.exp(L[0].double().numpy())), np.broadcast_to(count, (Hq, S)))
    # document channel: only same-document keys contribute
    assert np.array_equal(O[0, :, :, 0].double().numpy(), np.broadcast_to(doc[:, None], (S, Hq)))
    # KV-head channel: head h reads KV head h // g
    assert np.array_equal(O[0, :, :, 1].double().numpy(),
                          np.broadcast_to((np.arange(Hq) // g)[None, :], (S, Hq)))
    if S <= 256:   # key-position channel: the mean of the visible key indices, in bf16
        want = torch.tensor((start + np.arange(S)) / 2.0).bfloat16().double().numpy()
        assert np.array_equal(O[0, :, :, 2].double().numpy(), np.broadcast_to(want[:, None], (S, Hq)))


def test_first_token_of_each_document_is_its_value_row():
    S, Hq, Hkv, D = 600, 32, 8, 128
    H.say("first token of document")
    q, k, v = draw_prefill_inputs(1, S, Hq, Hkv, D, "bf16", 51)
    cu = np.array([0, 100, 101, 350, 600], dtype=np.int32)
    O, _, _, _ = H.run_prefill(q, k, v, cu)
    for a in cu[:-1]:
        assert torch.equal(O[0, a], v[0, a].repeat_interleave(Hq // Hkv, dim=0))


def test_deterministic_and_no_out_of_bounds_writes():
    import gqa_attention_rope_02_amd as la
    S, Hq, Hkv, D = 300, 16, 1, 128
    H.say("determinism / guard")
    q, k, v = draw_prefill_inputs(1, S, Hq, Hkv, D, "bf16", 52)
    cu = torch.tensor([[0, 150, 300]], dtype=torch.int32).cuda()
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    guard = torch.full((1, S + 8, Hq, D), 7.0, dtype=torch.bfloat16, device="cuda")
    o = guard[:, 4:4 + S]
    lse = torch.empty(1, Hq, S, dtype=torch.float32, device="cuda")
    la.gqa_prefill(qd, kd, vd, o, lse, cu)
    first = guard.clone()
    la.gqa_prefill(qd, kd, vd, o, lse, cu)
    torch.cuda.synchronize()
    assert torch.equal(first, guard)
    assert (guard[:, :4] == 7.0).all() and (guard[:, 4 + S:] == 7.0).all()


def test_softmax_scale_argument():
    S, Hq, Hkv, D = 150, 8, 2, 64
    H.say("softmax scale")
    q, k, v = draw_prefill_inputs(1, S, Hq, Hkv, D, "bf16", 53)
    O, L, _, _ = H.run_prefill(q, k, v, None, softmax_scale=0.05)
    Ow, Lw = orc.rope_attention(q, k, v, None, 500000.0, scale=0.05)
    H.assert_close(O, Ow)
    H.assert_lse_close(L, Lw, "LSE")
