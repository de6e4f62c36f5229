"""gqa_attention_backward and rope_qk_backward on the GPU against the oracle.

The forward (gqa_prefill on the GPU) supplies o and lse; dq, dk, dv are
compared with the oracle's fp64 gradients of the same bf16 inputs
(oracle.reference.attention_backward_rows, which also gives each element's
term magnitudes). The bar is per element, from the arithmetic: every element
within 2^-7 of the sum of its terms' absolute values plus 2^-8 of its own
value (twice the worst case of two bf16 roundings per term and the output's
rounding), and the mean error within 2^-8 of the mean of (root of the sum of
squared terms + |value|) (the expected error of independent roundings, with
room); the derivation sits beside the constants in gpu_helpers.
"""

import numpy as np
import pytest
import torch

import gpu_helpers as H
from oracle import reference as orc
from workloads import draw_cu_docs, draw_grad_output, draw_positions, draw_prefill_inputs, sample_rows

pytestmark = pytest.mark.gpu

BASE = 500000.0


def _dev(x):
    return x.to(torch.device("cuda"))


def check_grads(dq, dk, dv, q, k, v, dout, rows, keys, cu, scale=None, what=""):
    """dq at rows and dk, dv at keys of one sequence against the oracle."""
    Wq, Wk, Wv, (l1, l2) = H.backward_oracle_threaded(q, k, v, dout, rows, keys, cu, scale=scale)
    H.assert_grad_bar(dq[rows], Wq, l1[0], l2[0], f"dq{what}")
    H.assert_grad_bar(dk[keys], Wk, l1[1], l2[1], f"dk{what}")
    H.assert_grad_bar(dv[keys], Wv, l1[2], l2[2], f"dv{what}")


def run_backward(qr, kr, v, dout, cu, softmax_scale=0.0, workspace="auto"):
    """gqa_prefill then gqa_attention_backward on device tensors; (dq, dk, dv) on the CPU."""
    import gqa_attention_rope_02_amd as la
    B, S, Hq, D = qr.shape
    cud = None if cu is None else _dev(torch.as_tensor(np.asarray(cu), dtype=torch.int32).reshape(B, -1))
    o = torch.full_like(qr, float("nan"))
    lse = torch.full((B, Hq, S), float("nan"), dtype=torch.float32, device=qr.device)
    la.gqa_prefill(qr, kr, v, o, lse, cud, softmax_scale)
    dq = torch.full_like(qr, float("nan"))
    dk = torch.full_like(kr, float("nan"))
    dv = torch.full_like(v, float("nan"))
    delta = torch.full((B, Hq, S), float("nan"), dtype=torch.float32, device=qr.device)
    if workspace == "nan":      # slots a piece leaves unwritten show up as NaN
        workspace = la.backward_workspace(B, S, kr.shape[2], D, qr.device).fill_(float("nan"))
    la.gqa_attention_backward(qr, kr, v, o, dout, lse, dq, dk, dv, delta, cud, softmax_scale, workspace)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def _check_case(B, S, Hq, Hkv, D, seed, cus, softmax_scale=0.0, workspace="nan"):
    q, k, v = draw_prefill_inputs(B, S, Hq, Hkv, D, "bf16", seed)
    dout = draw_grad_output(B, S, Hq, D, "bf16", seed)
    cu = None
    if cus is not None:
        width = max(c.size for c in cus)
        cu = np.stack([np.concatenate([c, np.full(width - c.size, S, dtype=np.int32)]) for c in cus])
    dq, dk, dv = run_backward(_dev(q), _dev(k), _dev(v), _dev(dout), cu, softmax_scale, workspace)
    sc = None if softmax_scale == 0.0 else softmax_scale
    every = np.arange(S)
    for b in range(B):
        check_grads(dq[b], dk[b], dv[b], q[b], k[b], v[b], dout[b], every, every,
                    None if cu is None else cu[b], sc, f" seq {b}")


@pytest.mark.parametrize("B,S,Hq,Hkv,D,seed,nd", [
    (1, 700, 32, 8, 128, 201, 3),     # 8B heads, ragged length, documents
    (1, 520, 16, 1, 128, 202, 2),     # g = 16
    (2, 300, 8, 8, 64, 203, 3),       # g = 1, D = 64, two sequences
    (1, 257, 8, 2, 128, 204, None),   # one document, one token past a block
    (1, 450, 128, 8, 128, 205, 4),    # 405B heads (g = 16)
    (1, 390, 16, 4, 128, 206, 6),     # many short documents
    (1, 2200, 32, 8, 128, 210, 1),    # long query ranges cut into pieces (g = 4: 137 query blocks)
    (1, 1300, 16, 2, 64, 213, 1),     # g = 8, D = 64, cut into pieces (162 query blocks)
    (1, 400, 4, 2, 128, 214, 3),      # g = 2
])
def test_backward_matches_oracle(B, S, Hq, Hkv, D, seed, nd):
    H.say("backward", dict(B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, seed=seed, nd=nd))
    cus = None if nd is None else [draw_cu_docs(S, seed + 100 * b, nd, 6) for b in range(B)]
    _check_case(B, S, Hq, Hkv, D, seed, cus)


def test_backward_without_workspace():
    """No workspace: every key block's whole query range on one workgroup
    (the ranges here are long enough to be cut when a workspace is given)."""
    H.say("backward without workspace")
    _check_case(1, 1100, 16, 1, 128, 211, [draw_cu_docs(1100, 211, 2, 6)], workspace=None)


def test_backward_empty_documents_and_explicit_scale():
    """Empty documents (repeated offsets) and a softmax scale that is not 1/sqrt(D)."""
    S = 333
    H.say("backward empty documents")
    cu = np.array([0, 0, 50, 50, 51, 200, 200, S], dtype=np.int32)
    _check_case(1, S, 16, 2, 128, 207, [cu], softmax_scale=0.05)


def test_backward_single_token_gives_dv_dout_and_zero_dq_dk():
    """S = 1: the only weight is 1, so dv = dout and dS = dout.v - dout.o = 0
    (o = v): dq and dk vanish up to the rounding of the two dot products,
    which are summed in different orders (about 1e-6 of |dout| |v|)."""
    import gqa_attention_rope_02_amd as la
    H.say("backward single token")
    q, k, v = draw_prefill_inputs(2, 1, 32, 8, 128, "bf16", 208)
    dout = draw_grad_output(2, 1, 32, 128, "bf16", 208)
    dq, dk, dv = run_backward(_dev(q), _dev(k), _dev(v), _dev(dout), None)
    assert dq.abs().max().item() < 1e-4 and dk.abs().max().item() < 1e-4
    want = dout.float().reshape(2, 1, 8, 4, 128).sum(dim=3)
    assert torch.allclose(dv.float(), want, rtol=1e-2, atol=1e-2)


def test_rope_backward_is_the_transpose():
    """rope_qk_backward against the oracle's rotation by the negated angles,
    and undoing rope_qk (both pairings, explicit positions)."""
    import gqa_attention_rope_02_amd as la
    B, S, Hq, Hkv, D = 1, 200, 8, 2, 128
    H.say("rope backward")
    q, k, _ = draw_prefill_inputs(B, S, Hq, Hkv, D, "fp32", 209)
    pos = draw_positions(B, S, 131071, 209)
    pd = _dev(torch.as_tensor(pos))
    for pairing in ("adjacent", "half"):
        qo, ko = torch.empty_like(_dev(q)), torch.empty_like(_dev(k))
        la.rope_qk_backward(_dev(q), qo, _dev(k), ko, positions=pd, rope_base=BASE, rope_pairing=pairing)
        Wq = orc.rope(q, -pos.astype(np.int64), BASE, pairing)
        Wk = orc.rope(k, -pos.astype(np.int64), BASE, pairing)
        assert np.abs(qo.cpu().double().numpy() - Wq).max() < 1e-5
        assert np.abs(ko.cpu().double().numpy() - Wk).max() < 1e-5
        qr = torch.empty_like(qo)
        la.rope_qk(qo, qr, None, None, positions=pd, rope_base=BASE, rope_pairing=pairing)
        assert (qr.cpu() - q).abs().max().item() < 1e-5


# documents up to this length are compared in full (every row, every key)
FULL_DOC = 5000
# longer documents: dq on sampled rows; dk, dv on every key of the last
# LAST_KEYS of the document (key blocks whose query ranges are long enough to
# be cut into pieces; a key earlier in the document needs the softmax of every
# later row, beyond what the oracle affords there)
LAST_KEYS = 1024


@pytest.mark.parametrize("name", ["llama8b", "llama405b"])
def test_backward_full_size(name):
    """The workloads' full shapes, in the launch configuration the benchmark
    times. The mask keeps documents apart, so every gradient of a document is
    that of the document alone; the oracle works on the whole sequence with
    its document boundaries all the same. Documents of up to 5000 tokens (the
    8B workload's 4623-token one included) are compared at every row and key.
    Longer ones (405B: 16754 and 12125 tokens) are compared at sampled query
    rows (the first and last two, both sides of drawn query-tile edges, and
    uniform draws) for dq, and for dk, dv at every key of the document's last
    1024 (whose query ranges run past the length at which the key-stationary
    kernel cuts them into pieces). Every document is also checked against two identities of the
    gradients (the weights of a row sum to one): per KV head, the dv of a
    document's keys sum to the dout of its queries over the head's group, and
    the dk sum to zero (each row of dS sums to zero); both within 2^-7 of the
    sum of magnitudes (every term within a few bf16 roundings)."""
    from workloads import CONFIGS
    w = CONFIGS[name]
    H.say("backward full size", name)
    q, k, v = draw_prefill_inputs(w.B, w.S, w.Hq, w.Hkv, w.D, w.dtype, w.seed)
    dout = draw_grad_output(w.B, w.S, w.Hq, w.D, w.dtype, w.seed)
    cu = draw_cu_docs(w.S, w.seed, w.n_docs, w.n_docs_max)
    dq, dk, dv = run_backward(_dev(q), _dev(k), _dev(v), _dev(dout), cu[None, :])
    g = w.Hq // w.Hkv
    rng = np.random.default_rng(w.seed + 11)
    tile = 256 // g                            # query tokens per dq workgroup
    full_rows, rows, keys = [], [], []
    for a, b in zip(cu[:-1].tolist(), cu[1:].tolist()):
        if b == a:
            continue
        sdv = dv[0, a:b].double().sum(dim=0)                               # [Hkv, D]
        sdo = dout[0, a:b].double().reshape(b - a, w.Hkv, g, w.D).sum(dim=(0, 2))
        assert ((sdv - sdo).abs() <= 2 ** -7 * dv[0, a:b].double().abs().sum(dim=0) + 1e-6).all()
        sdk = dk[0, a:b].double().sum(dim=0)
        assert (sdk.abs() <= 2 ** -7 * dk[0, a:b].double().abs().sum(dim=0) + 1e-6).all()
        if b - a <= FULL_DOC:
            full_rows.append(np.arange(a, b))
            continue
        r = sample_rows(b - a, [0, b - a], int(rng.integers(1 << 30)), n_random=256, tile=tile, n_edges=32)
        rows.append(np.unique(np.concatenate([r, [1, b - a - 2]])) + a)
        keys.append(np.arange(b - LAST_KEYS, b))
    every = np.concatenate(full_rows)
    H.say("backward full size oracle: whole documents", every.size, "rows and keys")
    check_grads(dq[0], dk[0], dv[0], q[0], k[0], v[0], dout[0], every, every, cu, what=" short documents")
    if rows:
        rows, keys = np.concatenate(rows), np.concatenate(keys)
        H.say("backward full size oracle: long documents", rows.size, "rows", keys.size, "keys")
        check_grads(dq[0], dk[0], dv[0], q[0], k[0], v[0], dout[0], rows, keys, cu, what=" long documents")


def test_backward_is_deterministic_and_writes_in_bounds():
    """Two calls give the same bits (no atomics; pieces merged in a fixed
    order), and nothing is written outside dq, dk, dv: the outputs are views
    into NaN-filled buffers with a guard token before and after."""
    import gqa_attention_rope_02_amd as la
    B, S, Hq, Hkv, D = 1, 1200, 32, 8, 128
    H.say("backward determinism and bounds")
    q, k, v = draw_prefill_inputs(B, S, Hq, Hkv, D, "bf16", 212)
    dout = _dev(draw_grad_output(B, S, Hq, D, "bf16", 212))
    cu = _dev(torch.as_tensor(draw_cu_docs(S, 212, 2, 6), dtype=torch.int32).reshape(1, -1))
    qd, kd, vd = _dev(q), _dev(k), _dev(v)
    o = torch.empty_like(qd)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=qd.device)
    la.gqa_prefill(qd, kd, vd, o, lse, cu)
    outs = []
    for _ in range(2):
        gq = torch.full((B, S + 2, Hq, D), float("nan"), dtype=torch.bfloat16, device=qd.device)
        gk = torch.full((B, S + 2, Hkv, D), float("nan"), dtype=torch.bfloat16, device=qd.device)
        gv = torch.full_like(gk, float("nan"))
        la.gqa_attention_backward(qd, kd, vd, o, dout, lse, gq[:, 1:S + 1], gk[:, 1:S + 1], gv[:, 1:S + 1],
                                  None, cu)
        torch.cuda.synchronize()
        for g in (gq, gk, gv):
            assert torch.isnan(g[:, 0]).all() and torch.isnan(g[:, S + 1]).all()
            assert torch.isfinite(g[:, 1:S + 1]).all()
        outs.append((gq.cpu(), gk.cpu(), gv.cpu()))
    for a, b in zip(*outs):
        assert torch.equal(a[:, 1:S + 1], b[:, 1:S + 1])


def test_backward_on_views_of_a_packed_projection():
    """q, k, v as head slices of one [B, S, Hq + 2 Hkv, D] tensor (the output of
    a fused projection; token stride (Hq + 2 Hkv) D), dq written into a view
    of a wider buffer: strides are honoured and the result equals the
    contiguous call's bit for bit."""
    import gqa_attention_rope_02_amd as la
    B, S, Hq, Hkv, D = 1, 700, 16, 4, 128
    H.say("backward on packed views")
    q, k, v = draw_prefill_inputs(B, S, Hq, Hkv, D, "bf16", 215)
    dout = _dev(draw_grad_output(B, S, Hq, D, "bf16", 215))
    cu = _dev(torch.as_tensor(draw_cu_docs(S, 215, 3, 6), dtype=torch.int32).reshape(1, -1))
    qkv = torch.cat([q, k, v], dim=2).to(torch.device("cuda"))
    qv, kv_, vv = qkv[:, :, :Hq], qkv[:, :, Hq:Hq + Hkv], qkv[:, :, Hq + Hkv:]
    qd, kd, vd = qv.contiguous(), kv_.contiguous(), vv.contiguous()
    o = torch.empty_like(qd)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=qd.device)
    la.gqa_prefill(qd, kd, vd, o, lse, cu)
    ref = [torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)]
    la.gqa_attention_backward(qd, kd, vd, o, dout, lse, *ref, None, cu)
    wide = torch.full((B, S, 2 * Hq, D), float("nan"), dtype=torch.bfloat16, device=qd.device)
    gq = wide[:, :, Hq:]
    gk, gv = torch.empty_like(kd), torch.empty_like(vd)
    la.gqa_attention_backward(qv, kv_, vv, o, dout, lse, gq, gk, gv, None, cu)
    torch.cuda.synchronize()
    assert torch.equal(gq.cpu(), ref[0].cpu()) and torch.equal(gk.cpu(), ref[1].cpu())
    assert torch.equal(gv.cpu(), ref[2].cpu())
    assert torch.isnan(wide[:, :, :Hq]).all()
