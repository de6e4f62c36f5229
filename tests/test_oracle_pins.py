"""Pins of the fp64 oracle against things other than itself (CPU only).

Each check ties the oracle to brute force, to a library routine, or to an
invariant / closed form the method fixes, so that a plausible slip (a dropped
scale, a wrong sign in the rotation, the wrong channel pairing, h % Hkv instead
of h // g, a strict instead of non-strict causal test, a mask leaking across
documents, d_model instead of head_dim in theta_k) fails at least one of them.
``test_oracle_mutations.py`` plants those slips and checks that they do.
"""

import math

import numpy as np
import pytest
import torch

from oracle import brute, reference as orc
from workloads import draw_cu_docs, draw_positions, draw_prefill_inputs

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _tiny(seed=0, B=2, S=13, Hq=4, Hkv=2, D=8, dtype="fp32"):
    q, k, v = draw_prefill_inputs(B, S, Hq, Hkv, D, dtype, seed)
    return q, k, v


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("seed,S,Hq,Hkv,D,ndocs,pos", [
    (0, 13, 4, 2, 8, 3, False),
    (1, 9, 4, 1, 6, 1, False),
    (2, 16, 4, 4, 4, 2, True),
    (3, 11, 6, 2, 8, 4, True),
])
def test_brute_force_equals_oracle(seed, S, Hq, Hkv, D, ndocs, pos):
    q, k, v = _tiny(seed, 2, S, Hq, Hkv, D, "bf16")
    cu = draw_cu_docs(S, seed, n_docs=ndocs)
    positions = draw_positions(2, S, 131071, seed) if pos else None
    O, L = orc.rope_attention(q, k, v, cu, 500000.0, positions)
    qb, kb, vb = (x.double().numpy().tolist() for x in (q, k, v))
    Ob, Lb = brute.brute_rope_attention(qb, kb, vb, cu.tolist(), 500000.0,
                                        None if positions is None else positions.tolist())
    np.testing.assert_allclose(O, np.array(Ob), rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, np.array(Lb), rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed,S,Hq,Hkv,D,ndocs", [(7, 15, 4, 2, 8, 3), (8, 12, 8, 1, 6, 1)])
def test_brute_force_equals_row_oracle(seed, S, Hq, Hkv, D, ndocs):
    """The row-restricted oracle (rotating only the rows and document windows it
    needs) against brute force, rows in a scrambled order."""
    q, k, v = _tiny(seed, 1, S, Hq, Hkv, D, "bf16")
    cu = draw_cu_docs(S, seed, n_docs=ndocs)
    rows = np.random.default_rng(seed).permutation(S)[: S - 2]
    O, L = orc.rope_attention_rows(q[0], k[0], v[0], rows, cu, 500000.0)
    qb, kb, vb = (x.double().numpy().tolist() for x in (q, k, v))
    Ob, Lb = brute.brute_rope_attention(qb, kb, vb, cu.tolist(), 500000.0)
    np.testing.assert_allclose(O, np.array(Ob)[0][rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, np.array(Lb)[0][:, rows], rtol=0, atol=1e-12)


def test_row_oracle_matches_block_oracle_at_moderate_size():
    """Many documents, GQA 4:1, rows spanning block and document edges."""
    S, Hq, Hkv, D = 700, 16, 4, 64
    q, k, v = draw_prefill_inputs(1, S, Hq, Hkv, D, "bf16", 9)
    cu = draw_cu_docs(S, 9, n_docs_max=8)
    rows = np.unique(np.concatenate([cu[:-1], cu[1:] - 1, np.arange(0, S, 37), [63, 64, 65]]))
    O, L = orc.rope_attention_rows(q[0], k[0], v[0], rows, cu, 500000.0, block=16)
    Ow, Lw = orc.rope_attention(q, k, v, cu, 500000.0, rows=rows)
    np.testing.assert_allclose(O, Ow[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Lw[0], rtol=0, atol=1e-12)


# ----------------------------------------------------------- library routine

def _torch_rope_complex(x, positions, base):
    """RoPE as complex multiplication: (x_2k + i x_2k+1) * e^{i m theta_k}."""
    x = x.double()
    D = x.shape[-1]
    inv_freq = 1.0 / (base ** (torch.arange(0, D, 2, dtype=torch.float64) / D))
    ang = torch.as_tensor(positions, dtype=torch.float64)[..., None] * inv_freq
    rot = torch.polar(torch.ones_like(ang), ang)[:, :, None, :]
    xc = torch.view_as_complex(x.reshape(*x.shape[:-1], D // 2, 2).contiguous())
    return torch.view_as_real(xc * rot).reshape(x.shape)


@pytest.mark.parametrize("seed,S,Hq,Hkv,D,ndocs", [(4, 40, 8, 2, 16, 3), (5, 33, 16, 1, 32, 1),
                                                    (6, 64, 4, 4, 64, 5)])
def test_sdpa_library_route(seed, S, Hq, Hkv, D, ndocs):
    B = 2
    q, k, v = _tiny(seed, B, S, Hq, Hkv, D, "bf16")
    cu = draw_cu_docs(S, seed, n_docs=ndocs)
    positions = draw_positions(B, S, 100000, seed)
    O, _ = orc.rope_attention(q, k, v, cu, 500000.0, positions)
    g = Hq // Hkv
    qr = _torch_rope_complex(q, positions, 500000.0).transpose(1, 2)            # [B,H,S,D]
    kr = _torch_rope_complex(k, positions, 500000.0).repeat_interleave(g, dim=2).transpose(1, 2)
    vv = v.double().repeat_interleave(g, dim=2).transpose(1, 2)
    doc = torch.bucketize(torch.arange(S), torch.as_tensor(cu[1:-1]), right=True)
    i = torch.arange(S)
    mask = (i[None, :] <= i[:, None]) & (doc[None, :] == doc[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(
        qr.contiguous(), kr.contiguous(), vv.contiguous(), attn_mask=mask)
    np.testing.assert_allclose(O, ref.transpose(1, 2).numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- backward

def test_rope_at_negated_positions_undoes_rope():
    """The rotation is orthogonal and its inverse is the rotation by minus the
    angle: rope at -m after rope at m returns the input (both pairings), and
    it preserves every pair's norm."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((1, 9, 3, 16))
    pos = rng.integers(0, 131072, size=(1, 9))
    for pairing in ("adjacent", "half"):
        y = orc.rope(x, pos, 500000.0, pairing)
        np.testing.assert_allclose(orc.rope(y, -pos, 500000.0, pairing), x, rtol=0, atol=1e-12)
        np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


def test_backward_matches_finite_differences():
    """Central differences of L = sum(dO * O) through ``attention`` (the
    forward oracle) on a tiny GQA problem with two documents: every gradient
    entry of q, k and v agrees to 1e-7 (step 1e-5 in fp64)."""
    rng = np.random.default_rng(5)
    B, S, Hq, Hkv, D = 1, 7, 4, 2, 4
    qr, kr, v = (rng.standard_normal((B, S, H, D)) for H in (Hq, Hkv, Hkv))
    dO = rng.standard_normal((B, S, Hq, D))
    cu = np.array([0, 3, 7])
    dq, dk, dv = orc.attention_backward(qr, kr, v, dO, cu)
    loss = lambda a, b_, c: float(np.sum(orc.attention(a, b_, c, cu)[0] * dO))
    eps = 1e-5
    for x, grad, which in ((qr, dq, 0), (kr, dk, 1), (v, dv, 2)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [qr, kr, v]
            args_m = [qr, kr, v]
            args_p[which], args_m[which] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=0, atol=1e-7)


def test_backward_matches_autograd_of_sdpa():
    """Library route: torch autograd of fp64 scaled_dot_product_attention with
    the KV heads repeated and the causal + document mask; the repeated heads'
    gradients summed per KV head."""
    rng = np.random.default_rng(6)
    B, S, Hq, Hkv, D = 2, 20, 8, 2, 16
    g = Hq // Hkv
    qr, kr, v = (rng.standard_normal((B, S, H, D)) for H in (Hq, Hkv, Hkv))
    dO = rng.standard_normal((B, S, Hq, D))
    cu = np.array([0, 6, 13, 20])
    dq, dk, dv = orc.attention_backward(qr, kr, v, dO, cu)
    tq = torch.tensor(qr, requires_grad=True)
    tk = torch.tensor(kr, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    doc = torch.bucketize(torch.arange(S), torch.as_tensor(cu[1:-1]), right=True)
    i = torch.arange(S)
    mask = (i[None, :] <= i[:, None]) & (doc[None, :] == doc[:, None])
    out = torch.nn.functional.scaled_dot_product_attention(
        tq.transpose(1, 2), tk.repeat_interleave(g, dim=2).transpose(1, 2),
        tv.repeat_interleave(g, dim=2).transpose(1, 2), attn_mask=mask)
    (out.transpose(1, 2) * torch.tensor(dO)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed,S,Hq,Hkv,D,cu", [
    (11, 29, 4, 2, 8, [0, 9, 9, 21, 29]),    # an empty document
    (12, 40, 6, 3, 4, [0, 40]),
    (13, 33, 8, 1, 8, [0, 1, 2, 17, 33]),   # one-token documents, g = 8
])
def test_restricted_backward_equals_full_backward(seed, S, Hq, Hkv, D, cu):
    """The row/key-restricted backward returns exactly the full backward's
    dq at the asked rows and dk, dv at the asked keys, for any subsets (rows in
    any order, keys repeated), with blocks smaller than a document."""
    rng = np.random.default_rng(seed)
    qr, kr, v = (rng.standard_normal((1, S, H, D)) for H in (Hq, Hkv, Hkv))
    dO = rng.standard_normal((1, S, Hq, D))
    cu = np.array(cu)
    Wq, Wk, Wv = orc.attention_backward(qr, kr, v, dO, cu)
    for trial in range(3):
        rows = rng.permutation(S)[:rng.integers(1, S)]
        keys = rng.integers(0, S, size=rng.integers(1, S))
        dq, dk, dv = orc.attention_backward_rows(qr[0], kr[0], v[0], dO[0], rows, keys, cu, block=5)
        np.testing.assert_allclose(dq, Wq[0, rows], rtol=0, atol=1e-12)
        np.testing.assert_allclose(dk, Wk[0, keys], rtol=0, atol=1e-12)
        np.testing.assert_allclose(dv, Wv[0, keys], rtol=0, atol=1e-12)


def test_restricted_backward_matches_autograd_of_sdpa():
    """The restricted backward against the library route directly (torch
    autograd of fp64 scaled_dot_product_attention, KV heads repeated), with an
    explicit softmax scale."""
    rng = np.random.default_rng(14)
    S, Hq, Hkv, D = 24, 8, 2, 16
    g = Hq // Hkv
    qr, kr, v = (rng.standard_normal((S, H, D)) for H in (Hq, Hkv, Hkv))
    dO = rng.standard_normal((S, Hq, D))
    cu = np.array([0, 10, 24])
    tq, tk, tv = (torch.tensor(x[None], requires_grad=True) for x in (qr, kr, v))
    doc = torch.bucketize(torch.arange(S), torch.as_tensor(cu[1:-1]), right=True)
    i = torch.arange(S)
    mask = (i[None, :] <= i[:, None]) & (doc[None, :] == doc[:, None])
    out = torch.nn.functional.scaled_dot_product_attention(
        tq.transpose(1, 2), tk.repeat_interleave(g, dim=2).transpose(1, 2),
        tv.repeat_interleave(g, dim=2).transpose(1, 2), attn_mask=mask, scale=0.3)
    (out.transpose(1, 2) * torch.tensor(dO[None])).sum().backward()
    rows, keys = np.array([23, 0, 10, 9, 15]), np.array([0, 9, 10, 23, 4])
    dq, dk, dv = orc.attention_backward_rows(qr, kr, v, dO, rows, keys, cu, scale=0.3)
    np.testing.assert_allclose(dq, tq.grad[0].numpy()[rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad[0].numpy()[keys], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad[0].numpy()[keys], rtol=0, atol=1e-12)


def test_restricted_backward_magnitudes():
    """The per-element magnitudes: with zero queries every visible weight
    of row i is 1 / (i - start + 1), so dv_j's terms are dO_i / (i - start + 1)
    over the rows i >= j of j's document (closed forms for the sum of absolute
    values and the root of the sum of squares), and dk's terms are all zero;
    a document of one token has P = 1 and dS = 0, so dq vanishes and only its
    row term's share is left: l1 = scale (sum_d |dO_d| |v_d|) |k| and
    l2 = scale sqrt(sum_d dO_d^2 v_d^2) |k|. For random inputs,
    |gradient| <= l1, l2 <= l1, and for dk and dv l1 <= sqrt(terms * D) l2."""
    rng = np.random.default_rng(15)
    S, Hq, Hkv, D = 20, 4, 2, 8
    g = Hq // Hkv
    cu = np.array([0, 1, 12, 20])
    kr, v = (rng.standard_normal((S, Hkv, D)) for _ in range(2))
    dO = rng.standard_normal((S, Hq, D))
    rows, keys = np.arange(S), np.arange(S)
    dq, dk, dv, (l1, l2) = orc.attention_backward_rows(np.zeros((S, Hq, D)), kr, v, dO, rows, keys, cu,
                                                       magnitudes=True)
    doc = orc.document_of(cu, S)
    for j in range(S):
        a, e = cu[doc[j]], cu[doc[j] + 1]
        w = 1.0 / (np.arange(j, e) - a + 1)                                  # P_ij for i >= j
        t = w[:, None, None, None] * dO[j:e].reshape(e - j, Hkv, g, D)     # terms over (i, head)
        t = t.transpose(0, 2, 1, 3).reshape(-1, Hkv, D)
        np.testing.assert_allclose(dv[j], t.sum(axis=0), rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(l1[2][j], np.abs(t).sum(axis=0), rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(l2[2][j], np.sqrt((t * t).sum(axis=0)), rtol=1e-13, atol=1e-13)
    assert np.all(dk == 0) and np.all(l1[1] == 0) and np.all(l2[1] == 0)
    assert np.all(dq[0] == 0)
    sc = 1.0 / np.sqrt(D)
    for h in range(Hq):
        kv = h // g
        A = np.sum(np.abs(dO[0, h]) * np.abs(v[0, kv]))
        R = np.sqrt(np.sum((dO[0, h] * v[0, kv]) ** 2))
        np.testing.assert_allclose(l1[0][0, h], sc * A * np.abs(kr[0, kv]), rtol=1e-13, atol=0)
        np.testing.assert_allclose(l2[0][0, h], sc * R * np.abs(kr[0, kv]), rtol=1e-13, atol=0)
    qr = rng.standard_normal((S, Hq, D))
    dq, dk, dv, (l1, l2) = orc.attention_backward_rows(qr, kr, v, dO, rows, keys, cu, magnitudes=True)
    for x, a1, a2 in zip((dq, dk, dv), l1, l2):
        assert np.all(np.abs(x) <= a1 * (1 + 1e-12) + 1e-15)
        assert np.all(a2 <= a1 * (1 + 1e-12) + 1e-15)
    for a1, a2 in zip(l1[1:], l2[1:]):          # dk, dv: at most S g terms of D-fold row terms
        assert np.all(a1 <= np.sqrt(S * g * D) * a2 * (1 + 1e-12) + 1e-15)


# ---------------------------------------------------------------- invariants

def test_gqa_equals_mha_with_repeated_kv():
    q, k, v = _tiny(7, 1, 24, 8, 2, 16, "bf16")
    cu = np.array([0, 10, 24], dtype=np.int32)
    O1, L1 = orc.rope_attention(q, k, v, cu)
    O2, L2 = orc.rope_attention(q, k.repeat_interleave(4, dim=2), v.repeat_interleave(4, dim=2), cu)
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L1, L2, rtol=0, atol=1e-13)


def test_document_mask_equals_separate_documents():
    S = 50
    q, k, v = _tiny(8, 1, S, 8, 2, 16, "bf16")
    cu = np.array([0, 1, 17, 18, 41, 50], dtype=np.int32)     # includes length-1 documents
    O, L = orc.rope_attention(q, k, v, cu)
    for a, b in zip(cu[:-1], cu[1:]):
        # each document alone, positions restarted at 0 (relative-offset property)
        Od, Ld = orc.rope_attention(q[:, a:b], k[:, a:b], v[:, a:b])
        np.testing.assert_allclose(O[:, a:b], Od, rtol=0, atol=1e-10)
        np.testing.assert_allclose(L[:, :, a:b], Ld, rtol=0, atol=1e-10)


def test_scores_depend_only_on_offset():
    q, k, v = _tiny(9, 1, 20, 4, 2, 32, "fp32")
    base_pos = np.arange(20)[None, :]
    O0, L0 = orc.rope_attention(q, k, v, None, 500000.0, base_pos)
    for shift in (1, 777, 123456):
        O1, L1 = orc.rope_attention(q, k, v, None, 500000.0, base_pos + shift)
        np.testing.assert_allclose(O1, O0, rtol=0, atol=1e-10)
        np.testing.assert_allclose(L1, L0, rtol=0, atol=1e-10)


def test_rope_position_zero_is_identity_and_norms_preserved():
    x = torch.randn(1, 5, 3, 16, generator=torch.Generator().manual_seed(3), dtype=torch.float64)
    r0 = orc.rope(x, np.zeros((1, 5)), 500000.0)
    assert np.array_equal(r0, x.numpy())
    r = orc.rope(x, np.array([[1, 10, 1000, 65536, 131071]]), 500000.0)
    pairs = lambda a: np.hypot(a[..., 0::2], a[..., 1::2])
    np.testing.assert_allclose(pairs(r), pairs(x.numpy()), rtol=1e-14, atol=0)


def test_rope_unit_vectors_show_pairing_and_direction():
    """e_{2k} at position m rotates to (cos m theta_k, sin m theta_k) in channels
    (2k, 2k+1); e_{2k+1} to (-sin, cos). Channels of other pairs stay 0."""
    D, m = 8, 3
    theta = [1.0, 500000.0 ** -0.25, 500000.0 ** -0.5, 500000.0 ** -0.75]  # base^(-2k/8)
    for kk in range(D // 2):
        for which in (0, 1):
            x = np.zeros((1, 1, 1, D))
            x[..., 2 * kk + which] = 1.0
            r = orc.rope(x, np.array([[m]]), 500000.0)[0, 0, 0]
            c, s = math.cos(m * theta[kk]), math.sin(m * theta[kk])
            want = np.zeros(D)
            want[2 * kk], want[2 * kk + 1] = (c, s) if which == 0 else (-s, c)
            np.testing.assert_allclose(r, want, rtol=0, atol=1e-15)


def _to_adjacent(x):
    """Channel permutation taking the half-split layout to the adjacent one:
    half channel k goes to 2k and half channel k + D/2 to 2k + 1."""
    x = np.asarray(x)
    D = x.shape[-1]
    out = np.empty_like(x)
    out[..., 0::2], out[..., 1::2] = x[..., :D // 2], x[..., D // 2:]
    return out


def test_rope_half_pairing_is_adjacent_pairing_under_a_channel_permutation():
    """Both layouts rotate the same pairs by the same angles; only where the
    pair's channels sit differs. So rotating in the half layout equals moving
    the channels to the adjacent layout, rotating there, and moving back."""
    x = torch.randn(2, 6, 3, 16, generator=torch.Generator().manual_seed(11), dtype=torch.float64).numpy()
    pos = np.array([[0, 1, 7, 1000, 65536, 131071], [3, 4, 5, 6, 7, 8]])
    half = orc.rope(x, pos, 500000.0, "half")
    adj = orc.rope(_to_adjacent(x), pos, 500000.0, "adjacent")
    np.testing.assert_array_equal(_to_adjacent(half), adj)
    assert np.array_equal(orc.rope(x, np.zeros((2, 6)), 500000.0, "half"), x)
    with pytest.raises(ValueError):
        orc.rope(x, pos, 500000.0, "interleaved")


def test_rope_half_unit_vector():
    """e_k (k < D/2) at position m goes to cos m theta_k in channel k and
    sin m theta_k in channel k + D/2; e_{k+D/2} to (-sin, cos) there."""
    D, m = 8, 5
    th = orc.rope_frequencies(D, 500000.0)
    for kk in range(D // 2):
        c, s = math.cos(m * th[kk]), math.sin(m * th[kk])
        for which, want_pair in ((0, (c, s)), (1, (-s, c))):
            x = np.zeros((1, 1, 1, D))
            x[..., kk + which * D // 2] = 1.0
            r = orc.rope(x, np.array([[m]]), 500000.0, "half")[0, 0, 0]
            want = np.zeros(D)
            want[kk], want[kk + D // 2] = want_pair
            np.testing.assert_allclose(r, want, rtol=0, atol=1e-15)


def test_attention_with_half_pairing_equals_permuted_adjacent():
    """Scores are dot products, unchanged when q and k get the same channel
    permutation: half-pairing attention on (q, k) equals adjacent-pairing
    attention on the permuted (q, k), and the pairings differ in general."""
    q, k, v = _tiny(12, 1, 24, 4, 2, 16, "fp32")
    cu = np.array([0, 9, 24])
    Oh, Lh = orc.rope_attention(q, k, v, cu, 500000.0, pairing="half")
    Oa, La = orc.rope_attention(_to_adjacent(q.numpy()), _to_adjacent(k.numpy()), v, cu, 500000.0)
    np.testing.assert_allclose(Oh, Oa, rtol=0, atol=1e-12)
    np.testing.assert_allclose(Lh, La, rtol=0, atol=1e-12)
    Ox, _ = orc.rope_attention(q, k, v, cu, 500000.0)
    assert np.abs(Ox - Oh).max() > 1e-3


def test_rope_frequency_closed_forms():
    for D in (64, 128):
        th = orc.rope_frequencies(D, 500000.0)
        assert th.shape == (D // 2,)
        assert th[0] == 1.0
        assert th[D // 4] == pytest.approx(1.0 / math.sqrt(500000.0), rel=1e-15)
        ratios = th[1:] / th[:-1]                                # geometric progression
        np.testing.assert_allclose(ratios, 500000.0 ** (-2.0 / D), rtol=1e-14)
        # slowest band, against the same power written as exp(-(D-2)/D * ln base)
        assert th[-1] == pytest.approx(math.exp(-(D - 2) / D * math.log(500000.0)), rel=1e-14)


# -------------------------------------------------------------- closed forms

def test_zero_query_gives_mean_of_visible_values_and_log_count():
    S = 30
    _, k, v = _tiny(10, 1, S, 4, 2, 8, "bf16")
    q = torch.zeros(1, S, 4, 8)
    cu = np.array([0, 7, 8, 30], dtype=np.int32)
    O, L = orc.rope_attention(q, k, v, cu)
    vv = v.double().numpy()
    for i in range(S):
        a = cu[np.searchsorted(cu, i, side="right") - 1]
        n = i - a + 1
        for h in range(4):
            np.testing.assert_allclose(O[0, i, h], vv[0, a:i + 1, h // 2].mean(axis=0), atol=1e-14)
            assert L[0, h, i] == pytest.approx(math.log(n), abs=1e-14)


def test_first_token_of_each_document_returns_its_value_row():
    q, k, v = _tiny(11, 1, 40, 8, 2, 16, "bf16")
    cu = np.array([0, 5, 6, 23, 40], dtype=np.int32)
    O, _ = orc.rope_attention(q, k, v, cu)
    for a in cu[:-1]:
        for h in range(8):
            assert np.array_equal(O[0, a, h], v[0, a, h // 4].double().numpy())


def test_constant_values_give_constant_output():
    q, k, _ = _tiny(12, 1, 25, 4, 1, 8, "bf16")
    v = torch.full((1, 25, 1, 8), 0.375)
    O, _ = orc.rope_attention(q, k, v, np.array([0, 12, 25]))
    np.testing.assert_allclose(O, 0.375, rtol=0, atol=1e-15)


def test_two_key_document_is_a_logistic_mix():
    """Row 1 of a 2-token document: O = (v0 + e^{s1-s0} v1) / (1 + e^{s1-s0})."""
    D = 2
    q = torch.tensor([[[[0.3, -0.2]], [[0.7, 0.4]]]], dtype=torch.float64)
    k = torch.tensor([[[[1.1, 0.5]], [[-0.6, 0.9]]]], dtype=torch.float64)
    v = torch.tensor([[[[2.0, -1.0]], [[0.5, 3.0]]]], dtype=torch.float64)
    O, L = orc.rope_attention(q, k, v, None, 500000.0)
    # D = 2: one band, theta_0 = 1; position 0 unrotated, position 1 rotated by 1 rad
    c, s = math.cos(1.0), math.sin(1.0)
    q1 = (0.7 * c - 0.4 * s, 0.7 * s + 0.4 * c)
    k1 = (-0.6 * c - 0.9 * s, -0.6 * s + 0.9 * c)
    s0 = (q1[0] * 1.1 + q1[1] * 0.5) / math.sqrt(D)
    s1 = (q1[0] * k1[0] + q1[1] * k1[1]) / math.sqrt(D)
    w = 1.0 / (1.0 + math.exp(s0 - s1))                          # weight of key 1
    np.testing.assert_allclose(O[0, 1, 0], [(1 - w) * 2.0 + w * 0.5, (1 - w) * -1.0 + w * 3.0],
                               atol=1e-15)
    assert L[0, 0, 1] == pytest.approx(math.log(math.exp(s0) + math.exp(s1)), abs=1e-14)


# -------------------------------------------------------------------- decode

def _decode_case(seed, B=3, Hq=8, Hkv=2, D=16, lens=(5, 17, 40)):
    gen = torch.Generator().manual_seed(seed)
    lens = np.array(lens, dtype=np.int32)
    k_raw = [torch.randn(Hkv, L, D, generator=gen).bfloat16() for L in lens]
    v = [torch.randn(Hkv, L, D, generator=gen).bfloat16() for L in lens]
    q_raw = torch.randn(B, Hq, D, generator=gen).bfloat16()
    return q_raw, k_raw, v, lens


def test_decode_equals_last_row_of_prefill():
    q_raw, k_raw, v, lens = _decode_case(13)
    B, Hq, D = q_raw.shape
    k_rot = [orc.rope(kb.transpose(0, 1)[None], np.arange(kb.shape[1])[None])[0].transpose(1, 0, 2)
             for kb in k_raw]
    q_rot = np.stack([orc.rope(q_raw[b][None, None], np.array([[lens[b] - 1]]))[0, 0] for b in range(B)])
    O, L = orc.decode(q_rot, k_rot, v, lens)
    for b in range(B):
        n = int(lens[b])
        # a prefill of n tokens whose last query is the new token
        qp = torch.zeros(1, n, Hq, D, dtype=torch.float64)
        qp[0, -1] = q_raw[b].double()
        kp = k_raw[b].transpose(0, 1)[None].double()
        vp = v[b].transpose(0, 1)[None].double()
        Op, Lp = orc.rope_attention(qp, kp, vp, None, 500000.0, rows=[n - 1])
        np.testing.assert_allclose(O[b], Op[0, 0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(L[b], Lp[0, :, 0], rtol=0, atol=1e-12)


@pytest.mark.parametrize("chunk,max_splits", [(1, 40), (4, 12), (7, 6), (16, 8), (40, 1), (64, 3)])
def test_split_partials_combine_to_unsplit_result(chunk, max_splits):
    q_raw, k_raw, v, lens = _decode_case(14)
    q = q_raw.double().numpy()
    O, L = orc.decode(q, k_raw, v, lens)
    op, lp = orc.decode_partials(q, k_raw, v, lens, chunk, max_splits)
    # empty trailing splits are -inf / 0
    for b, n in enumerate(lens):
        used = -(-int(n) // chunk)
        assert np.all(np.isneginf(lp[b, :, used:])) and np.all(op[b, :, used:] == 0)
        assert np.all(np.isfinite(lp[b, :, :used]))
    Oc, Lc = orc.combine(op, lp)
    np.testing.assert_allclose(Oc, O, rtol=0, atol=1e-12)
    np.testing.assert_allclose(Lc, L, rtol=0, atol=1e-12)


def test_single_split_partial_equals_decode():
    q_raw, k_raw, v, lens = _decode_case(15)
    q = q_raw.double().numpy()
    O, L = orc.decode(q, k_raw, v, lens)
    op, lp = orc.decode_partials(q, k_raw, v, lens, 64, 1)
    np.testing.assert_allclose(op[:, :, 0], O, atol=1e-13)
    np.testing.assert_allclose(lp[:, :, 0], L, atol=1e-13)
