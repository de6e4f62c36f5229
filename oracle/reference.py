"""Plain fp64 definitions of the attention path (test infrastructure only).

Every input is upcast exactly to fp64 (bf16 and fp32 values are representable)
and every step is the textbook definition, written out:

1. RoPE ("Llama 3.1 Architecture: Dense Scaling to 405B and 128K Context",
   "Context Expansion ... RoPE Frequency Scaling", "1. High Base Frequency",
   the theta_k equation): theta_k = base^(-2k/D) for k = 0 .. D/2-1, d being the
   head dimension because the rotation acts on each head's vector. Each pair of
   channels (2k, 2k+1) of a query or key at position m is rotated by the angle
   m * theta_k. The pairing of adjacent channels follows RoFormer (Su et al.,
   in the same page's references). Values are not rotated.
2. Scores ("The Llama 3 Herd of Models", "A Deliberately Standard Dense
   Transformer"): s_ij = <q_i, k_j> * scale with scale = 1/sqrt(D) unless given;
   query head h reads KV head floor(h / g), g = Hq / Hkv (contiguous groups of
   query heads share a KV head: "How Meta's Llama 3.1 405B Architecture
   Actually Works", GQA paragraph).
3. Mask: key j is visible to query i iff j <= i (decoder-only, causal) and both
   lie in the same document, documents being the contiguous segments
   [cu_docs[d], cu_docs[d+1]) of the packed sequence (the cross-document mask
   of the same "Deliberately Standard Dense Transformer" entry).
4. Exact softmax per row: m_i = max_j s_ij, p_ij = exp(s_ij - m_i) / l_i with
   l_i = sum_j exp(s_ij - m_i); O_i = sum_j p_ij v_j, LSE_i = m_i + ln l_i.
5. Backward (the training step's gradient pass under the same masks): the
   chain rule through steps 2-4 for a given output gradient dO; the pages fix
   the forward only, so the gradients are the plain derivatives of it, pinned
   by finite differences and by a library's automatic differentiation.

Rows are processed in blocks only to bound memory; each row's softmax is
computed in one pass over all of its keys, and keys outside the union of the
block's visible windows (which contribute exactly zero) are not materialised.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np


def _f64(x) -> np.ndarray:
    """Exact upcast to a float64 numpy array (torch tensors or array-likes)."""
    if hasattr(x, "detach"):  # torch.Tensor, without importing torch here
        import torch
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def rope_frequencies(D: int, base: float = 500000.0) -> np.ndarray:
    """theta_k = base^(-2k/D), k = 0 .. D/2-1, in fp64."""
    k = np.arange(D // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * k / np.float64(D))


def rope(x, positions, base: float = 500000.0, pairing: str = "adjacent") -> np.ndarray:
    """Rotate channel pairs of x [..., S, H, D] by positions * theta_k.

    Pair k is channels (2k, 2k+1) ("adjacent", RoFormer's layout, which the
    pages cite) or channels (k, k + D/2) ("half": the pages do not fix the
    layout, and this is the other one in common use); either way the first
    channel of the pair becomes x0 cos - x1 sin and the second x0 sin + x1 cos.
    ``positions`` has the shape of x's leading dims up to S (e.g. [B, S]);
    returns fp64 of x's shape.
    """
    x = _f64(x)
    D = x.shape[-1]
    pos = np.asarray(positions, dtype=np.float64)
    angle = pos[..., None] * rope_frequencies(D, base)        # [..., S, D/2]
    c = np.cos(angle)[..., None, :]                            # broadcast over H
    s = np.sin(angle)[..., None, :]
    if pairing == "adjacent":
        first, second = np.s_[..., 0::2], np.s_[..., 1::2]
    elif pairing == "half":
        first, second = np.s_[..., :D // 2], np.s_[..., D // 2:]
    else:
        raise ValueError(f"unknown pairing {pairing!r}")
    x0, x1 = x[first], x[second]
    out = np.empty_like(x)
    out[first] = x0 * c - x1 * s
    out[second] = x0 * s + x1 * c
    return out


def document_of(cu_docs, S: int) -> np.ndarray:
    """Document index of every token 0..S-1 for offsets cu_docs [n+1]."""
    cu = np.asarray(cu_docs, dtype=np.int64)
    return np.searchsorted(cu, np.arange(S), side="right") - 1


def attention(qr, kr, v, cu_docs=None, scale: Optional[float] = None,
              rows: Optional[Sequence[int]] = None,
              block: int = 256) -> Tuple[np.ndarray, np.ndarray]:
    """Masked GQA softmax attention on already-rotated queries and keys.

    qr [B,S,Hq,D], kr and v [B,S,Hkv,D]. Returns O [B,R,Hq,D] and LSE [B,Hq,R]
    in fp64, R = S or len(rows) (the query rows asked for, in that order).
    """
    qr, kr, v = _f64(qr), _f64(kr), _f64(v)
    B, S, Hq, D = qr.shape
    Hkv = kr.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    cu = np.asarray([0, S] if cu_docs is None else cu_docs, dtype=np.int64)
    doc = document_of(cu, S)
    start = cu[doc]                                            # first key of each row's document
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.size
    O = np.zeros((B, R, Hq, D))
    LSE = np.zeros((B, Hq, R))
    for b in range(B):
        for r0 in range(0, R, block):
            ri = rows[r0:r0 + block]
            lo, hi = int(start[ri].min()), int(ri.max()) + 1   # keys any of these rows may see
            j = np.arange(lo, hi)
            visible = (j[None, :] <= ri[:, None]) & (doc[j][None, :] == doc[ri][:, None])
            for kv in range(Hkv):
                heads = slice(kv * g, (kv + 1) * g)
                q = qr[b, ri, heads, :]                        # [r, g, D]
                n = q.shape[0]
                s = (q.reshape(n * g, D) @ kr[b, lo:hi, kv, :].T).reshape(n, g, hi - lo) * scale
                s = np.where(visible[:, None, :], s, -np.inf)
                m = s.max(axis=2, keepdims=True)               # every row sees itself: finite
                e = np.exp(s - m)
                l = e.sum(axis=2, keepdims=True)
                pv = (e.reshape(n * g, hi - lo) @ v[b, lo:hi, kv, :]).reshape(n, g, D)
                O[b, r0:r0 + n, heads, :] = pv / l
                LSE[b, heads, r0:r0 + n] = (m + np.log(l))[:, :, 0].T
    return O, LSE


def rope_attention(q, k, v, cu_docs=None, base: float = 500000.0, positions=None,
                   scale: Optional[float] = None, rows=None,
                   pairing: str = "adjacent") -> Tuple[np.ndarray, np.ndarray]:
    """The whole prefill path: RoPE on Q and K at ``positions`` (default: the
    token index), then masked GQA attention. Shapes as in ``attention``."""
    q = _f64(q)
    B, S = q.shape[:2]
    if positions is None:
        positions = np.broadcast_to(np.arange(S), (B, S))
    return attention(rope(q, positions, base, pairing), rope(k, positions, base, pairing), v,
                     cu_docs, scale, rows)


def rope_attention_rows(q, k, v, rows, cu_docs=None, base: float = 500000.0,
                        scale: Optional[float] = None, block: int = 64
                        ) -> Tuple[np.ndarray, np.ndarray]:
    """``rope_attention`` of one sequence, restricted to the query rows asked
    for, at sizes where rotating every token in fp64 is out of reach.

    q [S,Hq,D], k and v [S,Hkv,D] (raw, unrotated; any array type), rows the
    token indices to evaluate. Row i sees keys j in [start of its document, i];
    only those keys and the asked-for query rows are rotated (at their token
    index) and converted to fp64, one document at a time. Returns O [R,Hq,D]
    and LSE [Hq,R] for the rows in the order given.
    """
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    cu = np.asarray([0, S] if cu_docs is None else cu_docs, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    doc = document_of(cu, S)
    O = np.zeros((rows.size, Hq, D))
    LSE = np.zeros((Hq, rows.size))
    for d in np.unique(doc[rows]):
        sel = np.flatnonzero(doc[rows] == d)
        lo, hi = int(cu[d]), int(rows[sel].max()) + 1
        kr = rope(k[lo:hi], np.arange(lo, hi), base)            # [W, Hkv, D]
        vw = _f64(v[lo:hi])
        for b0 in range(0, sel.size, block):
            idx = sel[b0:b0 + block]
            ri = rows[idx]
            qr = rope(q[ri], ri, base)                         # [n, Hq, D]
            visible = np.arange(lo, hi)[None, :] <= ri[:, None]
            n = ri.size
            for kv in range(Hkv):
                heads = slice(kv * g, (kv + 1) * g)
                s = (qr[:, heads, :].reshape(n * g, D) @ kr[:, kv, :].T).reshape(n, g, hi - lo) * scale
                s = np.where(visible[:, None, :], s, -np.inf)
                m = s.max(axis=2, keepdims=True)
                e = np.exp(s - m)
                l = e.sum(axis=2, keepdims=True)
                pv = (e.reshape(n * g, hi - lo) @ vw[:, kv, :]).reshape(n, g, D)
                O[idx, heads, :] = pv / l
                LSE[heads, idx] = (m + np.log(l))[:, :, 0].T
    return O, LSE


def _decode_scores(qb, kb, scale):
    # qb [g, D] (the g query heads of one KV head), kb [L, D] -> [g, L]
    return (qb @ kb.T) * scale


def decode(q_rot, k_cache, v_cache, seq_lens, scale: Optional[float] = None
           ) -> Tuple[np.ndarray, np.ndarray]:
    """One new token per sequence attending to its whole cache.

    q_rot [B,Hq,D] is the new token's query, already rotated at position
    L_b - 1; k_cache[b] / v_cache[b] are [Hkv, >= L_b, D] with rotated keys in
    slots 0..L_b-1. Every cached token is visible (causal: all are earlier or
    the token itself). Returns O [B,Hq,D] and LSE [B,Hq].
    """
    q_rot = _f64(q_rot)
    B, Hq, D = q_rot.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    O = np.zeros((B, Hq, D))
    LSE = np.zeros((B, Hq))
    for b in range(B):
        L = int(seq_lens[b])
        kb, vb = _f64(k_cache[b]), _f64(v_cache[b])
        Hkv = kb.shape[0]
        g = Hq // Hkv
        for kv in range(Hkv):
            heads = slice(kv * g, (kv + 1) * g)
            s = _decode_scores(q_rot[b, heads], kb[kv, :L], scale)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            l = e.sum(axis=1, keepdims=True)
            O[b, heads] = (e @ vb[kv, :L]) / l
            LSE[b, heads] = (m + np.log(l))[:, 0]
    return O, LSE


def attention_backward(qr, kr, v, dO, cu_docs=None, scale: Optional[float] = None
                       ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of L = sum(dO * O) for ``attention`` (rotated queries and
    keys, same mask and GQA head mapping): the chain rule through the softmax
    written out. With P the row-softmax of S = qr kr^T * scale over the
    visible keys and O = P v:
      dv_j  = sum_i P_ij dO_i                  (summed over the g query heads
                                                 of the KV head as well)
      dP_ij = dO_i . v_j
      dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)  (the softmax Jacobian)
      dq_i  = scale sum_j dS_ij kr_j
      dkr_j = scale sum_i dS_ij qr_i           (summed over the g heads)
    qr, dO [B,S,Hq,D]; kr, v [B,S,Hkv,D]. Returns (dq, dk, dv) in fp64 with
    the shapes of qr, kr, v; gradients with respect to the unrotated queries
    and keys follow by rotating back (``rope`` at the negated positions).
    """
    qr, kr, v, dO = _f64(qr), _f64(kr), _f64(v), _f64(dO)
    B, S, Hq, D = qr.shape
    Hkv = kr.shape[2]
    g = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    cu = np.asarray([0, S] if cu_docs is None else cu_docs, dtype=np.int64)
    doc = document_of(cu, S)
    i = np.arange(S)
    visible = (i[None, :] <= i[:, None]) & (doc[None, :] == doc[:, None])   # [query, key]
    dq = np.zeros_like(qr)
    dk = np.zeros_like(kr)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            kv = h // g
            s = np.where(visible, qr[b, :, h] @ kr[b, :, kv].T * scale, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            P = e / e.sum(axis=1, keepdims=True)
            dv[b, :, kv] += P.T @ dO[b, :, h]
            dP = dO[b, :, h] @ v[b, :, kv].T
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            dq[b, :, h] = scale * dS @ kr[b, :, kv]
            dk[b, :, kv] += scale * dS.T @ qr[b, :, h]
    return dq, dk, dv


def attention_backward_rows(qr, kr, v, dO, rows, keys, cu_docs=None, scale: Optional[float] = None,
                            block: int = 64, magnitudes: bool = False):
    """``attention_backward`` of one sequence, restricted to the query rows
    whose dq and the keys whose dk, dv are asked for, at sizes where the whole
    gradient in fp64 is out of reach.

    qr, dO [S,Hq,D]; kr, v [S,Hkv,D] (rotated; any array type). dq_i needs only
    row i's own softmax; dk_j and dv_j sum over every query row i >= j of
    j's document, so those rows' softmaxes are formed as well (each over its
    whole visible window, in blocks of ``block`` rows). The terms are those of
    ``attention_backward``, summed over rows (and the g heads of a KV head)
    for dk, dv and over keys for dq:
      dv_j = sum P_ij dO_i,  dk_j = scale sum dS_ij qr_i,  dq_i = scale sum_j dS_ij kr_j.
    Returns dq [R,Hq,D], dk [K,Hkv,D], dv [K,Hkv,D] in the order asked.

    With ``magnitudes``, also (l1, l2), per element of each of the three: the
    scale of what rounding can do to it. l1 is the sum of the absolute values
    of its terms and l2 the root of the sum of their squares, where a dS term
    also carries its row term: D_i = sum_j P_ij dP_ij equals dO_i . O_i, and
    formed from a rounded O it is off by at most a small multiple of
    A_i = sum_d |dO_id| sum_j P_ij |v_jd| (typically of R_i, the root of the
    sum over d of (dO_id sum_j P_ij |v_jd|)^2). So for dq (and likewise dk,
    summed over rows and heads)
      l1 = scale sum_j P_ij (|dP_ij - D_i| + A_i) |kr_jd|,
      l2 = scale sqrt(sum_j dS_ij^2 kr_jd^2) + scale R_i |sum_j P_ij kr_jd|
    (for dk, l2 = scale sqrt(sum_i (dS_ij^2 + P_ij^2 R_i^2) qr_id^2), the
    rows' D errors being independent), and for dv, l1 = sum_i P_ij |dO_id|,
    l2 = sqrt(sum_i P_ij^2 dO_id^2).
    """
    S, Hq, D = qr.shape
    Hkv = kr.shape[1]
    g = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    cu = np.asarray([0, S] if cu_docs is None else cu_docs, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    if np.unique(rows).size != rows.size:
        raise ValueError("rows must be distinct")
    doc = document_of(cu, S)
    dq = np.zeros((rows.size, Hq, D))
    dk = np.zeros((keys.size, Hkv, D))
    dv = np.zeros((keys.size, Hkv, D))
    l1 = [np.zeros_like(dq), np.zeros_like(dk), np.zeros_like(dv)]
    sq = [np.zeros_like(dq), np.zeros_like(dk), np.zeros_like(dv)]
    # rows whose softmax is needed: those asked for, and every row at or after
    # an asked-for key within its document
    need = np.zeros(S, dtype=bool)
    need[rows] = True
    for d in np.unique(doc[keys]):
        need[int(keys[doc[keys] == d].min()):int(cu[d + 1])] = True
    want_row = {int(r): n for n, r in enumerate(rows)}
    for d in np.unique(doc[np.flatnonzero(need)]):
        lo = int(cu[d])
        rows_d = np.flatnonzero(need & (doc == d))
        hi_d = int(rows_d.max()) + 1
        kw, vw = _f64(kr[lo:hi_d]), _f64(v[lo:hi_d])          # [W, Hkv, D]
        kd = np.flatnonzero(doc[keys] == d)                     # output slots of d's keys
        kcol = keys[kd] - lo
        for b0 in range(0, rows_d.size, block):
            ri = rows_d[b0:b0 + block]
            n, W = ri.size, int(ri.max()) + 1 - lo
            qi, gi = _f64(qr[ri]), _f64(dO[ri])                # [n, Hq, D]
            visible = np.arange(lo, lo + W)[None, :] <= ri[:, None]
            asked = [(m, want_row[int(r)]) for m, r in enumerate(ri) if int(r) in want_row]
            am = np.array([m for m, _ in asked], dtype=np.int64)
            ao = np.array([o for _, o in asked], dtype=np.int64)
            kin = kcol < W
            cols, slots = kcol[kin], kd[kin]
            for kv in range(Hkv):
                heads = slice(kv * g, (kv + 1) * g)
                qh = qi[:, heads, :].reshape(n * g, D)
                gh = gi[:, heads, :].reshape(n * g, D)
                s = (qh @ kw[:W, kv, :].T).reshape(n, g, W) * scale
                s = np.where(visible[:, None, :], s, -np.inf)
                e = np.exp(s - s.max(axis=2, keepdims=True))
                P = e / e.sum(axis=2, keepdims=True)
                dP = (gh @ vw[:W, kv, :].T).reshape(n, g, W)
                Dr = (P * dP).sum(axis=2, keepdims=True)
                dS = P * (dP - Dr)
                if magnitudes:
                    pva = (P.reshape(n * g, W) @ np.abs(vw[:W, kv, :]))          # sum_j P_ij |v_jd|
                    A = (np.abs(gh) * pva).sum(axis=1).reshape(n, g, 1)
                    R = np.sqrt(((gh * pva) ** 2).sum(axis=1)).reshape(n, g, 1)
                    M = P * (np.abs(dP - Dr) + A)
                if am.size:
                    t = scale * dS[am].reshape(am.size * g, W)
                    kk = kw[:W, kv, :]
                    dq[ao, heads, :] = (t @ kk).reshape(am.size, g, D)
                    if magnitudes:
                        Pa = P[am].reshape(am.size * g, W)
                        l1[0][ao, heads, :] = (scale * M[am].reshape(am.size * g, W)
                                               @ np.abs(kk)).reshape(am.size, g, D)
                        sq[0][ao, heads, :] = (np.sqrt((t * t) @ (kk * kk)) + scale * R[am].reshape(-1, 1)
                                               * np.abs(Pa @ kk)).reshape(am.size, g, D)
                if cols.size:
                    Pc = P[:, :, cols].reshape(n * g, cols.size).T          # [C, n*g]
                    Sc = scale * dS[:, :, cols].reshape(n * g, cols.size).T
                    np.add.at(dv, (slots, kv), Pc @ gh)
                    np.add.at(dk, (slots, kv), Sc @ qh)
                    if magnitudes:
                        Mc = scale * M[:, :, cols].reshape(n * g, cols.size).T
                        PRc = scale * (P * R)[:, :, cols].reshape(n * g, cols.size).T
                        np.add.at(l1[2], (slots, kv), Pc @ np.abs(gh))
                        np.add.at(l1[1], (slots, kv), Mc @ np.abs(qh))
                        np.add.at(sq[2], (slots, kv), (Pc * Pc) @ (gh * gh))
                        np.add.at(sq[1], (slots, kv), (Sc * Sc + PRc * PRc) @ (qh * qh))
    if magnitudes:
        # dq's l2 is formed whole per element above; dk's and dv's from sums of squares
        return dq, dk, dv, (l1, [sq[0], np.sqrt(sq[1]), np.sqrt(sq[2])])
    return dq, dk, dv


def decode_partials(q_rot, k_cache, v_cache, seq_lens, kv_chunk: int, max_splits: int,
                    scale: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of each new token restricted to each chunk of its cache.

    Split s of sequence b covers keys [s*kv_chunk, min((s+1)*kv_chunk, L_b)).
    o_part [B,Hq,max_splits,D] is the softmax-weighted mean of V over the
    split's keys and lse_part [B,Hq,max_splits] the log of the split's sum of
    exp(scores). A split with no keys has o = 0 and lse = -inf.
    """
    q_rot = _f64(q_rot)
    B, Hq, D = q_rot.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    o_part = np.zeros((B, Hq, max_splits, D))
    lse_part = np.full((B, Hq, max_splits), -np.inf)
    for b in range(B):
        L = int(seq_lens[b])
        kb, vb = _f64(k_cache[b]), _f64(v_cache[b])
        Hkv = kb.shape[0]
        g = Hq // Hkv
        for s_i in range(max_splits):
            a, e_ = s_i * kv_chunk, min((s_i + 1) * kv_chunk, L)
            if a >= e_:
                continue
            for kv in range(Hkv):
                heads = slice(kv * g, (kv + 1) * g)
                s = _decode_scores(q_rot[b, heads], kb[kv, a:e_], scale)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                l = e.sum(axis=1, keepdims=True)
                o_part[b, heads, s_i] = (e @ vb[kv, a:e_]) / l
                lse_part[b, heads, s_i] = (m + np.log(l))[:, 0]
    return o_part, lse_part


def combine(o_part, lse_part) -> Tuple[np.ndarray, np.ndarray]:
    """Merge per-split results by their log-sum-exp weights.

    With M = max_s lse_s and w_s = exp(lse_s - M) (w_s = 0 where lse_s = -inf),
    O = sum_s w_s o_s / sum_s w_s and LSE = M + ln sum_s w_s. Inputs
    [..., n_splits, D] and [..., n_splits]; at least one split must be finite.
    """
    o_part, lse_part = _f64(o_part), _f64(lse_part)
    M = lse_part.max(axis=-1, keepdims=True)
    w = np.exp(lse_part - M)                                   # exp(-inf) = 0
    W = w.sum(axis=-1, keepdims=True)
    O = (w[..., None] * o_part).sum(axis=-2) / W
    return O, (M + np.log(W))[..., 0]
