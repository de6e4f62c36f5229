"""Planted slips in the oracle (on the CPU) must each fail at least one pin.

Each mutation swaps one function of ``oracle.reference`` for a plausibly wrong
variant; the pin tests of ``test_oracle_pins`` are then run against it and at
least one must raise. This shows the pins are tight enough to catch the slips
they are meant for.
"""

import math

import numpy as np
import pytest

import oracle.reference as orc
import test_oracle_pins as pins

_real_attention = orc.attention
_real_rope = orc.rope
_real_freq = orc.rope_frequencies


def _attention_variant(kv_map=None, strict=False, leak=False, scale_one=False, lse_no_max=False):
    """A copy of the oracle's attention with one deliberate slip switched on."""
    def attention(qr, kr, v, cu_docs=None, scale=None, rows=None, block=256):
        qr, kr, v = orc._f64(qr), orc._f64(kr), orc._f64(v)
        B, S, Hq, D = qr.shape
        Hkv = kr.shape[2]
        g = Hq // Hkv
        sc = 1.0 if scale_one else (1.0 / math.sqrt(D) if scale is None else scale)
        cu = np.asarray([0, S] if cu_docs is None else cu_docs)
        doc = np.zeros(S, dtype=np.int64) if leak else orc.document_of(cu, S)
        rows = np.arange(S) if rows is None else np.asarray(rows)
        O = np.zeros((B, rows.size, Hq, D))
        L = np.zeros((B, Hq, rows.size))
        j = np.arange(S)
        for b in range(B):
            for n, i in enumerate(rows):
                vis = ((j < i) if strict else (j <= i)) & (doc == doc[i])
                for h in range(Hq):
                    kv = kv_map(h, g, Hkv) if kv_map else h // g
                    s = np.where(vis, kr[b, :, kv] @ qr[b, i, h] * sc, -np.inf)
                    m = s.max()
                    e = np.exp(s - m)
                    O[b, n, h] = e @ v[b, :, kv] / e.sum()
                    L[b, h, n] = (0.0 if lse_no_max else m) + np.log(e.sum())
        return O, L
    return attention


def _rope_half_split(x, positions, base=500000.0, pairing="adjacent"):
    x = orc._f64(x)
    D = x.shape[-1]
    ang = np.asarray(positions, dtype=np.float64)[..., None] * orc.rope_frequencies(D, base)
    c, s = np.cos(ang)[..., None, :], np.sin(ang)[..., None, :]
    a, b = x[..., :D // 2], x[..., D // 2:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def _rope_wrong_sign(x, positions, base=500000.0, pairing="adjacent"):
    return _real_rope(x, -np.asarray(positions), base, pairing)


def _rope_half_backwards(x, positions, base=500000.0, pairing="adjacent"):
    p = -np.asarray(positions) if pairing == "half" else positions
    return _real_rope(x, p, base, pairing)


def _rope_half_is_adjacent(x, positions, base=500000.0, pairing="adjacent"):
    return _real_rope(x, positions, base, "adjacent")


def _backward_variant(no_row_term=False, overwrite_heads=False, dq_unscaled=False, dk_from_keys=False):
    """A copy of the oracle's attention_backward with one slip switched on."""
    def attention_backward(qr, kr, v, dO, cu_docs=None, scale=None):
        qr, kr, v, dO = (orc._f64(x) for x in (qr, kr, v, dO))
        B, S, Hq, D = qr.shape
        g = Hq // kr.shape[2]
        sc = 1.0 / math.sqrt(D) if scale is None else scale
        cu = np.asarray([0, S] if cu_docs is None else cu_docs)
        doc = orc.document_of(cu, S)
        i = np.arange(S)
        vis = (i[None, :] <= i[:, None]) & (doc[None, :] == doc[:, None])
        dq, dk, dv = np.zeros_like(qr), np.zeros_like(kr), np.zeros_like(v)
        for b in range(B):
            for h in range(Hq):
                kv = h // g
                s = np.where(vis, qr[b, :, h] @ kr[b, :, kv].T * sc, -np.inf)
                e = np.exp(s - s.max(axis=1, keepdims=True))
                P = e / e.sum(axis=1, keepdims=True)
                dP = dO[b, :, h] @ v[b, :, kv].T
                dS = P * dP if no_row_term else P * (dP - (P * dP).sum(axis=1, keepdims=True))
                if overwrite_heads:
                    dv[b, :, kv] = P.T @ dO[b, :, h]
                    dk[b, :, kv] = sc * dS.T @ qr[b, :, h]
                else:
                    dv[b, :, kv] += P.T @ dO[b, :, h]
                    dk[b, :, kv] += sc * dS.T @ (kr[b, :, kv] if dk_from_keys else qr[b, :, h])
                dq[b, :, h] = (1.0 if dq_unscaled else sc) * dS @ kr[b, :, kv]
        return dq, dk, dv
    return attention_backward


_real_bwd_rows = orc.attention_backward_rows


def _bwd_rows_keys_from_asked_rows(qr, kr, v, dO, rows, keys, cu_docs=None, scale=None, block=64,
                                   magnitudes=False):
    """Slip: dk and dv summed over the asked-for query rows only, not over
    every row that sees the key (the other rows' output gradients dropped)."""
    keep = np.zeros(qr.shape[0], dtype=bool)
    keep[np.asarray(rows)] = True
    dO = np.where(keep[:, None, None], orc._f64(dO), 0.0)
    return _real_bwd_rows(qr, kr, v, dO, rows, keys, cu_docs, scale, block, magnitudes)


def _bwd_rows_no_documents(qr, kr, v, dO, rows, keys, cu_docs=None, scale=None, block=64, magnitudes=False):
    """Slip: the rows' softmax windows start at the sequence start."""
    return _real_bwd_rows(qr, kr, v, dO, rows, keys, None, scale, block, magnitudes)


def _bwd_rows_magnitude_of_sum(qr, kr, v, dO, rows, keys, cu_docs=None, scale=None, block=64,
                               magnitudes=False):
    """Slip: the l1 magnitude taken as |sum of terms| instead of the sum of |terms|."""
    out = _real_bwd_rows(qr, kr, v, dO, rows, keys, cu_docs, scale, block, magnitudes)
    if not magnitudes:
        return out
    return out[:3] + (([np.abs(x) for x in out[:3]], out[3][1]),)


MUTATIONS = {
    "restricted backward: keys fed by the asked rows only": ("attention_backward_rows",
                                                            _bwd_rows_keys_from_asked_rows),
    "restricted backward: no document starts": ("attention_backward_rows", _bwd_rows_no_documents),
    "restricted backward: l1 of the sum": ("attention_backward_rows", _bwd_rows_magnitude_of_sum),
    "backward drops the softmax row term": ("attention_backward", _backward_variant(no_row_term=True)),
    "backward keeps one head per KV head": ("attention_backward", _backward_variant(overwrite_heads=True)),
    "backward dq without the scale": ("attention_backward", _backward_variant(dq_unscaled=True)),
    "backward dk from the keys": ("attention_backward", _backward_variant(dk_from_keys=True)),
    "kv head h % Hkv": ("attention", _attention_variant(kv_map=lambda h, g, Hkv: h % Hkv)),
    "strict causal j < i": ("attention", _attention_variant(strict=True)),
    "mask leaks across documents": ("attention", _attention_variant(leak=True)),
    "softmax scale dropped": ("attention", _attention_variant(scale_one=True)),
    "LSE without the max": ("attention", _attention_variant(lse_no_max=True)),
    "RoPE half-split pairs": ("rope", _rope_half_split),
    "RoPE rotates backwards": ("rope", _rope_wrong_sign),
    "half-split RoPE rotates backwards": ("rope", _rope_half_backwards),
    "half-split RoPE pairs adjacent channels": ("rope", _rope_half_is_adjacent),
    "theta uses k/D": ("rope_frequencies", lambda D, base=500000.0: _real_freq(2 * D, base)),
    "theta uses d_model": ("rope_frequencies", lambda D, base=500000.0: _real_freq(128 * D, base)),
}

PIN_CALLS = [
    lambda: pins.test_brute_force_equals_oracle(0, 13, 4, 2, 8, 3, False),
    lambda: pins.test_brute_force_equals_oracle(3, 11, 6, 2, 8, 4, True),
    lambda: pins.test_sdpa_library_route(4, 40, 8, 2, 16, 3),
    pins.test_gqa_equals_mha_with_repeated_kv,
    pins.test_document_mask_equals_separate_documents,
    pins.test_scores_depend_only_on_offset,
    pins.test_rope_unit_vectors_show_pairing_and_direction,
    pins.test_rope_frequency_closed_forms,
    pins.test_zero_query_gives_mean_of_visible_values_and_log_count,
    pins.test_first_token_of_each_document_returns_its_value_row,
    pins.test_two_key_document_is_a_logistic_mix,
    pins.test_rope_half_pairing_is_adjacent_pairing_under_a_channel_permutation,
    pins.test_rope_half_unit_vector,
    pins.test_attention_with_half_pairing_equals_permuted_adjacent,
    pins.test_backward_matches_finite_differences,
    pins.test_backward_matches_autograd_of_sdpa,
    lambda: pins.test_restricted_backward_equals_full_backward(11, 29, 4, 2, 8, [0, 9, 9, 21, 29]),
    pins.test_restricted_backward_matches_autograd_of_sdpa,
    pins.test_restricted_backward_magnitudes,
]


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_slip_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(orc, attr, fn)
    caught = 0
    for call in PIN_CALLS:
        try:
            call()
        except (AssertionError, ValueError, FloatingPointError):
            caught += 1
    assert caught >= 1, f"no pin catches the slip: {name}"


def test_unmutated_oracle_passes_every_pin_call():
    assert orc.attention is _real_attention
    for call in PIN_CALLS:
        call()
