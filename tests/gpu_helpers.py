"""Shared plumbing of the GPU parity tests: run the HIP path through the
binding and compare with the oracle. Tolerances are the ones the parity bar
states: max-abs 2e-2 and mean-abs 2e-3 on outputs from bf16 inputs."""

from __future__ import annotations

import sys

import numpy as np
import torch

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
LSE_MAX_ABS = 2e-2


def say(*args):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print("[case]", *args, flush=True)
    sys.stdout.flush()


def run_prefill(q, k, v, cu_docs=None, positions=None, rope_base=500000.0, with_lse=True,
                softmax_scale=0.0):
    """rope_qk then gqa_prefill on the GPU; returns (O, LSE, q_rot, k_rot) on the CPU."""
    import gqa_attention_rope_02_amd as la
    dev = torch.device("cuda")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    B, S, Hq, D = q.shape
    qr = torch.full_like(qd, float("nan"))
    kr = torch.full_like(kd, float("nan"))
    pos = None if positions is None else torch.as_tensor(np.asarray(positions), dtype=torch.int32).to(dev)
    la.rope_qk(qd, qr, kd, kr, positions=pos, rope_base=rope_base)
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, Hq, S), float("nan"), dtype=torch.float32, device=dev) if with_lse else None
    cu = None
    if cu_docs is not None:
        cu = torch.as_tensor(np.asarray(cu_docs), dtype=torch.int32).reshape(B, -1).to(dev)
    la.gqa_prefill(qr, kr, vd, o, lse, cu, softmax_scale)
    torch.cuda.synchronize()
    return o.cpu(), (lse.cpu() if with_lse else None), qr.cpu(), kr.cpu()


def errors(got, want):
    d = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(want, dtype=np.float64))
    return float(d.max()), float(d.mean())


def assert_close(got, want, max_abs=MAX_ABS, mean_abs=MEAN_ABS, what="O"):
    got = got.double().numpy() if isinstance(got, torch.Tensor) else np.asarray(got)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    mx, mn = errors(got, want)
    assert mx <= max_abs and mn <= mean_abs, f"{what}: max-abs {mx:.3e} mean-abs {mn:.3e}"
    return mx, mn


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    a = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def fp32_ulp(x):
    a = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 23)


def check_partials(op, lp, q_rot, k_rot, vs, lens, chunk):
    """The workspace holds runs of consecutive splits: a finite lse at slot s
    starts a run that ends at the next finite slot (or at the last split); its
    o and lse are those of all keys of the run, i.e. the oracle's per-split
    partials merged over the run. Slot 0 always starts a run, and slots past
    the last split are never written (they keep the NaN fill)."""
    from oracle import reference as orc
    op, lp = np.asarray(op), np.asarray(lp)
    max_splits = op.shape[2]
    opw, lpw = orc.decode_partials(q_rot, k_rot, vs, lens, chunk, max_splits)
    got_o, got_l, want_o, want_l = [], [], [], []
    n_runs = 0
    for b, L in enumerate(lens):
        n = -(-int(L) // chunk)
        assert np.isnan(lp[b, :, n:]).all() and np.isnan(op[b, :, n:]).all()
        for h in range(lp.shape[1]):
            live = np.flatnonzero(np.isfinite(lp[b, h, :n]))
            assert live.size and live[0] == 0
            assert np.isneginf(np.delete(lp[b, h, :n], live)).all()
            ends = list(live[1:]) + [n]
            for s, t in zip(live, ends):
                mo, ml = orc.combine(opw[b, h, s:t], lpw[b, h, s:t])
                got_o.append(op[b, h, s])
                got_l.append(lp[b, h, s])
                want_o.append(mo)
                want_l.append(ml)
                n_runs += 1
    assert_close(np.array(got_o), np.array(want_o), what="o_part runs")
    assert_close(np.array(got_l), np.array(want_l), LSE_MAX_ABS, LSE_MAX_ABS, "lse_part runs")
    return n_runs
