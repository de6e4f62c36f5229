"""Shared plumbing of the GPU parity tests: run the HIP path through the
binding and compare with the oracle. Tolerances are the ones the parity bar
states: max-abs 2e-2 and mean-abs 2e-3 on outputs from bf16 inputs."""

from __future__ import annotations

import sys

import numpy as np
import torch

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
# LSE: max-abs 2e-2 as for O; mean-abs the same 2e-3 bar (the bf16 rounding of
# the weights inside the row sum bounds |dLSE| by ln(1 + 2^-9) ~ 2e-3 per row in
# the worst case and averages far below it)
LSE_MAX_ABS = 2e-2
LSE_MEAN_ABS = 2e-3


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
    print(f"[err] {what}: max-abs {mx:.3e} mean-abs {mn:.3e}", flush=True)
    assert mx <= max_abs and mn <= mean_abs, f"{what}: max-abs {mx:.3e} mean-abs {mn:.3e}"
    return mx, mn


def assert_lse_close(got, want, what="LSE"):
    """LSE against the oracle at the LSE bar (max-abs 2e-2, mean-abs 2e-3)."""
    return assert_close(got, want, LSE_MAX_ABS, LSE_MEAN_ABS, what)


def oracle_rows_threaded(q, k, v, rows, cu, base, n_threads=16, chunk=64):
    """The fp64 row oracle (oracle.reference.rope_attention_rows) evaluated on
    chunks of the asked-for rows by a pool of threads, each with a
    single-threaded BLAS: NumPy releases the interpreter lock in its matrix
    products and large element-wise passes, so the chunks run in parallel.
    Every row's value is computed by the oracle itself; only the work is
    divided. Returns O [R,Hq,D] and LSE [Hq,R] in the order of rows."""
    import concurrent.futures as cf
    from threadpoolctl import threadpool_limits
    from oracle import reference as orc
    rows = np.asarray(rows, dtype=np.int64)
    parts = [rows[i:i + chunk] for i in range(0, rows.size, chunk)]
    with threadpool_limits(limits=1, user_api="blas"):
        with cf.ThreadPoolExecutor(max_workers=n_threads) as ex:
            res = list(ex.map(lambda r: orc.rope_attention_rows(q, k, v, r, cu, base), parts))
    O = np.concatenate([r[0] for r in res], axis=0)
    L = np.concatenate([r[1] for r in res], axis=1)
    return O, L


# Gradient bar. Each term of a gradient sum (P_ij dO_i for dv, scale dS_ij q_i
# for dk, scale dS_ij k_j for dq) is formed from bf16 inputs and goes through
# at most two bf16 roundings (P or dS rounded for the matrix product, dS
# carrying P's error), each at most 2^-9 relative; the sums run in fp32 and the
# result is rounded once more to bf16 (at most 2^-9 |ref|). The row term of
# dS_ij = P_ij (dP_ij - D_i), D_i = dO_i . O_i, is formed from the forward's
# output, itself rounded: its error is at most about 2^-8 of A_i, the absolute
# sum behind it, and the oracle's magnitudes count it (l1 with A_i, l2 with
# its typical size R_i). Worst case, per element: |err| <= 2^-8 l1 + 2^-9 |ref|;
# the bar allows 2^-7 l1 + 2^-8 |ref| (twice that) plus 1e-6 for fp32 rounding
# of sums that cancel to nearly zero. On average the roundings are
# independent and uniform, so the terms' share of an element's error has
# standard deviation at most 2^-9 sqrt(2/3) of their root-sum-square, mean
# absolute value at most sqrt(2/pi) times that (0.66 2^-9), the row term's
# share is about 2^-9 of its l2 part, and the final rounding adds 2^-10 |ref|
# on average: the mean bar is 2^-8 mean(l2 + |ref|).
GRAD_MAX_L1 = 2.0 ** -7
GRAD_MAX_REF = 2.0 ** -8
GRAD_MAX_FLOOR = 1e-6
GRAD_MEAN = 2.0 ** -8


def assert_grad_bar(got, want, l1, l2, what):
    """A gradient against the oracle's fp64 values at the bar above: every
    element within 2^-7 l1 + 2^-8 |ref| + 1e-6 and mean |err| within
    2^-8 mean(l2 + |ref|)."""
    got = got.double().numpy() if isinstance(got, torch.Tensor) else np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    d = np.abs(got - want)
    lim = GRAD_MAX_L1 * l1 + GRAD_MAX_REF * np.abs(want) + GRAD_MAX_FLOOR
    worst = float((d / lim).max())
    mean_lim = GRAD_MEAN * float(np.mean(l2 + np.abs(want)))
    mn = float(d.mean())
    print(f"[grad] {what}: n {d.size} max|ref| {np.abs(want).max():.3e} max-abs {d.max():.3e} "
          f"worst err/bar {worst:.3e} mean-abs {mn:.3e} (bar {mean_lim:.3e}) "
          f"mean-abs / mean|ref| {mn / max(float(np.abs(want).mean()), 1e-30):.3e}", flush=True)
    assert worst <= 1.0, f"{what}: an element exceeds its bar by {worst:.3f}x"
    assert mn <= mean_lim, f"{what}: mean-abs {mn:.3e} above {mean_lim:.3e}"


def backward_oracle_threaded(q, k, v, dout, rows, keys, cu, n_threads=16, scale=None):
    """oracle.reference.attention_backward_rows (with term magnitudes) for one
    sequence, one KV head group per task: the groups' gradients are
    independent, so each task runs the oracle on its heads' slices (the
    oracle's own arithmetic, only the work divided). Returns dq [R,Hq,D],
    dk [K,Hkv,D], dv [K,Hkv,D] and (l1, l2) as the oracle does."""
    import concurrent.futures as cf
    from threadpoolctl import threadpool_limits
    from oracle import reference as orc
    Hq, Hkv = q.shape[1], k.shape[1]
    g = Hq // Hkv
    blas = max(1, n_threads // Hkv)

    def one(kv):
        h = slice(kv * g, (kv + 1) * g)
        return orc.attention_backward_rows(q[:, h], k[:, kv:kv + 1], v[:, kv:kv + 1], dout[:, h], rows, keys,
                                           cu, scale, magnitudes=True)

    with threadpool_limits(limits=blas, user_api="blas"):
        with cf.ThreadPoolExecutor(max_workers=min(Hkv, n_threads)) as ex:
            res = list(ex.map(one, range(Hkv)))
    cat = lambda i, ax: np.concatenate([r[i] for r in res], axis=ax)            # noqa: E731
    l1 = [np.concatenate([r[3][0][t] for r in res], axis=1) for t in range(3)]
    l2 = [np.concatenate([r[3][1][t] for r in res], axis=1) for t in range(3)]
    return cat(0, 1), cat(1, 1), cat(2, 1), (l1, l2)


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
    assert_lse_close(np.array(got_l), np.array(want_l), "lse_part runs")
    return n_runs
