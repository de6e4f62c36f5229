"""Throughput of the GQA + RoPE attention path on one MI355X.

One step = one pass of the prefill path (rope_qk on the keys, then
gqa_prefill_rope, which rotates the queries in the kernel and applies the
causal + cross-document mask, writing O and the log-sum-exp) over one batch of
seeded synthetic input of the Llama-3.1-8B layer shape (S=8192, 32 query heads
on 8 KV heads, head_dim 128, bf16, 1-8 documents). Inputs are resident in HBM
before the timed region starts.

The JSON line also carries the 8B-shape chunked prefill (the last 2048 tokens
over a cached prefix of 6144), the 405B-shape prefill (S=32768, 128/8 heads)
and the 405B-shape split-KV decode (16 sequences, cache lengths
U[4096, 131072], measured as cache-read GB/s), each against its own roofline,
plus the fp64 oracle timed on a bounded row sample of the headline workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--only prefill|decode] [--with-128k]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "GQA prefill TFLOP/s (% MFMA peak) + decode KV-read GB/s (% HBM peak), 1 GPU"
KV_CHUNK = 256


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def allowed_pairs(cu_docs: np.ndarray) -> int:
    """Visible (query, key) pairs of one sequence under causal + document mask."""
    n = np.diff(np.asarray(cu_docs, dtype=np.int64))
    return int(np.sum(n * (n + 1) // 2))


def kernel_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gqa_attention_rope_02_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str, src_hash: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None
    e = table.get(f"{kernel}/{workload}")
    if not e or e.get("source_hash") != src_hash:
        return None
    return e.get("bytes_per_launch")


# --------------------------------------------------------------------- prefill

def setup_prefill(name: str):
    import torch
    from workloads import CONFIGS, draw_cu_docs, draw_prefill_inputs
    w = CONFIGS[name]
    t = time.time()
    q, k, v = draw_prefill_inputs(w.B, w.S, w.Hq, w.Hkv, w.D, w.dtype, w.seed)
    cu = draw_cu_docs(w.S, w.seed, w.n_docs, w.n_docs_max)
    dev = torch.device("cuda")
    st = dict(w=w, cu=cu, q=q.to(dev), k=k.to(dev), v=v.to(dev),
              cu_d=torch.as_tensor(cu, dtype=torch.int32).reshape(1, -1).to(dev))
    st["qr"] = torch.empty_like(st["q"])
    st["kr"] = torch.empty_like(st["k"])
    st["o"] = torch.empty_like(st["q"])
    st["lse"] = torch.empty(w.B, w.Hq, w.S, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"{name}: inputs ready in {time.time() - t:.1f}s, documents {np.diff(cu).tolist()}")
    return st, (q, k, v)


def settle(step, seconds: float):
    """Run whole steps, untimed, for `seconds` of wall time before the warmup
    steps: the GPU's clocks ramp up over the first tens of milliseconds of
    sustained load, and a step of a quarter millisecond would otherwise be
    timed partly at the idle clock."""
    import torch
    t = time.perf_counter()
    n = 0
    while time.perf_counter() - t < seconds:
        step()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def time_prefill(st, steps: int, warmup: int, settle_s: float = 0.0):
    import torch
    import gqa_attention_rope_02_amd as la

    def step(evs=None):
        if evs:
            evs[0].record()
        la.rope_qk(None, None, st["k"], st["kr"])          # keys; the queries rotate in the kernel
        if evs:
            evs[1].record()
        la.gqa_prefill_rope(st["q"], st["kr"], st["v"], st["o"], st["lse"], st["cu_d"])
        if evs:
            evs[2].record()

    settle(step, settle_s)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    rope_ms = [e[0].elapsed_time(e[1]) for e in evs]
    attn_ms = [e[1].elapsed_time(e[2]) for e in evs]
    gpu_ms = [e[0].elapsed_time(e[2]) for e in evs]
    return dict(wall_ms_per_step=1e3 * wall / steps, rope_ms=float(np.mean(rope_ms)),
                prefill_ms=float(np.mean(attn_ms)), gpu_ms_per_step=float(np.mean(gpu_ms)),
                prefill_ms_median=float(np.median(attn_ms)))


def time_backward(st, steps: int, warmup: int, settle_s: float = 0.0):
    """gqa_attention_backward on the workload (rotated q and k, the forward's o
    and lse computed once beforehand, seeded N(0,1) output gradient)."""
    import torch
    import gqa_attention_rope_02_amd as la
    from workloads import draw_grad_output
    w = st["w"]
    la.rope_qk(st["q"], st["qr"], st["k"], st["kr"])
    la.gqa_prefill(st["qr"], st["kr"], st["v"], st["o"], st["lse"], st["cu_d"])
    dout = draw_grad_output(w.B, w.S, w.Hq, w.D, w.dtype, w.seed).to(st["q"].device)
    dq, dk, dv = torch.empty_like(st["q"]), torch.empty_like(st["k"]), torch.empty_like(st["v"])
    delta = torch.empty_like(st["lse"])

    def step():
        la.gqa_attention_backward(st["qr"], st["kr"], st["v"], st["o"], dout, st["lse"], dq, dk, dv,
                                  delta, st["cu_d"])

    settle(step, settle_s)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record()
        step()
        evs[i][1].record()
    torch.cuda.synchronize()
    ms = [e[0].elapsed_time(e[1]) for e in evs]
    return dict(backward_ms=float(np.mean(ms)), backward_ms_median=float(np.median(ms)))


def prefill_flops(w, cu) -> float:
    return 4.0 * w.D * w.Hq * w.B * allowed_pairs(cu)


def chunk_pairs(cu_docs: np.ndarray, S: int, Sq: int) -> int:
    """Visible (query, key) pairs of the last Sq query rows of a sequence."""
    cu = np.asarray(cu_docs, dtype=np.int64)
    rows = np.arange(S - Sq, S)
    start = cu[np.searchsorted(cu, rows, side="right") - 1]
    return int(np.sum(rows - start + 1))


CHUNK_SPLIT_TILES = 24   # key tiles per piece for the chunked prefill (gqa_prefill_split)


def time_chunk(st, Sq: int, steps: int, warmup: int, settle_s: float = 0.0, split_tiles: int = 0):
    """Chunked prefill of the last Sq tokens over the cached prefix: rope_qk on
    the block's keys (at their positions), then gqa_prefill_chunk with the
    block's queries rotated in the kernel (or gqa_prefill_split with key ranges
    cut into pieces of split_tiles tiles, its workspace allocated beforehand)."""
    import torch
    import gqa_attention_rope_02_amd as la
    w = st["w"]
    S = w.S
    dev = st["q"].device
    qb = st["q"][:, S - Sq:]
    kb_in, kb_out = st["k"][:, S - Sq:], st["kr"][:, S - Sq:]
    pos = torch.arange(S - Sq, S, dtype=torch.int32, device=dev).reshape(1, Sq).expand(w.B, Sq).contiguous()
    ob = torch.empty_like(qb)
    lse = torch.empty(w.B, w.Hq, Sq, dtype=torch.float32, device=dev)
    la.rope_qk(None, None, st["k"], st["kr"])               # the cached prefix (and block), once
    if split_tiles:
        op, lp = la.prefill_split_workspace(w.B, Sq, S, w.Hq, w.D, split_tiles, dev)

    def step(evs=None):
        if evs:
            evs[0].record()
        la.rope_qk(None, None, kb_in, kb_out, positions=pos)
        if evs:
            evs[1].record()
        if split_tiles:
            la.gqa_prefill_split(qb, st["kr"], st["v"], ob, split_tiles, op, lp, lse, st["cu_d"],
                                 rope_base=w.rope_base)
        else:
            la.gqa_prefill_chunk(qb, st["kr"], st["v"], ob, lse, st["cu_d"], rope_base=w.rope_base)
        if evs:
            evs[2].record()

    settle(step, settle_s)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    return dict(rope_ms=float(np.mean([e[0].elapsed_time(e[1]) for e in evs])),
                chunk_ms=float(np.mean([e[1].elapsed_time(e[2]) for e in evs])),
                gpu_ms_per_step=float(np.mean([e[0].elapsed_time(e[2]) for e in evs])))


def time_ring(st, P: int, reps: int):
    """Context-parallel attention as P devices of a ring would run it, all on
    this GPU: the sequence in P equal shards; every query shard against every
    key shard (its own first, then the ring order), partials merged into fp32
    accumulators, then finalized. Queries rotated in the kernel, keys rotated
    once beforehand (outside the timed region). Returns ms per whole ring."""
    import torch
    import gqa_attention_rope_02_amd as la
    w = st["w"]
    S, dev = w.S, st["q"].device
    L = S // P
    la.rope_qk(None, None, st["k"], st["kr"])
    oa = torch.empty(w.B, L, w.Hq, w.D, dtype=torch.float32, device=dev)
    lsa = torch.empty(w.B, w.Hq, L, dtype=torch.float32, device=dev)
    lse_blk = torch.empty(w.B, w.Hq, L, dtype=torch.float32, device=dev)

    def ring():
        for i in range(P):
            q0 = i * L
            for step in range(P):
                j = (i - step) % P
                la.gqa_prefill_ring_step(st["q"][:, q0:q0 + L], st["kr"][:, j * L:(j + 1) * L],
                                         st["v"][:, j * L:(j + 1) * L], q0, j * L, oa, lsa,
                                         first=(step == 0), cu_docs=st["cu_d"], rope_base=w.rope_base)
            la.gqa_prefill_ring_finalize(oa, lsa, st["o"][:, q0:q0 + L], lse_blk)

    ring()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        ring()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


# ---------------------------------------------------------------------- decode

def setup_decode():
    import torch
    from workloads import CONFIGS, draw_seq_lens
    w = CONFIGS["decode405b"]
    lens = draw_seq_lens(w.B, w.len_lo, w.len_hi, w.seed)
    Lmax = w.len_hi
    dev = torch.device("cuda")
    t = time.time()
    g = torch.Generator(device=dev).manual_seed(w.seed)
    kc = torch.empty(w.B, w.Hkv, Lmax, w.D, dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    for b in range(w.B):     # random cache contents (keys as if already rotated)
        kc[b].normal_(generator=g)
        vc[b].normal_(generator=g)
    q = torch.randn(w.B, w.Hq, w.D, generator=g, device=dev).bfloat16()
    max_splits = -(-Lmax // KV_CHUNK)
    st = dict(w=w, lens=lens, q=q, kc=kc, vc=vc, Lmax=Lmax, max_splits=max_splits,
              sl=torch.as_tensor(lens, dtype=torch.int32).to(dev),
              op=torch.empty(w.B, w.Hq, max_splits, w.D, dtype=torch.float32, device=dev),
              lp=torch.empty(w.B, w.Hq, max_splits, dtype=torch.float32, device=dev),
              o=torch.empty(w.B, w.Hq, w.D, dtype=torch.bfloat16, device=dev))
    torch.cuda.synchronize()
    log(f"decode405b: cache ready in {time.time() - t:.1f}s, lengths {lens.tolist()}")
    return st


PAGE_SIZE = 64


def page_decode_cache(st):
    """The decode workload's caches as a pool of PAGE_SIZE-slot pages, each
    page head-major ([n_pages, Hkv, PAGE_SIZE, D] in memory, passed as the
    [n_pages, PAGE_SIZE, Hkv, D] view the call takes), in a seeded random
    order, one block table row per sequence; the contiguous caches are freed."""
    import torch
    w, lens, dev = st["w"], st["lens"], st["q"].device
    need = [-(-int(L) // PAGE_SIZE) for L in lens]
    n_pages = int(sum(need))
    order = np.random.default_rng(w.seed).permutation(n_pages)
    table = np.zeros((w.B, -(-st["Lmax"] // PAGE_SIZE)), dtype=np.int32)
    n = 0
    for b in range(w.B):
        table[b, :need[b]] = order[n:n + need[b]]
        n += need[b]
    del st["kc"], st["vc"]
    torch.cuda.empty_cache()
    g = torch.Generator(device=dev).manual_seed(w.seed + 1)
    kp = torch.empty(n_pages, w.Hkv, PAGE_SIZE, w.D, dtype=torch.bfloat16, device=dev).normal_(generator=g)
    vp = torch.empty_like(kp).normal_(generator=g)
    st["kp"], st["vp"] = kp.permute(0, 2, 1, 3), vp.permute(0, 2, 1, 3)
    st["table"] = torch.as_tensor(table).to(dev)
    torch.cuda.synchronize()


def time_decode(st, steps: int, warmup: int, settle_s: float = 0.0, paged: bool = False):
    import torch
    import gqa_attention_rope_02_amd as la

    def step(evs=None):
        if evs:
            evs[0].record()
        if paged:
            la.gqa_decode_paged(st["q"], st["kp"], st["vp"], st["table"], st["sl"], KV_CHUNK, st["op"],
                                st["lp"], st["Lmax"])
        else:
            la.gqa_decode(st["q"], st["kc"], st["vc"], st["sl"], KV_CHUNK, st["op"], st["lp"])
        if evs:
            evs[1].record()
        la.gqa_decode_combine(st["op"], st["lp"], st["sl"], KV_CHUNK, st["o"])
        if evs:
            evs[2].record()

    settle(step, settle_s)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    dec = [e[0].elapsed_time(e[1]) for e in evs]
    comb = [e[1].elapsed_time(e[2]) for e in evs]
    tot = [e[0].elapsed_time(e[2]) for e in evs]
    return dict(decode_ms=float(np.mean(dec)), combine_ms=float(np.mean(comb)),
                ms_per_step=float(np.mean(tot)), decode_ms_median=float(np.median(dec)))


def decode_bytes(st) -> float:
    w = st["w"]
    return float(np.sum(st["lens"].astype(np.int64))) * w.Hkv * w.D * 2 * 2


# ------------------------------------------------------------ counter scale

COPY_BYTES = 1 << 30


def copy_calibration(reps: int = 3):
    """A plain elementwise device copy of COPY_BYTES (read once, written once):
    what FETCH_SIZE and WRITE_SIZE read for it is the scale that turns those
    counters into HBM bytes for the attention kernels of the same run."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.mul(src, 1.0, out=dst)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"kernel": "elementwise mul by 1.0 (plain copy)", "bytes_read": COPY_BYTES,
            "bytes_written": COPY_BYTES, "ms": round(ms, 4),
            "gbs": round(2 * COPY_BYTES / (ms * 1e-3) / 1e9, 1)}


# ----------------------------------------------------------------- cpu oracle

def cpu_baseline(host_inputs, w, cu, budget_s: float = 20.0):
    """The fp64 oracle on a row sample of the same workload, as TFLOP/s."""
    from oracle import reference as orc
    from workloads import sample_rows
    q, k, v = host_inputs
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    rows_all = sample_rows(w.S, cu, w.seed, n_random=4096, tile=64, n_edges=0)
    rng = np.random.default_rng(w.seed + 7)
    rows_all = rng.permutation(rows_all)
    doc = orc.document_of(cu, w.S)
    start = np.asarray(cu)[doc]
    done, flops, t_used = 0, 0.0, 0.0
    t0 = time.perf_counter()
    chunk = 256
    while done < rows_all.size and t_used < budget_s:
        rows = np.sort(rows_all[done:done + chunk])
        orc.rope_attention(q, k, v, cu, w.rope_base, None, None, rows)
        done += rows.size
        flops += 4.0 * w.D * w.Hq * float(np.sum(rows - start[rows] + 1))
        t_used = time.perf_counter() - t0
    return dict(value=flops / t_used / 1e12, unit="TFLOP/s", cores=int(cores), kind="oracle",
                sample=f"{done} query rows x all {w.Hq} heads of the {w.name} prefill "
                       f"(fp64 NumPy oracle incl. RoPE), {t_used:.1f}s")


# ------------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of untimed whole steps before the warmup steps (GPU clock ramp)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "llama8b", "llama405b", "decode405b", "copy", "backward"],
                    default=None, help="run one part: both prefills, the decode, one workload, "
                                       "or only the copy used to scale HBM counters")
    ap.add_argument("--with-128k", action="store_true", help="also time the S=131072 prefill")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain device copy of known size (scale for FETCH/WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the attention path here runs unsharded on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import gqa_attention_rope_02_amd  # noqa: F401  (fails loudly without the HIP library)

    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "settle_s": args.settle,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1) Q/K/V, seeded document cuts)"}
    phash = kernel_hash("gqa_prefill.hip")
    run_8b = args.only in (None, "prefill", "llama8b")
    run_405 = args.only in (None, "prefill", "llama405b")
    run_dec = args.only in (None, "decode", "decode405b")

    if args.calibrate_copy or args.only == "copy":
        out["copy_calibration"] = copy_calibration()
        if args.only == "copy":
            out.update(value=out["copy_calibration"]["gbs"], unit="GB/s",
                       config={"workload": "plain device copy of 1 GiB"})

    if args.only == "backward":
        st, _ = setup_prefill("llama8b")
        tb = time_backward(st, args.steps, args.warmup, args.settle)
        flb = 10.0 * st["w"].D * st["w"].Hq * st["w"].B * allowed_pairs(st["cu"])
        tf = flb / (tb["backward_ms"] * 1e-3) / 1e12
        out.update(value=round(tf, 2), unit="TFLOP/s", ms_per_step=round(tb["backward_ms"], 4),
                   config={"workload": "llama-3.1-8b attention layer backward (gqa_attention_backward)"},
                   frac=round(tf / PEAK_BF16_TFLOPS, 4))

    if run_8b:
        st, host = setup_prefill("llama8b")
        w, cu = st["w"], st["cu"]
        t = time_prefill(st, args.steps, args.warmup, args.settle)
        fl = prefill_flops(w, cu)
        value = fl / (t["gpu_ms_per_step"] * 1e-3) / 1e12
        achieved = fl / (t["prefill_ms"] * 1e-3) / 1e12
        out.update(value=round(value, 2), unit="TFLOP/s", ms_per_step=round(t["gpu_ms_per_step"], 4))
        out["config"] = {"workload": "llama-3.1-8b attention layer prefill: rope_qk (keys) + "
                                     "gqa_prefill_rope (queries rotated in the kernel), "
                                     "causal + cross-document mask",
                         "batch": w.B, "seq_len": w.S, "q_heads": w.Hq, "kv_heads": w.Hkv,
                         "head_dim": w.D, "rope_base": w.rope_base, "documents": int(cu.size - 1),
                         "allowed_pairs": allowed_pairs(cu), "flops_per_step": fl,
                         "parallelism": "none (1 GPU)"}
        out["roofline"] = {"kernel": "gqa_prefill_rope", "bound": "mfma", "achieved": round(achieved, 2),
                           "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                           "traffic": measured_traffic("gqa_prefill", "llama8b", phash),
                           "launch_ms": round(t["prefill_ms"], 4)}
        out["timing"] = {k: round(x, 4) for k, x in t.items()}
        Sq = 2048
        tc = time_chunk(st, Sq, args.steps, args.warmup, args.settle, CHUNK_SPLIT_TILES)
        tu = time_chunk(st, Sq, args.steps, args.warmup, 0.0)
        flc = 4.0 * w.D * w.Hq * w.B * chunk_pairs(cu, w.S, Sq)
        out["prefill_chunk_8b"] = {
            "workload": f"llama-3.1-8b chunked prefill: the last {Sq} of {w.S} tokens over the "
                        f"cached prefix (rope_qk on the block's keys + gqa_prefill_split, key ranges "
                        f"in pieces of {CHUNK_SPLIT_TILES} x 64 keys, partials merged)",
            "flops": flc,
            "tflops_path": round(flc / (tc["gpu_ms_per_step"] * 1e-3) / 1e12, 2),
            "tflops_kernel": round(flc / (tc["chunk_ms"] * 1e-3) / 1e12, 2),
            "frac_kernel": round(flc / (tc["chunk_ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "chunk_ms": round(tc["chunk_ms"], 4), "rope_ms": round(tc["rope_ms"], 4),
            "unsplit_chunk_ms": round(tu["chunk_ms"], 4),
            "unsplit_tflops_kernel": round(flc / (tu["chunk_ms"] * 1e-3) / 1e12, 2)}
        tb = time_backward(st, max(args.steps // 4, 5), max(args.warmup // 2, 2), args.settle)
        flb = 10.0 * w.D * w.Hq * w.B * allowed_pairs(cu)
        out["backward_8b"] = {
            "workload": "llama-3.1-8b attention layer backward: gqa_attention_backward (delta, "
                        "key-stationary dk/dv, query-stationary dq) on the prefill's shapes and documents",
            "flops": flb, "flops_note": "5 products per visible pair (10 D per pair and head); "
                                        "the kernels run 7 (S and dP are recomputed for dq)",
            "tflops": round(flb / (tb["backward_ms"] * 1e-3) / 1e12, 2),
            "frac": round(flb / (tb["backward_ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "backward_ms": round(tb["backward_ms"], 4)}
        if not args.no_cpu_baseline:
            log("timing the fp64 oracle on a row sample ...")
            out["cpu_baseline"] = cpu_baseline(host, w, cu)
        del st

    if run_405:
        st3, _ = setup_prefill("llama405b")
        t3 = time_prefill(st3, max(3, args.steps // 2), args.warmup, args.settle)
        fl3 = prefill_flops(st3["w"], st3["cu"])
        out["prefill_405b"] = {
            "workload": "llama-3.1-405b attention layer prefill S=32768, 128 q / 8 kv heads",
            "documents": int(st3["cu"].size - 1),
            "tflops_path": round(fl3 / (t3["gpu_ms_per_step"] * 1e-3) / 1e12, 2),
            "tflops_kernel": round(fl3 / (t3["prefill_ms"] * 1e-3) / 1e12, 2),
            "frac_kernel": round(fl3 / (t3["prefill_ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "ms_per_step": round(t3["gpu_ms_per_step"], 4), "prefill_ms": round(t3["prefill_ms"], 4),
            "rope_ms": round(t3["rope_ms"], 4), "traffic": measured_traffic("gqa_prefill", "llama405b", phash)}
        P = 8
        tr = time_ring(st3, P, 2)
        out["ring_405b"] = {
            "workload": f"405b-shape context-parallel attention, S=32768 in {P} shards of {32768 // P}: "
                        f"all {P * P} ring steps (gqa_prefill_ring_step) and {P} finalizes on one GPU",
            "tflops": round(fl3 / (tr * 1e-3) / 1e12, 2),
            "frac": round(fl3 / (tr * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "ms_per_ring": round(tr, 3)}
        if not run_8b:
            out.update(value=out["prefill_405b"]["tflops_path"], unit="TFLOP/s",
                       ms_per_step=out["prefill_405b"]["ms_per_step"],
                       config={"workload": out["prefill_405b"]["workload"]})
        del st3
        if args.with_128k:
            st5, _ = setup_prefill("long128k")
            t5 = time_prefill(st5, 3, 1)
            fl5 = prefill_flops(st5["w"], st5["cu"])
            out["prefill_128k"] = {
                "workload": "405b-shape long-context prefill S=131072, 4 documents",
                "tflops_kernel": round(fl5 / (t5["prefill_ms"] * 1e-3) / 1e12, 2),
                "frac_kernel": round(fl5 / (t5["prefill_ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "prefill_ms": round(t5["prefill_ms"], 3), "rope_ms": round(t5["rope_ms"], 3)}
            del st5
        torch.cuda.empty_cache()

    if run_dec:
        sd = setup_decode()
        td = time_decode(sd, args.steps, args.warmup, args.settle)
        nbytes = decode_bytes(sd)
        gbs = nbytes / (td["decode_ms"] * 1e-3) / 1e9
        dhash = kernel_hash("gqa_decode.hip")
        out["decode_405b"] = {
            "workload": "405b-shape decode: 16 sequences x 1 token, 128 q / 8 kv heads, "
                        "cache lengths U[4096,131072]", "kv_chunk": KV_CHUNK,
            "kv_bytes": nbytes, "gbs_path": round(nbytes / (td["ms_per_step"] * 1e-3) / 1e9, 1),
            "ms_per_step": round(td["ms_per_step"], 4),
            "roofline": {"kernel": "gqa_decode", "bound": "hbm", "achieved": round(gbs, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic("gqa_decode", "decode405b", dhash),
                         "launch_ms": round(td["decode_ms"], 4)},
            "combine_ms": round(td["combine_ms"], 4)}
        page_decode_cache(sd)
        tp = time_decode(sd, args.steps, args.warmup, args.settle, paged=True)
        gbp = nbytes / (tp["decode_ms"] * 1e-3) / 1e9
        out["decode_405b_paged"] = {
            "workload": f"the same decode over a paged cache: {PAGE_SIZE}-slot head-major pages of a pool "
                        "in random order, one block table per sequence (gqa_decode_paged)",
            "gbs": round(gbp, 1), "frac": round(gbp / PEAK_HBM_GBS, 4),
            "decode_ms": round(tp["decode_ms"], 4), "ms_per_step": round(tp["ms_per_step"], 4)}
        if not (run_8b or run_405):
            out.update(value=round(gbs, 1), unit="GB/s", ms_per_step=round(td["ms_per_step"], 4),
                       config={"workload": out["decode_405b"]["workload"]},
                       roofline=out["decode_405b"]["roofline"])

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
