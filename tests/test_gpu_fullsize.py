"""The full-size workloads on the GPU, in the launch configuration bench.py
times: rope_qk on the keys then gqa_prefill_rope (queries rotated in the
kernel) over the whole packed sequence, and
gqa_decode + gqa_decode_combine over the whole cache with bench.py's kv_chunk.

Outputs the oracle cannot afford everywhere are checked on sampled query rows
(every document's first and last row, rows either side of drawn 64-row tile
edges, uniformly drawn rows) against the fp64 row oracle; closed-form probes
(q = 0: uniform attention over the visible keys) check the mask and the head
mapping exactly over every row and head.
"""

import numpy as np
import pytest
import torch

import gpu_helpers as H
from oracle import reference as orc
from workloads import CONFIGS, draw_cu_docs, draw_prefill_inputs, sample_rows

pytestmark = pytest.mark.gpu

# sampled rows per workload: (uniform draws, tile edges drawn (None: every
# edge), parts the oracle's share is split into)
SAMPLES = {"llama8b": (2048, None, 1), "llama405b": (2048, None, 3), "long128k": (1024, 256, 4)}


def _run_full_prefill(q, k, v, cu):
    """The prefill path exactly as bench.py launches it: rope_qk on the keys,
    then gqa_prefill_rope (queries rotated in the kernel); device outputs."""
    import gqa_attention_rope_02_amd as la
    dev = torch.device("cuda")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    kr = torch.empty_like(kd)
    la.rope_qk(None, None, kd, kr)
    del kd
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((q.shape[0], q.shape[2], q.shape[1]), float("nan"), device=dev)
    cu_d = torch.as_tensor(cu, dtype=torch.int32).reshape(1, -1).to(dev)
    la.gqa_prefill_rope(qd, kr, vd, o, lse, cu_d)
    torch.cuda.synchronize()
    return o, lse


_SAMPLED = {}


def _sampled_outputs(name):
    """One GPU run per workload: the sampled rows' O and LSE (kept on the host
    for the parts of the oracle check), with the host inputs."""
    if name not in _SAMPLED:
        _SAMPLED.clear()
        w = CONFIGS[name]
        H.say("full-size prefill", name, w.S, w.Hq, w.Hkv)
        q, k, v = draw_prefill_inputs(w.B, w.S, w.Hq, w.Hkv, w.D, w.dtype, w.seed)
        cu = draw_cu_docs(w.S, w.seed, w.n_docs, w.n_docs_max)
        o, lse = _run_full_prefill(q, k, v, cu)
        assert torch.isfinite(o).all() and torch.isfinite(lse).all()
        n_random, n_edges, _ = SAMPLES[name]
        rows = sample_rows(w.S, cu, w.seed, n_random=n_random, n_edges=n_edges)
        idx = torch.as_tensor(rows, device=o.device)
        got_o = o[0].index_select(0, idx).cpu()
        got_l = lse[0].index_select(1, idx).cpu()
        del o, lse, idx
        torch.cuda.empty_cache()
        _SAMPLED[name] = (w, cu, rows, got_o, got_l, (q, k, v))
    return _SAMPLED[name]


@pytest.mark.parametrize("name,part", [(n, p) for n, (_, _, P) in SAMPLES.items() for p in range(P)])
def test_full_size_prefill_sampled_rows(name, part):
    """Every document's first and last row, the rows either side of every
    64-row tile edge (drawn edges at 128K) and uniformly drawn rows, all heads,
    against the fp64 row oracle; the sample is checked in interleaved parts."""
    w, cu, rows, got_o, got_l, (q, k, v) = _sampled_outputs(name)
    P = SAMPLES[name][2]
    sel = np.arange(rows.size)[part::P]
    H.say("  rows", rows.size, "part", part, "of", P, ":", sel.size)
    Ow, Lw = H.oracle_rows_threaded(q[0], k[0], v[0], rows[sel], cu, w.rope_base)
    H.assert_close(got_o[sel], Ow, what=f"O {name} part {part}")
    H.assert_lse_close(got_l[:, sel], Lw, f"LSE {name} part {part}")
    if part == P - 1:
        _SAMPLED.clear()


def _code(j):
    """A key position in three channels of 6 bits, as n / 64 (n = 0..63: exact
    in bf16, and of the size of the other values, so the output's rounding stays
    within the parity bar)."""
    return np.array([j >> 12, (j >> 6) & 63, j & 63], dtype=np.float64) / 64.0


def _decode(x):
    return np.rint(np.asarray(x, dtype=np.float64) * 64.0) / 64.0


# (query row, query head, distance to the planted key)
NEEDLES = [(131071, 5, 131071), (131071, 77, 1), (100000, 120, 65536), (65535, 0, 64),
           (8191, 33, 4095), (131000, 64, 100001), (77777, 100, 0), (4096, 17, 4096),
           (120001, 126, 9999)]


def _plant(q, k, v, needles, base, c=3.0):
    """For each needle: the key at position j = row - distance (of the query
    head's KV head) is set, unrotated, to R(-j) (c R(row) q_row), so that after
    RoPE it is c times the rotated query; its V row carries the code of j in
    channels 0..2. Rotations in fp64 by the oracle's RoPE."""
    from oracle import reference as orc
    Hq, Hkv = q.shape[2], k.shape[2]
    g = Hq // Hkv
    for i, h, dist in needles:
        j = i - dist
        kvh = h // g
        qr = orc.rope(q[0, i:i + 1, h:h + 1].double().numpy(), np.array([i]), base)   # [1, 1, D]
        kraw = orc.rope(c * qr, np.array([-j]), base)
        k[0, j, kvh] = torch.as_tensor(kraw[0, 0]).to(k.dtype)
        v[0, j, kvh, :3] = torch.as_tensor(_code(j)).to(v.dtype)


def test_needles_at_128k():
    """Planted needles in the 128K context (one document): a key made equal,
    after RoPE, to 3x the rotated query of one (row, head) dominates that row's
    softmax, so the row's output returns the key's V row: the position coded in
    it comes back exactly for distances from 0 to 131071 (long-range positions,
    the fp64 angle reduction at position 131071 and the causal mask at its
    edge), and the needle rows match the fp64 row oracle."""
    w = CONFIGS["long128k"]
    H.say("needles at 128K", len(NEEDLES))
    q, k, v = draw_prefill_inputs(w.B, w.S, w.Hq, w.Hkv, w.D, w.dtype, w.seed)
    assert len({(i - d, h // (w.Hq // w.Hkv)) for i, h, d in NEEDLES}) == len(NEEDLES)
    _plant(q, k, v, NEEDLES, w.rope_base)
    cu = np.array([0, w.S], dtype=np.int32)
    o, lse = _run_full_prefill(q, k, v, cu)
    rows = np.array(sorted({i for i, _, _ in NEEDLES}))
    got_o = o[0].index_select(0, torch.as_tensor(rows, device=o.device)).cpu()
    got_l = lse[0].index_select(1, torch.as_tensor(rows, device=o.device)).cpu()
    del o, lse
    for i, h, dist in NEEDLES:
        r = int(np.searchsorted(rows, i))
        code = _decode(got_o[r, h, :3].double().numpy())
        assert np.array_equal(code, _code(i - dist)), (i, h, dist, got_o[r, h, :3])
    Ow, Lw = H.oracle_rows_threaded(q[0], k[0], v[0], rows, cu, w.rope_base)
    H.assert_close(got_o, Ow, what="O needle rows")
    H.assert_lse_close(got_l, Lw, "LSE needle rows")
    # the oracle agrees that each needle is its row's heaviest key by far
    for i, h, dist in NEEDLES:
        r = int(np.searchsorted(rows, i))
        assert np.array_equal(_decode(Ow[r, h, :3]), _code(i - dist))


def test_needle_across_a_document_boundary_is_not_retrieved():
    """The same planted keys with the 128K workload's four documents: a needle
    whose key lies in an earlier document than its query row is masked, so the
    row's output is an ordinary mixture (matching the oracle), not the key's
    V row; needles inside the row's own document are still retrieved."""
    w = CONFIGS["long128k"]
    cu = draw_cu_docs(w.S, w.seed, w.n_docs, w.n_docs_max)
    doc = orc.document_of(cu, w.S)
    H.say("needles across documents", cu.tolist())
    q, k, v = draw_prefill_inputs(w.B, w.S, w.Hq, w.Hkv, w.D, w.dtype, w.seed)
    _plant(q, k, v, NEEDLES, w.rope_base)
    o, lse = _run_full_prefill(q, k, v, cu)
    rows = np.array(sorted({i for i, _, _ in NEEDLES}))
    got_o = o[0].index_select(0, torch.as_tensor(rows, device=o.device)).cpu()
    got_l = lse[0].index_select(1, torch.as_tensor(rows, device=o.device)).cpu()
    del o, lse
    crossing = 0
    for i, h, dist in NEEDLES:
        r = int(np.searchsorted(rows, i))
        code = _decode(got_o[r, h, :3].double().numpy())
        if doc[i] == doc[i - dist]:
            assert np.array_equal(code, _code(i - dist))
        else:
            crossing += 1
            assert not np.array_equal(code, _code(i - dist))
    assert crossing >= 3
    Ow, Lw = H.oracle_rows_threaded(q[0], k[0], v[0], rows, cu, w.rope_base)
    H.assert_close(got_o, Ow, what="O needle rows, 4 documents")
    H.assert_lse_close(got_l, Lw, "LSE needle rows, 4 documents")


@pytest.mark.parametrize("name", ["llama8b", "llama405b", "long128k"])
def test_full_size_prefill_exact_probes(name):
    """q = 0 makes every visible key weigh 1: exp(LSE) is the exact count of
    visible keys; a V channel holding the document index comes back exactly
    (only same-document keys mix); one holding the KV head index comes back as
    h // g for query head h."""
    w = CONFIGS[name]
    H.say("full-size probes", name)
    dev = torch.device("cuda")
    cu = draw_cu_docs(w.S, w.seed, w.n_docs, w.n_docs_max)
    doc = orc.document_of(cu, w.S)
    _, k, v = draw_prefill_inputs(w.B, w.S, 1, w.Hkv, w.D, w.dtype, w.seed)
    v[0, :, :, 0] = torch.as_tensor(doc, dtype=torch.bfloat16)[:, None]
    v[0, :, :, 1] = torch.arange(w.Hkv, dtype=torch.bfloat16)[None, :]
    q = torch.zeros(w.B, w.S, w.Hq, w.D, dtype=torch.bfloat16, device=dev)
    o, lse = _run_full_prefill(q, k, v, cu)
    g = w.Hq // w.Hkv
    count = np.arange(w.S) - cu[doc] + 1
    got = np.rint(np.exp(lse[0].double().cpu().numpy()))
    assert np.array_equal(got, np.broadcast_to(count, (w.Hq, w.S)))
    ch = o[0, :, :, :2].float().cpu().numpy()
    assert np.array_equal(ch[:, :, 0], np.broadcast_to(doc[:, None], (w.S, w.Hq)))
    assert np.array_equal(ch[:, :, 1], np.broadcast_to((np.arange(w.Hq) // g)[None, :], (w.S, w.Hq)))


def test_full_size_decode_sampled_heads():
    """The 405B-shape decode of bench.py (16 sequences, cache lengths up to
    128K, 128 query heads on 8 KV heads, its kv_chunk): for every sequence the
    16 query heads of two KV heads against the oracle, and the partial-result
    workspace of those heads (runs of merged splits) against the oracle's
    per-split partials merged over each run."""
    import bench
    import gqa_attention_rope_02_amd as la
    H.say("full-size decode405b")
    st = bench.setup_decode()
    w, lens, chunk = st["w"], st["lens"], bench.KV_CHUNK
    op = torch.full_like(st["op"], float("nan"))
    lp = torch.full_like(st["lp"], float("nan"))
    o = torch.full_like(st["o"], float("nan"))
    lse = torch.full((w.B, w.Hq), float("nan"), device=o.device)
    la.gqa_decode(st["q"], st["kc"], st["vc"], st["sl"], chunk, op, lp)
    la.gqa_decode_combine(op, lp, st["sl"], chunk, o, lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    g = w.Hq // w.Hkv
    n_runs = 0
    for b in range(w.B):
        L = int(lens[b])
        for kvh in (b % w.Hkv, (b + 3) % w.Hkv):
            heads = slice(kvh * g, (kvh + 1) * g)
            qb = st["q"][b:b + 1, heads].cpu()
            kb = [st["kc"][b, kvh:kvh + 1, :L].cpu()]
            vb = [st["vc"][b, kvh:kvh + 1, :L].cpu()]
            Ow, Lw = orc.decode(qb, kb, vb, [L])
            H.assert_close(o[b:b + 1, heads].cpu(), Ow, what=f"O b={b} kvh={kvh}")
            H.assert_lse_close(lse[b:b + 1, heads].cpu(), Lw, "LSE")
            n_runs += H.check_partials(op[b:b + 1, heads].cpu(), lp[b:b + 1, heads].cpu(),
                                       qb, kb, vb, [L], chunk)
    H.say("  runs checked", n_runs)


def test_full_size_decode_is_deterministic():
    """The 405B-shape decode three times on the same inputs, workspaces
    NaN-filled before each call: partial results, their LSE and the combined
    output agree bit for bit (a result that depends on timing, such as a read
    of a matrix-core result before it is ready, shows up here)."""
    import bench
    import gqa_attention_rope_02_amd as la
    H.say("full-size decode determinism")
    st = bench.setup_decode()
    chunk = bench.KV_CHUNK
    first = None
    for _ in range(3):
        op = torch.full_like(st["op"], float("nan"))
        lp = torch.full_like(st["lp"], float("nan"))
        o = torch.full_like(st["o"], float("nan"))
        la.gqa_decode(st["q"], st["kc"], st["vc"], st["sl"], chunk, op, lp)
        la.gqa_decode_combine(op, lp, st["sl"], chunk, o)
        torch.cuda.synchronize()
        live = torch.isfinite(lp)
        got = (lp.nan_to_num(0.0), op * live[..., None], o)
        if first is None:
            first = got
        else:
            for a, b in zip(first, got):
                assert torch.equal(a.nan_to_num(0.0), b.nan_to_num(0.0))


@pytest.mark.parametrize("name", ["llama8b", "llama405b"])
def test_full_size_prefill_is_deterministic(name):
    """The bench prefill three times on the same rotated inputs: O and LSE
    agree bit for bit."""
    import bench
    import gqa_attention_rope_02_amd as la
    H.say("full-size prefill determinism", name)
    st, _ = bench.setup_prefill(name)
    la.rope_qk(None, None, st["k"], st["kr"])
    first = None
    for _ in range(3):
        o = torch.full_like(st["o"], float("nan"))
        lse = torch.full_like(st["lse"], float("nan"))
        la.gqa_prefill_rope(st["q"], st["kr"], st["v"], o, lse, st["cu_d"])
        torch.cuda.synchronize()
        if first is None:
            first = (o, lse)
        else:
            assert torch.equal(first[0], o) and torch.equal(first[1], lse)


def test_full_size_chunked_prefill_sampled_rows():
    """bench.py's chunked prefill: the last 2048 of the llama8b workload's 8192
    tokens over the cached prefix, gqa_prefill_split with its piece size
    (queries rotated in the kernel at their positions), sampled block rows
    against the fp64 row oracle."""
    import bench
    import gqa_attention_rope_02_amd as la
    w = CONFIGS["llama8b"]
    S, Sq = w.S, 2048
    H.say("full-size chunked prefill", S, Sq, bench.CHUNK_SPLIT_TILES)
    q, k, v = draw_prefill_inputs(w.B, w.S, w.Hq, w.Hkv, w.D, w.dtype, w.seed)
    cu = draw_cu_docs(w.S, w.seed, w.n_docs, w.n_docs_max)
    dev = torch.device("cuda")
    kd, vd = k.to(dev), v.to(dev)
    kr = torch.empty_like(kd)
    la.rope_qk(None, None, kd, kr)
    qb = q[:, S - Sq:].contiguous().to(dev)
    o = torch.full_like(qb, float("nan"))
    lse = torch.full((w.B, w.Hq, Sq), float("nan"), device=dev)
    op, lp = la.prefill_split_workspace(w.B, Sq, S, w.Hq, w.D, bench.CHUNK_SPLIT_TILES, dev)
    cu_d = torch.as_tensor(cu, dtype=torch.int32).reshape(1, -1).to(dev)
    la.gqa_prefill_split(qb, kr, vd, o, bench.CHUNK_SPLIT_TILES, op, lp, lse, cu_d, rope_base=w.rope_base)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    rows = sample_rows(S, cu, w.seed + 1, n_random=512)
    rows = rows[rows >= S - Sq]
    idx = torch.as_tensor(rows - (S - Sq), device=dev)
    Ow, Lw = orc.rope_attention_rows(q[0], k[0], v[0], rows, cu, w.rope_base)
    H.say("  rows", rows.size)
    H.assert_close(o[0].index_select(0, idx).cpu(), Ow)
    H.assert_lse_close(lse[0].index_select(1, idx).cpu(), Lw, "LSE")


def test_full_size_paged_decode_equals_contiguous():
    """bench.py's paged decode shape (405B decode, 64-slot head-major pages in a
    seeded random order, its kv_chunk) on pages copied from the contiguous
    cache: partials and merged output equal gqa_decode's bit for bit (the
    contiguous decode is checked against the oracle above)."""
    import bench
    import gqa_attention_rope_02_amd as la
    H.say("full-size paged decode405b")
    st = bench.setup_decode()
    w, lens, chunk, P = st["w"], st["lens"], bench.KV_CHUNK, bench.PAGE_SIZE
    st["op"].fill_(float("nan"))
    st["lp"].fill_(float("nan"))
    la.gqa_decode(st["q"], st["kc"], st["vc"], st["sl"], chunk, st["op"], st["lp"])
    la.gqa_decode_combine(st["op"], st["lp"], st["sl"], chunk, st["o"])
    torch.cuda.synchronize()
    ref = (st["op"].cpu(), st["lp"].cpu(), st["o"].cpu())
    need = [-(-int(L) // P) for L in lens]
    order = np.random.default_rng(w.seed).permutation(int(sum(need)))
    table = np.zeros((w.B, -(-st["Lmax"] // P)), dtype=np.int32)
    dev = st["q"].device
    kp = torch.empty(int(sum(need)), w.Hkv, P, w.D, dtype=torch.bfloat16, device=dev)
    vp = torch.empty_like(kp)
    n = 0
    for b in range(w.B):
        ids = order[n:n + need[b]]
        n += need[b]
        table[b, :need[b]] = ids
        idt = torch.as_tensor(ids, device=dev)
        span = need[b] * P
        kp.index_copy_(0, idt, st["kc"][b, :, :span].reshape(w.Hkv, need[b], P, w.D).permute(1, 0, 2, 3))
        vp.index_copy_(0, idt, st["vc"][b, :, :span].reshape(w.Hkv, need[b], P, w.D).permute(1, 0, 2, 3))
    tb = torch.as_tensor(table).to(dev)
    op = torch.full_like(st["op"], float("nan"))
    lp = torch.full_like(st["lp"], float("nan"))
    o = torch.full_like(st["o"], float("nan"))
    la.gqa_decode_paged(st["q"], kp.permute(0, 2, 1, 3), vp.permute(0, 2, 1, 3), tb, st["sl"], chunk, op, lp,
                        st["Lmax"])
    la.gqa_decode_combine(op, lp, st["sl"], chunk, o)
    torch.cuda.synchronize()
    for got, want in zip((op.cpu(), lp.cpu(), o.cpu()), ref):
        assert torch.equal(torch.nan_to_num(got, nan=7.0), torch.nan_to_num(want, nan=7.0))


def test_full_size_ring_sampled_rows():
    """bench.py's ring: the llama405b workload as 8 devices of a context-
    parallel ring would run it (8 shards of 4096 tokens, every query shard
    against the key shards its rows can see in ring order, fp32 partials
    merged, the last step writing the output), all on this GPU; sampled rows
    (and their LSE) against the fp64 row oracle."""
    import bench
    import gqa_attention_rope_02_amd as la
    w = CONFIGS["llama405b"]
    P = 8
    S, L = w.S, w.S // P
    H.say("full-size ring", S, P)
    q, k, v = draw_prefill_inputs(w.B, w.S, w.Hq, w.Hkv, w.D, w.dtype, w.seed)
    cu = draw_cu_docs(w.S, w.seed, w.n_docs, w.n_docs_max)
    dev = torch.device("cuda")
    qd, vd = q.to(dev), v.to(dev)
    kr = torch.empty_like(k.to(dev))
    la.rope_qk(None, None, k.to(dev), kr)
    cu_d = torch.as_tensor(cu, dtype=torch.int32).reshape(1, -1).to(dev)
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((w.B, w.Hq, S), float("nan"), device=dev)
    oa = torch.empty(w.B, L, w.Hq, w.D, dtype=torch.float32, device=dev)
    lsa = torch.empty(w.B, w.Hq, L, dtype=torch.float32, device=dev)
    lb = torch.empty(w.B, w.Hq, L, dtype=torch.float32, device=dev)
    for i in range(P):
        q0 = i * L
        sched = bench.ring_schedule(cu, S, P, i)
        for n, j in enumerate(sched):
            args = (qd[:, q0:q0 + L], kr[:, j * L:(j + 1) * L], vd[:, j * L:(j + 1) * L], q0, j * L, oa, lsa)
            if n == len(sched) - 1:
                la.gqa_prefill_ring_step_final(*args, o[:, q0:q0 + L], lb, first=(n == 0), cu_docs=cu_d,
                                               rope_base=w.rope_base)
            else:
                la.gqa_prefill_ring_step(*args, first=(n == 0), cu_docs=cu_d, rope_base=w.rope_base)
        lse[:, :, q0:q0 + L] = lb
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    rows = sample_rows(S, cu, w.seed + 2, n_random=256, n_edges=32)
    idx = torch.as_tensor(rows, device=dev)
    got_o = o[0].index_select(0, idx).cpu()
    got_l = lse[0].index_select(1, idx).cpu()
    del o, lse, oa
    Ow, Lw = orc.rope_attention_rows(q[0], k[0], v[0], rows, cu, w.rope_base)
    H.say("  rows", rows.size)
    H.assert_close(got_o, Ow)
    H.assert_lse_close(got_l, Lw, "LSE")
