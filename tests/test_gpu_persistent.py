"""The persistent prefill grid (one workgroup per compute unit drawing its work
items from per-XCD queues, each item's first key tiles loaded while the
previous item ends) against the grid of one workgroup per item, on the GPU.

Both grids run the same per-item arithmetic in the same order, so their
outputs agree bit for bit. LLAMA_ATTN_PERSISTENT sets the persistent grid's
size: small grids run many items per workgroup, with every item length, ring
phase and start-load split, and grids that are not a multiple of 8 leave the
queues uneven so that workgroups take items from other queues. Each case runs
twice on one stream (the queue counters must be back at zero after a launch)
and once on a second stream (its own counters). One case is also checked
against the oracle."""

import os

import numpy as np
import pytest
import torch

import gpu_helpers as H
from oracle import reference as orc
from workloads import draw_cu_docs, draw_prefill_inputs

pytestmark = pytest.mark.gpu


def _grid(n):
    if n is None:
        os.environ.pop("LLAMA_ATTN_PERSISTENT", None)
    else:
        os.environ["LLAMA_ATTN_PERSISTENT"] = str(n)


@pytest.fixture(autouse=True)
def _restore_grid():
    old = os.environ.get("LLAMA_ATTN_PERSISTENT")
    yield
    _grid(None if old is None else int(old))


def _run(call, q, k, v, cu, Sq=None, stream=None):
    """One prefill through `call` on device tensors; O and LSE on the CPU."""
    B, S, Hq, D = q.shape
    Sq = S if Sq is None else Sq
    st = stream or torch.cuda.current_stream()
    with torch.cuda.stream(st):
        o = torch.full((B, Sq, Hq, D), float("nan"), dtype=q.dtype, device=q.device)
        lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=q.device)
        call(q[:, S - Sq:].contiguous() if Sq != S else q, k, v, o, lse, cu)
    st.synchronize()
    return o.cpu(), lse.cpu()


def _positions(B, S, seed):
    from workloads import draw_positions
    return torch.as_tensor(draw_positions(B, S, 131071 - S, seed), dtype=torch.int32, device="cuda")


def _calls():
    import gqa_attention_rope_02_amd as la
    return {
        # queries rotated in the kernel (the query operand carries the scale)
        "rope": lambda q, k, v, o, lse, cu: la.gqa_prefill_rope(q, k, v, o, lse, cu),
        # the same with explicit positions and half-split pairs, no LSE output
        "rope_pos_half": lambda q, k, v, o, lse, cu: la.gqa_prefill_rope(
            q, k, v, o, None, cu, positions=_positions(q.shape[0], q.shape[1], 5), rope_pairing="half"),
        # queries given rotated (one FMA per score)
        "plain": lambda q, k, v, o, lse, cu: la.gqa_prefill(q, k, v, o, lse, cu),
        # the last rows of the sequence over its whole key range
        "chunk": lambda q, k, v, o, lse, cu: la.gqa_prefill_chunk(q, k, v, o, lse, cu, rope_base=500000.0),
    }


CASES = [
    # name, B, S, Hq, Hkv, D, documents, call, Sq, grids
    ("8B heads, 5 documents", 1, 1100, 32, 8, 128, 5, "rope", None, (1, 3, 13, 64)),
    ("405B heads, two sequences", 2, 700, 128, 8, 128, 3, "rope", None, (16, 100)),
    ("g=1, D=64", 1, 520, 8, 8, 64, 2, "rope", None, (5,)),
    ("rotated queries, g=2", 1, 900, 16, 8, 128, 4, "plain", None, (7, 30)),
    ("no documents, g=4", 1, 640, 32, 8, 128, None, "rope", None, (9,)),
    ("chunk after a prefix", 1, 1300, 32, 8, 128, 3, "chunk", 500, (11,)),
    ("g=8, positions, half pairs", 2, 600, 64, 8, 128, 4, "rope_pos_half", None, (10,)),
    ("rotated queries, g=16, D=64", 1, 400, 128, 8, 64, 2, "plain", None, (12,)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_persistent_grid_matches_one_workgroup_per_item(case):
    name, B, S, Hq, Hkv, D, nd, call_name, Sq, grids = case
    H.say("persistent grid", dict(case=name, B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, grids=grids))
    dev = torch.device("cuda")
    q, k, v = draw_prefill_inputs(B, S, Hq, Hkv, D, "bf16", 90 + S)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    cu = None
    if nd is not None:
        rows = [draw_cu_docs(S, 90 + S + b, nd, 1) for b in range(B)]
        w = max(r.size for r in rows)
        cu = torch.as_tensor(np.stack([np.concatenate([r, np.full(w - r.size, S, np.int32)]) for r in rows]),
                             dtype=torch.int32, device=dev)
    call = _calls()[call_name]
    _grid(0)
    o0, l0 = _run(call, q, k, v, cu, Sq)
    side = torch.cuda.Stream()
    for g in grids:
        _grid(g)
        for rep, st in enumerate((None, None, side)):
            o1, l1 = _run(call, q, k, v, cu, Sq, st)
            H.say("  grid", dict(grid=g, run=rep))
            assert torch.equal(o1.view(torch.int16), o0.view(torch.int16)), f"O differs at grid {g}, run {rep}"
            assert torch.equal(l1.view(torch.int32), l0.view(torch.int32)), f"LSE differs at grid {g}, run {rep}"


def test_persistent_grid_matches_oracle():
    """The 8B head layout with 6 documents on a 6-workgroup persistent grid
    against the fp64 oracle (RoPE of keys by rope_qk, of queries in the
    kernel)."""
    import gqa_attention_rope_02_amd as la
    B, S, Hq, Hkv, D = 1, 777, 32, 8, 128
    H.say("persistent grid vs oracle", dict(S=S))
    q, k, v = draw_prefill_inputs(B, S, Hq, Hkv, D, "bf16", 97)
    cu = draw_cu_docs(S, 97, 6, 1)
    dev = torch.device("cuda")
    kr = torch.empty_like(k, device=dev)
    la.rope_qk(None, None, k.to(dev), kr)
    _grid(6)
    o, lse = _run(_calls()["rope"], q.to(dev), kr, v.to(dev),
                  torch.as_tensor(cu, dtype=torch.int32, device=dev).reshape(1, -1))
    Ow, Lw = orc.rope_attention(q, k, v, cu, 500000.0, None)
    H.assert_close(o, Ow)
    H.assert_lse_close(lse, Lw, "LSE")


def test_persistent_grid_under_graph_capture():
    """A prefill captured into a HIP graph runs one workgroup per item (a
    stream under capture gets no queue counters); its replays equal the eager
    persistent launch bit for bit. Eager persistent launches and
    synchronisations run between the replays, and the output is refilled
    outside the graph before each replay."""
    import gqa_attention_rope_02_amd as la
    B, S, Hq, Hkv, D = 1, 1100, 32, 8, 128
    H.say("persistent grid and graph capture", dict(S=S))
    dev = torch.device("cuda")
    q, k, v = draw_prefill_inputs(B, S, Hq, Hkv, D, "bf16", 98)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    cu = torch.as_tensor(draw_cu_docs(S, 98, 5, 1), dtype=torch.int32, device=dev).reshape(1, -1)
    _grid(13)
    o_e, l_e = _run(_calls()["rope"], q, k, v, cu)
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, S, dtype=torch.float32, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        la.gqa_prefill_rope(q, k, v, o, lse, cu)   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        la.gqa_prefill_rope(q, k, v, o, lse, cu)
    for rep in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        H.say("  replay", dict(run=rep))
        assert torch.equal(o.cpu().view(torch.int16), o_e.view(torch.int16)), f"O differs at replay {rep}"
        assert torch.equal(lse.cpu().view(torch.int32), l_e.view(torch.int32)), f"LSE differs at replay {rep}"
        o2, l2 = _run(_calls()["rope"], q, k, v, cu)   # eager persistent launch between replays
        assert torch.equal(o2.view(torch.int16), o_e.view(torch.int16))
        assert torch.equal(l2.view(torch.int32), l_e.view(torch.int32))
