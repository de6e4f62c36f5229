"""The allocation-free decode (gqa_decode_noalloc) through the C ABI: its
output and log-sum-exp equal those of gqa_decode + gqa_decode_combine with a
caller-owned workspace, bit for bit, on two calls in a row (the second with a
smaller input), and match the fp64 oracle within the parity bar; a working
set beyond the scratch is refused before anything is launched."""

import numpy as np
import pytest
import torch

from gpu_helpers import assert_close, assert_lse_close, say

pytestmark = pytest.mark.gpu


def _inputs(B, Hq, Hkv, D, Lmax, seed):
    g = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, Lmax + 1, size=B).astype(np.int32)
    q = torch.randn(B, Hq, D, generator=g).bfloat16()
    kc = torch.randn(B, Hkv, Lmax, D, generator=g).bfloat16()
    vc = torch.randn(B, Hkv, Lmax, D, generator=g).bfloat16()
    return q, kc, vc, lens


def _with_workspace(q, kc, vc, sl, chunk):
    import gqa_attention_rope_02_amd as la
    B, Hq, D = q.shape
    ms = -(-kc.shape[2] // chunk)
    op = torch.empty(B, Hq, ms, D, device="cuda")
    lp = torch.empty(B, Hq, ms, device="cuda")
    o = torch.full((B, Hq, D), float("nan"), device="cuda").bfloat16()
    lse = torch.full((B, Hq), float("nan"), device="cuda")
    la.gqa_decode(q, kc, vc, sl, chunk, op, lp)
    la.gqa_decode_combine(op, lp, sl, chunk, o, lse)
    torch.cuda.synchronize()
    return o, lse


def _noalloc(q, kc, vc, sl, chunk):
    import gqa_attention_rope_02_amd as la
    B, Hq, D = q.shape
    o = torch.full((B, Hq, D), float("nan"), device="cuda").bfloat16()
    lse = torch.full((B, Hq), float("nan"), device="cuda")
    la.gqa_decode_noalloc(q, kc, vc, sl, chunk, o, lse)
    torch.cuda.synchronize()
    return o, lse


def test_noalloc_equals_workspace_decode_on_two_calls(gpu_lib):
    from oracle import reference as orc
    for i, (B, Hq, Hkv, D, Lmax, chunk) in enumerate([(8, 32, 4, 128, 3000, 128), (3, 16, 1, 64, 700, 64)]):
        say("noalloc decode call", i, (B, Hq, Hkv, D, Lmax, chunk))
        q, kc, vc, lens = _inputs(B, Hq, Hkv, D, Lmax, 11 + i)
        dev = [t.to("cuda") for t in (q, kc, vc)]
        sl = torch.as_tensor(lens).to("cuda")
        o_ref, lse_ref = _with_workspace(*dev, sl, chunk)
        o, lse = _noalloc(*dev, sl, chunk)
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
        # and the oracle (keys in the cache are used as stored)
        ow, lw = orc.decode(q.double().numpy(), kc.double().numpy(), vc.double().numpy(), lens)
        assert_close(o.cpu(), ow, what="o")
        assert_lse_close(lse.cpu().double(), lw, "lse")


def test_noalloc_full_size_405b_decode_equals_workspace_decode(gpu_lib):
    """16 sequences of U[4096, 131072] tokens, 128 query heads on 8 KV heads:
    the bench's decode workload and launch configuration (kv_chunk 256)."""
    from workloads import CONFIGS, draw_seq_lens
    w = CONFIGS["decode405b"]
    lens = draw_seq_lens(w.B, w.len_lo, w.len_hi, w.seed)
    say("noalloc decode full size", lens.tolist())
    g = torch.Generator(device="cuda").manual_seed(w.seed)
    kc = torch.empty(w.B, w.Hkv, w.len_hi, w.D, dtype=torch.bfloat16, device="cuda").normal_(generator=g)
    vc = torch.empty_like(kc).normal_(generator=g)
    q = torch.randn(w.B, w.Hq, w.D, generator=g, device="cuda").bfloat16()
    sl = torch.as_tensor(lens, dtype=torch.int32).to("cuda")
    o_ref, lse_ref = _with_workspace(q, kc, vc, sl, 256)
    o, lse = _noalloc(q, kc, vc, sl, 256)
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)


def test_noalloc_refuses_a_working_set_beyond_its_scratch(gpu_lib):
    import gqa_attention_rope_02_amd as la
    say("noalloc decode scratch limit")
    B, Hq, Hkv, D, Lmax = 1024, 128, 8, 128, 64   # (waves + 8192) slots x 16 x 129 x 4 B > 32 MiB
    q = torch.zeros(B, Hq, D, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(B, Hkv, Lmax, D, dtype=torch.bfloat16, device="cuda")
    sl = torch.full((B,), Lmax, dtype=torch.int32, device="cuda")
    o = torch.full((B, Hq, D), float("nan"), device="cuda").bfloat16()
    with pytest.raises(la.LlamaAttnError) as e:
        la.gqa_decode_noalloc(q, kc, kc, sl, 64, o)
    assert e.value.status == 4
    torch.cuda.synchronize()
    assert torch.isnan(o.float()).all()
