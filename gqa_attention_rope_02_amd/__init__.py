"""Python binding of the gfx950 GQA + RoPE attention library.

The calls mirror the C ABI in ``include/llama_attn.h`` one to one and only
marshal arguments: tensor pointers, element strides, sizes and the current HIP
stream. Every step of the computation runs in the library's HIP kernels;
PyTorch provides device memory and streams. Tensors must live on the GPU.

Shapes (strides are taken from the tensors; the last dimension must be
contiguous):

* ``rope_qk(q_in, q_out, k_in, k_out, positions=None, rope_base=500000.0,
  rope_pairing="adjacent")``: q [B,S,Hq,D], k [B,S,Hkv,D] (either pair may be None);
  positions int32 [B,S]; rope_pairing "adjacent" (channels 2k, 2k+1) or "half"
  (k, k+D/2), also taken by every call below that takes rope_base.
* ``rope_qk_backward(dq_in, dq_out, dk_in=None, dk_out=None, positions=None,
  rope_base=500000.0, rope_pairing="adjacent")``: the transpose of rope_qk (rotation
  by minus the angles): gradients for rotated q/k to gradients for the inputs.
* ``gqa_prefill(q, k, v, o, lse=None, cu_docs=None, softmax_scale=0.0)``:
  q/o [B,S,Hq,D], k/v [B,S,Hkv,D], cu_docs int32 [B, n_docs+1], lse fp32 [B,Hq,S].
* ``gqa_prefill_rope(q, k, v, o, lse=None, cu_docs=None, softmax_scale=0.0,
  positions=None, rope_base=500000.0)``: as gqa_prefill with unrotated q (the
  kernel rotates it; k must be rotated, e.g. by rope_qk with q_in None).
* ``gqa_prefill_chunk(q, k, v, o, lse=None, cu_docs=None, softmax_scale=0.0,
  positions=None, rope_base=0.0)``: q/o [B,Sq,Hq,D] are the last Sq tokens of
  sequences whose k/v [B,S,Hkv,D] hold all S tokens (a cached prefix plus the
  block); lse fp32 [B,Hq,Sq]; rope_base 0 = q already rotated, > 0 = rotate q
  in the kernel at positions [B,Sq] (default S-Sq+i).
* ``gqa_prefill_split(q, k, v, o, split_tiles, o_part, lse_part, lse=None, cu_docs=None,
  softmax_scale=0.0, positions=None, rope_base=0.0)``: gqa_prefill_chunk with each query
  tile's key range cut into pieces of split_tiles x 64 keys (workspace o_part fp32
  [max_splits,B,Sq,Hq,D], lse_part fp32 [max_splits,B,Hq,Sq]; ``prefill_split_workspace``
  allocates it).
* ``gqa_prefill_ring_step(q, k, v, q_off, k_off, o_acc, lse_acc, first, cu_docs=None,
  softmax_scale=0.0, positions=None, rope_base=0.0)``: queries [B,Sq,Hq,D] at positions
  q_off.. against a key shard k/v [B,Skv,Hkv,D] at positions k_off..; writes (first) or
  merges the shard's result into o_acc fp32 [B,Sq,Hq,D], lse_acc fp32 [B,Hq,Sq].
* ``gqa_prefill_ring_finalize(o_acc, lse_acc, o, lse=None)``: o [B,Sq,Hq,D] from them.
* ``gqa_attention_backward(q, k, v, o, dout, lse, dq, dk, dv, delta=None, cu_docs=None,
  softmax_scale=0.0, workspace="auto")``: gradients of gqa_prefill (bf16): q, o, dout, dq
  [B,S,Hq,D]; k, v, dk, dv [B,S,Hkv,D]; lse fp32 [B,Hq,S] from the forward; delta fp32
  [B,Hq,S] workspace (allocated when None); workspace: ``backward_workspace(B, S, Hkv, D)``
  (allocated when "auto"; None runs without cutting long query ranges).
* kv_chunk (keys per split of the decode calls) may be None: the
  LLAMA_ATTN_KV_CHUNK environment variable, else 256 (``default_kv_chunk()``).
* ``gqa_decode(q, k_cache, v_cache, seq_lens, kv_chunk, o_part, lse_part,
  softmax_scale=0.0)``: q [B,Hq,D], caches [B,Hkv,Lmax,D], seq_lens int32 [B],
  o_part fp32 [B,Hq,max_splits,D], lse_part fp32 [B,Hq,max_splits].
* ``gqa_decode_paged(q, k_pages, v_pages, block_table, seq_lens, kv_chunk, o_part, lse_part,
  Lmax, softmax_scale=0.0)``: as gqa_decode over a paged cache: pools [n_pages, page_size,
  Hkv, D] (any page/slot/head strides), block_table int32 [B, pages per sequence].
* ``gqa_decode_combine(o_part, lse_part, seq_lens, kv_chunk, o, lse=None)``:
  o [B,Hq,D] (bf16 or fp32), lse fp32 [B,Hq].
* ``gqa_decode_noalloc(q, k_cache, v_cache, seq_lens, kv_chunk, o, lse=None,
  softmax_scale=0.0)``: gqa_decode + gqa_decode_combine with the partials in the
  library's own device scratch (no workspace, no allocation).
"""

from __future__ import annotations

import os

import torch

from . import _lib

__all__ = ["LlamaAttnError", "rope_qk", "rope_qk_backward", "gqa_attention_backward", "backward_workspace", "gqa_prefill", "gqa_prefill_rope", "gqa_prefill_chunk",
           "gqa_prefill_split", "prefill_split_workspace", "gqa_prefill_ring_step",
           "gqa_prefill_ring_finalize", "gqa_decode", "gqa_decode_paged",
           "gqa_decode_combine", "gqa_decode_noalloc", "default_kv_chunk", "version", "LA_BF16", "LA_FP32"]

LA_BF16, LA_FP32 = 0, 1
_DT = {torch.bfloat16: LA_BF16, torch.float32: LA_FP32}


class LlamaAttnError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        msg = _lib.load().la_status_str(status).decode()
        super().__init__(f"{call}: {msg} (status {status})")


def version() -> int:
    return _lib.load().la_version()


def _check(status: int, call: str) -> None:
    if status != 0:
        raise LlamaAttnError(status, call)


def _dev(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError("llama_attn tensors must be torch tensors on the GPU")
    return t.data_ptr()


def _i32(t):
    if t is None:
        return None
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise ValueError("index tensors (positions, cu_docs, seq_lens) must be contiguous int32")
    return _dev(t)


def _f32c(t):
    if t is None:
        return None
    if t.dtype != torch.float32 or not t.is_contiguous():
        raise ValueError("lse / split workspaces must be contiguous float32")
    return _dev(t)


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dtype(t) -> int:
    if t.dtype not in _DT:
        raise ValueError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _same_dtype(call, dt, **tensors):
    """Every given tensor must have dtype dt (the kernels index all of a call's
    tensors with one element size)."""
    for name, t in tensors.items():
        if t is not None and t.dtype != dt:
            raise ValueError(f"{call}: {name} is {t.dtype}, the call's tensors are {dt}")


def _strides(t, n):
    if t is None:
        return None
    if t.stride(-1) != 1:
        raise ValueError("the last (head_dim) dimension must be contiguous")
    return _lib.i64_array(t.stride()[:n])


def _same_shape(call, *pairs):
    for a, b in pairs:
        if a is not None and b is not None and tuple(a.shape) != tuple(b.shape):
            raise ValueError(f"{call}: shape mismatch {tuple(a.shape)} vs {tuple(b.shape)}")


_PAIRING = {"adjacent": 0, "half": 1}


def _pairing(p) -> int:
    """rope_pairing: "adjacent" (channels 2k, 2k+1) or "half" (k, k + D/2)."""
    if p not in _PAIRING:
        raise ValueError(f"rope_pairing must be one of {sorted(_PAIRING)}, not {p!r}")
    return _PAIRING[p]


def rope_qk(q_in, q_out, k_in=None, k_out=None, positions=None, rope_base: float = 500000.0,
            rope_pairing: str = "adjacent"):
    ref = q_in if q_in is not None else k_in
    B, S, _, D = ref.shape
    Hq = q_in.shape[2] if q_in is not None else 0
    Hkv = k_in.shape[2] if k_in is not None else 0
    _same_shape("rope_qk", (q_in, q_out), (k_in, k_out))
    if q_in is not None and k_in is not None and (k_in.shape[:2] != q_in.shape[:2] or k_in.shape[3] != D):
        raise ValueError("rope_qk: q and k must share B, S and D")
    if positions is not None and tuple(positions.shape) != (B, S):
        raise ValueError("rope_qk: positions must be [B, S]")
    _same_dtype("rope_qk", ref.dtype, q_in=q_in, q_out=q_out, k_in=k_in, k_out=k_out)
    st = _lib.load().rope_qk(
        _dev(q_in), _dev(q_out), _strides(q_in, 3), _strides(q_out, 3),
        _dev(k_in), _dev(k_out), _strides(k_in, 3), _strides(k_out, 3),
        _dtype(ref), B, S, Hq, Hkv, D, _i32(positions), float(rope_base), _pairing(rope_pairing),
        _stream())
    _check(st, "rope_qk")


def rope_qk_backward(dq_in, dq_out, dk_in=None, dk_out=None, positions=None,
                     rope_base: float = 500000.0, rope_pairing: str = "adjacent"):
    ref = dq_in if dq_in is not None else dk_in
    B, S, _, D = ref.shape
    Hq = dq_in.shape[2] if dq_in is not None else 0
    Hkv = dk_in.shape[2] if dk_in is not None else 0
    _same_shape("rope_qk_backward", (dq_in, dq_out), (dk_in, dk_out))
    if dq_in is not None and dk_in is not None and (dk_in.shape[:2] != dq_in.shape[:2] or dk_in.shape[3] != D):
        raise ValueError("rope_qk_backward: dq and dk must share B, S and D")
    if positions is not None and tuple(positions.shape) != (B, S):
        raise ValueError("rope_qk_backward: positions must be [B, S]")
    _same_dtype("rope_qk_backward", ref.dtype, dq_in=dq_in, dq_out=dq_out, dk_in=dk_in, dk_out=dk_out)
    st = _lib.load().rope_qk_backward(
        _dev(dq_in), _dev(dq_out), _strides(dq_in, 3), _strides(dq_out, 3),
        _dev(dk_in), _dev(dk_out), _strides(dk_in, 3), _strides(dk_out, 3),
        _dtype(ref), B, S, Hq, Hkv, D, _i32(positions), float(rope_base), _pairing(rope_pairing),
        _stream())
    _check(st, "rope_qk_backward")


BWD_PIECES = 4   # LA_BWD_PIECES


def backward_workspace(B: int, S: int, Hkv: int, D: int, device=None):
    """The fp32 workspace gqa_attention_backward cuts long query ranges with."""
    return torch.empty((BWD_PIECES, B, S, Hkv, 2, D), dtype=torch.float32, device=device)


def gqa_attention_backward(q, k, v, o, dout, lse, dq, dk, dv, delta=None, cu_docs=None,
                           softmax_scale: float = 0.0, workspace="auto"):
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    n_docs = cu_docs.shape[-1] - 1 if cu_docs is not None else 1
    _same_shape("gqa_attention_backward", (q, o), (q, dout), (q, dq), (k, v), (k, dk), (k, dv))
    if tuple(k.shape) != (B, S, Hkv, D):
        raise ValueError("gqa_attention_backward: k/v must be [B, S, Hkv, D]")
    if tuple(lse.shape) != (B, Hq, S):
        raise ValueError("gqa_attention_backward: lse must be [B, Hq, S]")
    if delta is None:
        delta = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    if tuple(delta.shape) != (B, Hq, S):
        raise ValueError("gqa_attention_backward: delta must be [B, Hq, S]")
    if cu_docs is not None and (cu_docs.dim() != 2 or cu_docs.shape[0] != B):
        raise ValueError("gqa_attention_backward: cu_docs must be [B, n_docs + 1]")
    _same_dtype("gqa_attention_backward", torch.bfloat16, q=q, k=k, v=v, o=o, dout=dout, dq=dq, dk=dk, dv=dv)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("gqa_attention_backward: workspace must be a tensor, None or 'auto'")
        workspace = backward_workspace(B, S, Hkv, D, q.device)
    if workspace is not None and (workspace.numel() != BWD_PIECES * B * S * Hkv * 2 * D
                                  or workspace.dtype != torch.float32):
        raise ValueError("gqa_attention_backward: workspace must be fp32 with "
                         "BWD_PIECES*B*S*Hkv*2*D elements")
    st = _lib.load().gqa_attention_backward(
        _dev(q), _dev(k), _dev(v), _dev(o), _dev(dout), _f32c(lse), _f32c(delta),
        _dev(dq), _dev(dk), _dev(dv), _dtype(q), B, S, Hq, Hkv, D,
        _strides(q, 3), _strides(k, 3), _strides(v, 3), _strides(o, 3), _strides(dout, 3),
        _strides(dq, 3), _strides(dk, 3), _strides(dv, 3),
        _i32(cu_docs), n_docs, float(softmax_scale), _f32c(workspace), _stream())
    _check(st, "gqa_attention_backward")


def gqa_prefill(q, k, v, o, lse=None, cu_docs=None, softmax_scale: float = 0.0):
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    n_docs = cu_docs.shape[-1] - 1 if cu_docs is not None else 1
    _same_shape("gqa_prefill", (q, o), (k, v))
    if tuple(k.shape) != (B, S, Hkv, D):
        raise ValueError("gqa_prefill: k/v must be [B, S, Hkv, D]")
    if lse is not None and tuple(lse.shape) != (B, Hq, S):
        raise ValueError("gqa_prefill: lse must be [B, Hq, S]")
    if cu_docs is not None and (cu_docs.dim() != 2 or cu_docs.shape[0] != B):
        raise ValueError("gqa_prefill: cu_docs must be [B, n_docs + 1]")
    _same_dtype("gqa_prefill", q.dtype, k=k, v=v, o=o)
    st = _lib.load().gqa_prefill(
        _dev(q), _dev(k), _dev(v), _dev(o), _f32c(lse), _dtype(q), B, S, Hq, Hkv, D,
        _strides(q, 3), _strides(k, 3), _strides(v, 3), _strides(o, 3),
        _i32(cu_docs), n_docs, float(softmax_scale), _stream())
    _check(st, "gqa_prefill")


def gqa_prefill_rope(q, k, v, o, lse=None, cu_docs=None, softmax_scale: float = 0.0,
                     positions=None, rope_base: float = 500000.0, rope_pairing: str = "adjacent"):
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    n_docs = cu_docs.shape[-1] - 1 if cu_docs is not None else 1
    _same_shape("gqa_prefill_rope", (q, o), (k, v))
    if tuple(k.shape) != (B, S, Hkv, D):
        raise ValueError("gqa_prefill_rope: k/v must be [B, S, Hkv, D]")
    if lse is not None and tuple(lse.shape) != (B, Hq, S):
        raise ValueError("gqa_prefill_rope: lse must be [B, Hq, S]")
    if cu_docs is not None and (cu_docs.dim() != 2 or cu_docs.shape[0] != B):
        raise ValueError("gqa_prefill_rope: cu_docs must be [B, n_docs + 1]")
    if positions is not None and tuple(positions.shape) != (B, S):
        raise ValueError("gqa_prefill_rope: positions must be [B, S]")
    _same_dtype("gqa_prefill_rope", q.dtype, k=k, v=v, o=o)
    st = _lib.load().gqa_prefill_rope(
        _dev(q), _dev(k), _dev(v), _dev(o), _f32c(lse), _dtype(q), B, S, Hq, Hkv, D,
        _strides(q, 3), _strides(k, 3), _strides(v, 3), _strides(o, 3),
        _i32(cu_docs), n_docs, float(softmax_scale), _i32(positions), float(rope_base),
        _pairing(rope_pairing), _stream())
    _check(st, "gqa_prefill_rope")


def gqa_prefill_chunk(q, k, v, o, lse=None, cu_docs=None, softmax_scale: float = 0.0,
                      positions=None, rope_base: float = 0.0, rope_pairing: str = "adjacent"):
    B, Sq, Hq, D = q.shape
    S, Hkv = k.shape[1], k.shape[2]
    n_docs = cu_docs.shape[-1] - 1 if cu_docs is not None else 1
    _same_shape("gqa_prefill_chunk", (q, o), (k, v))
    if tuple(k.shape) != (B, S, Hkv, D):
        raise ValueError("gqa_prefill_chunk: k/v must be [B, S, Hkv, D]")
    if lse is not None and tuple(lse.shape) != (B, Hq, Sq):
        raise ValueError("gqa_prefill_chunk: lse must be [B, Hq, Sq]")
    if cu_docs is not None and (cu_docs.dim() != 2 or cu_docs.shape[0] != B):
        raise ValueError("gqa_prefill_chunk: cu_docs must be [B, n_docs + 1]")
    if positions is not None and tuple(positions.shape) != (B, Sq):
        raise ValueError("gqa_prefill_chunk: positions must be [B, Sq]")
    _same_dtype("gqa_prefill_chunk", q.dtype, k=k, v=v, o=o)
    st = _lib.load().gqa_prefill_chunk(
        _dev(q), _dev(k), _dev(v), _dev(o), _f32c(lse), _dtype(q), B, Sq, S, Hq, Hkv, D,
        _strides(q, 3), _strides(k, 3), _strides(v, 3), _strides(o, 3),
        _i32(cu_docs), n_docs, float(softmax_scale), _i32(positions), float(rope_base),
        _pairing(rope_pairing), _stream())
    _check(st, "gqa_prefill_chunk")


def prefill_split_workspace(B: int, Sq: int, S: int, Hq: int, D: int, split_tiles: int, device=None):
    """(o_part, lse_part) of the smallest max_splits gqa_prefill_split accepts."""
    max_splits = (-(-S // 64) + split_tiles - 1) // split_tiles
    o_part = torch.empty(max_splits, B, Sq, Hq, D, dtype=torch.float32, device=device)
    lse_part = torch.empty(max_splits, B, Hq, Sq, dtype=torch.float32, device=device)
    return o_part, lse_part


def gqa_prefill_split(q, k, v, o, split_tiles: int, o_part, lse_part, lse=None, cu_docs=None,
                      softmax_scale: float = 0.0, positions=None, rope_base: float = 0.0,
                      rope_pairing: str = "adjacent"):
    B, Sq, Hq, D = q.shape
    S, Hkv = k.shape[1], k.shape[2]
    n_docs = cu_docs.shape[-1] - 1 if cu_docs is not None else 1
    _same_shape("gqa_prefill_split", (q, o), (k, v))
    max_splits = o_part.shape[0]
    if tuple(k.shape) != (B, S, Hkv, D):
        raise ValueError("gqa_prefill_split: k/v must be [B, S, Hkv, D]")
    if lse is not None and tuple(lse.shape) != (B, Hq, Sq):
        raise ValueError("gqa_prefill_split: lse must be [B, Hq, Sq]")
    if cu_docs is not None and (cu_docs.dim() != 2 or cu_docs.shape[0] != B):
        raise ValueError("gqa_prefill_split: cu_docs must be [B, n_docs + 1]")
    if positions is not None and tuple(positions.shape) != (B, Sq):
        raise ValueError("gqa_prefill_split: positions must be [B, Sq]")
    _same_dtype("gqa_prefill_split", q.dtype, k=k, v=v, o=o)
    if tuple(o_part.shape) != (max_splits, B, Sq, Hq, D) or tuple(lse_part.shape) != (max_splits, B, Hq, Sq) \
            or o_part.dtype != torch.float32 or lse_part.dtype != torch.float32 \
            or not o_part.is_contiguous() or not lse_part.is_contiguous():
        raise ValueError("gqa_prefill_split: workspace must be contiguous fp32 [max_splits, B, Sq, Hq, D] "
                         "and [max_splits, B, Hq, Sq]")
    st = _lib.load().gqa_prefill_split(
        _dev(q), _dev(k), _dev(v), _dev(o), _f32c(lse), _dtype(q), B, Sq, S, Hq, Hkv, D,
        _strides(q, 3), _strides(k, 3), _strides(v, 3), _strides(o, 3),
        _i32(cu_docs), n_docs, float(softmax_scale), _i32(positions), float(rope_base),
        _pairing(rope_pairing), int(split_tiles), int(max_splits), _dev(o_part), _dev(lse_part),
        _stream())
    _check(st, "gqa_prefill_split")


def gqa_prefill_ring_step(q, k, v, q_off: int, k_off: int, o_acc, lse_acc, first: bool,
                          cu_docs=None, softmax_scale: float = 0.0, positions=None,
                          rope_base: float = 0.0, rope_pairing: str = "adjacent"):
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    n_docs = cu_docs.shape[-1] - 1 if cu_docs is not None else 1
    _same_shape("gqa_prefill_ring_step", (k, v))
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError("gqa_prefill_ring_step: k/v must be [B, Skv, Hkv, D]")
    if tuple(o_acc.shape) != (B, Sq, Hq, D) or tuple(lse_acc.shape) != (B, Hq, Sq) \
            or o_acc.dtype != torch.float32 or lse_acc.dtype != torch.float32 \
            or not o_acc.is_contiguous() or not lse_acc.is_contiguous():
        raise ValueError("gqa_prefill_ring_step: accumulators must be contiguous fp32 "
                         "[B, Sq, Hq, D] and [B, Hq, Sq]")
    if cu_docs is not None and (cu_docs.dim() != 2 or cu_docs.shape[0] != B):
        raise ValueError("gqa_prefill_ring_step: cu_docs must be [B, n_docs + 1]")
    if positions is not None and tuple(positions.shape) != (B, Sq):
        raise ValueError("gqa_prefill_ring_step: positions must be [B, Sq]")
    _same_dtype("gqa_prefill_ring_step", q.dtype, k=k, v=v)
    st = _lib.load().gqa_prefill_ring_step(
        _dev(q), _dev(k), _dev(v), _dev(o_acc), _dev(lse_acc), _dtype(q), B, Sq, int(q_off), Skv,
        int(k_off), Hq, Hkv, D, _strides(q, 3), _strides(k, 3), _strides(v, 3), _i32(cu_docs),
        n_docs, float(softmax_scale), _i32(positions), float(rope_base), _pairing(rope_pairing),
        int(bool(first)), _stream())
    _check(st, "gqa_prefill_ring_step")


def gqa_prefill_ring_step_final(q, k, v, q_off: int, k_off: int, o_acc, lse_acc, o, lse=None,
                                first: bool = False, cu_docs=None, softmax_scale: float = 0.0,
                                positions=None, rope_base: float = 0.0, rope_pairing: str = "adjacent"):
    """The last step of a query shard's ring: gqa_prefill_ring_step, then the
    final o (and lse) written directly instead of into the accumulators (as
    gqa_prefill_ring_finalize would write them). With first=True the
    accumulators are not used and may be None."""
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    n_docs = cu_docs.shape[-1] - 1 if cu_docs is not None else 1
    _same_shape("gqa_prefill_ring_step_final", (k, v), (q, o))
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError("gqa_prefill_ring_step_final: k/v must be [B, Skv, Hkv, D]")
    if not first:
        if o_acc is None or lse_acc is None or tuple(o_acc.shape) != (B, Sq, Hq, D) \
                or tuple(lse_acc.shape) != (B, Hq, Sq) or o_acc.dtype != torch.float32 \
                or lse_acc.dtype != torch.float32 or not o_acc.is_contiguous() \
                or not lse_acc.is_contiguous():
            raise ValueError("gqa_prefill_ring_step_final: accumulators must be contiguous fp32 "
                             "[B, Sq, Hq, D] and [B, Hq, Sq]")
    if lse is not None and tuple(lse.shape) != (B, Hq, Sq):
        raise ValueError("gqa_prefill_ring_step_final: lse must be [B, Hq, Sq]")
    if cu_docs is not None and (cu_docs.dim() != 2 or cu_docs.shape[0] != B):
        raise ValueError("gqa_prefill_ring_step_final: cu_docs must be [B, n_docs + 1]")
    if positions is not None and tuple(positions.shape) != (B, Sq):
        raise ValueError("gqa_prefill_ring_step_final: positions must be [B, Sq]")
    _same_dtype("gqa_prefill_ring_step_final", q.dtype, k=k, v=v, o=o)
    st = _lib.load().gqa_prefill_ring_step_final(
        _dev(q), _dev(k), _dev(v), None if first else _dev(o_acc), None if first else _dev(lse_acc),
        _dev(o), _strides(o, 3), _f32c(lse), _dtype(q), B, Sq, int(q_off), Skv, int(k_off), Hq, Hkv, D,
        _strides(q, 3), _strides(k, 3), _strides(v, 3), _i32(cu_docs), n_docs, float(softmax_scale),
        _i32(positions), float(rope_base), _pairing(rope_pairing), int(bool(first)), _stream())
    _check(st, "gqa_prefill_ring_step_final")


def gqa_prefill_ring_finalize(o_acc, lse_acc, o, lse=None):
    B, Sq, Hq, D = o.shape
    if tuple(o_acc.shape) != (B, Sq, Hq, D) or tuple(lse_acc.shape) != (B, Hq, Sq):
        raise ValueError("gqa_prefill_ring_finalize: inconsistent shapes")
    if lse is not None and tuple(lse.shape) != (B, Hq, Sq):
        raise ValueError("gqa_prefill_ring_finalize: lse must be [B, Hq, Sq]")
    st = _lib.load().gqa_prefill_ring_finalize(
        _f32c(o_acc), _f32c(lse_acc), _dev(o), _strides(o, 3), _f32c(lse), _dtype(o), B, Sq, Hq, D,
        _stream())
    _check(st, "gqa_prefill_ring_finalize")


def default_kv_chunk() -> int:
    """The decode's keys per split when a call passes kv_chunk=None: the
    LLAMA_ATTN_KV_CHUNK environment variable if set, else 256."""
    v = os.environ.get("LLAMA_ATTN_KV_CHUNK")
    kv = int(v) if v else 256
    if kv < 1:
        raise ValueError("LLAMA_ATTN_KV_CHUNK must be a positive integer")
    return kv


def _kv_chunk(kv_chunk):
    return default_kv_chunk() if kv_chunk is None else int(kv_chunk)


def gqa_decode(q, k_cache, v_cache, seq_lens, kv_chunk: int, o_part, lse_part,
               softmax_scale: float = 0.0):
    B, Hq, D = q.shape
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    if k_cache.stride() != v_cache.stride():
        raise ValueError("k_cache and v_cache must share strides")
    max_splits = o_part.shape[2]
    _same_shape("gqa_decode", (k_cache, v_cache))
    if k_cache.shape[0] != B or k_cache.shape[3] != D or tuple(o_part.shape) != (B, Hq, max_splits, D) \
            or tuple(lse_part.shape) != (B, Hq, max_splits) or tuple(seq_lens.shape) != (B,):
        raise ValueError("gqa_decode: inconsistent shapes")
    _same_dtype("gqa_decode", torch.bfloat16, q=q, k_cache=k_cache, v_cache=v_cache)
    op, lp = _f32c(o_part), _f32c(lse_part)
    st = _lib.load().gqa_decode(
        _dev(q), _strides(q, 2), _dev(k_cache), _dev(v_cache), _strides(k_cache, 3),
        _i32(seq_lens), B, Hq, Hkv, D, Lmax, _kv_chunk(kv_chunk), max_splits, float(softmax_scale),
        op, lp, _stream())
    _check(st, "gqa_decode")


def gqa_decode_paged(q, k_pages, v_pages, block_table, seq_lens, kv_chunk: int, o_part, lse_part,
                     Lmax: int, softmax_scale: float = 0.0):
    B, Hq, D = q.shape
    n_pages, page_size, Hkv, Dk = k_pages.shape
    if k_pages.stride() != v_pages.stride() or tuple(k_pages.shape) != tuple(v_pages.shape):
        raise ValueError("gqa_decode_paged: k_pages and v_pages must share shape and strides")
    max_splits = o_part.shape[2]
    if Dk != D or tuple(o_part.shape) != (B, Hq, max_splits, D) \
            or tuple(lse_part.shape) != (B, Hq, max_splits) or tuple(seq_lens.shape) != (B,) \
            or block_table.dim() != 2 or block_table.shape[0] != B or block_table.stride(1) != 1:
        raise ValueError("gqa_decode_paged: inconsistent shapes")
    _same_dtype("gqa_decode_paged", torch.bfloat16, q=q, k_pages=k_pages, v_pages=v_pages)
    op, lp = _f32c(o_part), _f32c(lse_part)
    ps = k_pages.stride()
    if ps[-1] != 1:
        raise ValueError("the last (head_dim) dimension must be contiguous")
    page_strides = _lib.i64_array((ps[0], ps[2], ps[1]))   # (page, head, slot)
    st = _lib.load().gqa_decode_paged(
        _dev(q), _strides(q, 2), _dev(k_pages), _dev(v_pages), page_strides, page_size,
        _i32(block_table), block_table.stride(0), _i32(seq_lens), B, Hq, Hkv, D, int(Lmax),
        _kv_chunk(kv_chunk), max_splits, float(softmax_scale), op, lp, _stream())
    _check(st, "gqa_decode_paged")


def gqa_decode_combine(o_part, lse_part, seq_lens, kv_chunk: int, o, lse=None):
    B, Hq, max_splits, D = o_part.shape
    if tuple(lse_part.shape) != (B, Hq, max_splits) or tuple(o.shape) != (B, Hq, D) \
            or tuple(seq_lens.shape) != (B,) or (lse is not None and tuple(lse.shape) != (B, Hq)):
        raise ValueError("gqa_decode_combine: inconsistent shapes")
    st = _lib.load().gqa_decode_combine(
        _f32c(o_part), _f32c(lse_part), _i32(seq_lens), B, Hq, D, _kv_chunk(kv_chunk), max_splits,
        _dev(o), _strides(o, 2), _f32c(lse), _dtype(o), _stream())
    _check(st, "gqa_decode_combine")


def gqa_decode_noalloc(q, k_cache, v_cache, seq_lens, kv_chunk: int, o, lse=None,
                       softmax_scale: float = 0.0):
    B, Hq, D = q.shape
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    if k_cache.stride() != v_cache.stride():
        raise ValueError("k_cache and v_cache must share strides")
    _same_shape("gqa_decode_noalloc", (k_cache, v_cache))
    if k_cache.shape[0] != B or k_cache.shape[3] != D or tuple(seq_lens.shape) != (B,) \
            or tuple(o.shape) != (B, Hq, D) or (lse is not None and tuple(lse.shape) != (B, Hq)):
        raise ValueError("gqa_decode_noalloc: inconsistent shapes")
    _same_dtype("gqa_decode_noalloc", torch.bfloat16, q=q, k_cache=k_cache, v_cache=v_cache)
    lp = _f32c(lse)
    st = _lib.load().gqa_decode_noalloc(
        _dev(q), _strides(q, 2), _dev(k_cache), _dev(v_cache), _strides(k_cache, 3), _i32(seq_lens),
        B, Hq, Hkv, D, Lmax, _kv_chunk(kv_chunk), float(softmax_scale), _dev(o), _strides(o, 2), lp,
        _dtype(o), _stream())
    _check(st, "gqa_decode_noalloc")
