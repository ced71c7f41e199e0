"""Tensor-level wrappers over the C ABI (argument checking and marshalling only).

Each function validates shapes, dtypes, devices and contiguity of torch
tensors, fills the parameter struct and calls the library entry point of the
same name on the given stream (default: the current stream of the tensors'
device), with the tensors' device current.  No arithmetic of the method
happens here.
"""
from __future__ import annotations

import torch

from . import dcp as _abi


def _stream(stream, device: torch.device) -> int:
    """The raw hipStream_t: the given stream, or the current stream of the
    tensors' device."""
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        if stream.device != device:
            raise ValueError(f"stream is on {stream.device}, tensors on {device}")
        return stream.cuda_stream
    return int(stream)


def _one_device(*tensors) -> torch.device:
    """The single device of the call's tensors (None entries are skipped)."""
    devs = {t.device for t in tensors if t is not None}
    if len(devs) != 1:
        raise ValueError(f"all tensors must be on one device, got {sorted(str(d) for d in devs)}")
    return devs.pop()


def _req(t: torch.Tensor, dtype, ndim: int, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a HIP device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _req_ws(ws: torch.Tensor, *tensors) -> torch.device:
    """The workspace: a contiguous device tensor on the same device as the
    call's other tensors (its byte size is checked by the library).  Returns
    that device."""
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on a HIP device")
    return _one_device(ws, *tensors)


def mla_params(*, batch, num_heads, block_size, max_blocks_per_seq, num_blocks, shard_rank, num_shards,
               layout, max_seq_len_hint, softmax_scale, kv_lora_rank=512, rope_dim=64,
               q_len=1) -> _abi.dcp_mla_params:
    return _abi.dcp_mla_params(batch, num_heads, kv_lora_rank, rope_dim, block_size, max_blocks_per_seq,
                               num_blocks, shard_rank, num_shards, layout, max_seq_len_hint, softmax_scale, q_len)


def gqa_params(*, batch, num_q_heads, num_kv_heads, block_size, max_blocks_per_seq, num_blocks, shard_rank,
               num_shards, layout, max_seq_len_hint, softmax_scale, head_dim=128, q_len=1) -> _abi.dcp_gqa_params:
    return _abi.dcp_gqa_params(batch, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                               num_blocks, shard_rank, num_shards, layout, max_seq_len_hint, softmax_scale, q_len)


def _rows(p) -> int:
    """Row sets of a step: requests times query tokens (q, out and lse are
    [batch * q_len, heads, ...], request-major)."""
    return p.batch * max(1, p.q_len)


def mla_workspace(p: _abi.dcp_mla_params, device) -> torch.Tensor:
    n = _abi.dcp_mla_workspace_bytes(p)
    if n == 0:
        raise _abi.DcpError(_abi.DCP_ERR_INVALID_ARGUMENT, "dcp_mla_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def gqa_workspace(p: _abi.dcp_gqa_params, device) -> torch.Tensor:
    n = _abi.dcp_gqa_workspace_bytes(p)
    if n == 0:
        raise _abi.DcpError(_abi.DCP_ERR_INVALID_ARGUMENT, "dcp_gqa_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _mla_check(p, q, kv_cache, kv_dtypes, block_table, seq_lens, out, lse):
    _req(q, torch.bfloat16, 3, "q")
    if kv_cache.dtype not in kv_dtypes:
        raise TypeError(f"kv_cache: expected one of {kv_dtypes}, got {kv_cache.dtype}")
    _req(kv_cache, kv_cache.dtype, 3, "kv_cache")
    _req(block_table, torch.int32, 2, "block_table")
    _req(seq_lens, torch.int32, 1, "seq_lens")
    _req(out, torch.float32, 3, "out")
    _req(lse, torch.float32, 2, "lse")
    dk = p.kv_lora_rank + p.rope_dim
    if tuple(q.shape) != (_rows(p), p.num_heads, dk):
        raise ValueError(f"q shape {tuple(q.shape)} != {(_rows(p), p.num_heads, dk)}")
    if tuple(kv_cache.shape) != (p.num_blocks, p.block_size, dk):
        raise ValueError(f"kv_cache shape {tuple(kv_cache.shape)} != {(p.num_blocks, p.block_size, dk)}")
    if tuple(block_table.shape) != (p.batch, p.max_blocks_per_seq):
        raise ValueError(f"block_table shape {tuple(block_table.shape)}")
    if tuple(seq_lens.shape) != (p.batch,):
        raise ValueError("seq_lens shape")
    if tuple(out.shape) != (_rows(p), p.num_heads, p.kv_lora_rank) or tuple(lse.shape) != (_rows(p), p.num_heads):
        raise ValueError("out/lse shape")


def dcp_mla_decode_partial(p, q, kv_cache, block_table, seq_lens, out, lse, workspace, stream=None) -> None:
    _mla_check(p, q, kv_cache, (torch.bfloat16,), block_table, seq_lens, out, lse)
    dev = _req_ws(workspace, q, kv_cache, block_table, seq_lens, out, lse)
    with torch.cuda.device(dev):
        _abi.check(_abi.dcp_mla_decode_partial(p, q.data_ptr(), kv_cache.data_ptr(), block_table.data_ptr(),
                                               seq_lens.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                               workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                               _stream(stream, dev)), "dcp_mla_decode_partial")


def dcp_mla_decode_partial_noalloc(p, q, kv_cache, block_table, seq_lens, out, lse, stream=None) -> None:
    """dcp_mla_decode_partial with the library's fixed device scratch as the
    split workspace (nothing is allocated)."""
    _mla_check(p, q, kv_cache, (torch.bfloat16,), block_table, seq_lens, out, lse)
    dev = _one_device(q, kv_cache, block_table, seq_lens, out, lse)
    with torch.cuda.device(dev):
        _abi.check(_abi.dcp_mla_decode_partial_noalloc(p, q.data_ptr(), kv_cache.data_ptr(), block_table.data_ptr(),
                                                       seq_lens.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                                       _stream(stream, dev)), "dcp_mla_decode_partial_noalloc")


def dcp_mla_decode_partial_fp8(p, q, kv_cache, kv_scale, block_table, seq_lens, out, lse, workspace,
                               stream=None) -> None:
    """MLA partial over an fp8 cache: kv_cache holds E4M3 codes (torch.float8_e4m3fn
    or uint8) [num_blocks, block_size, 576]; kv_scale dequantizes the whole cache."""
    _mla_check(p, q, kv_cache, (torch.float8_e4m3fn, torch.uint8), block_table, seq_lens, out, lse)
    dev = _req_ws(workspace, q, kv_cache, block_table, seq_lens, out, lse)
    with torch.cuda.device(dev):
        _abi.check(_abi.dcp_mla_decode_partial_fp8(p, q.data_ptr(), kv_cache.data_ptr(), float(kv_scale),
                                                   block_table.data_ptr(), seq_lens.data_ptr(), out.data_ptr(),
                                                   lse.data_ptr(), workspace.data_ptr(),
                                                   workspace.numel() * workspace.element_size(),
                                                   _stream(stream, dev)), "dcp_mla_decode_partial_fp8")


def dcp_gqa_decode_partial(p, q, k_cache, v_cache, block_table, seq_lens, out, lse, workspace,
                           stream=None) -> None:
    _req(q, torch.bfloat16, 3, "q")
    _req(k_cache, torch.bfloat16, 4, "k_cache")
    _req(v_cache, torch.bfloat16, 4, "v_cache")
    _req(block_table, torch.int32, 2, "block_table")
    _req(seq_lens, torch.int32, 1, "seq_lens")
    _req(out, torch.float32, 3, "out")
    _req(lse, torch.float32, 2, "lse")
    if tuple(q.shape) != (_rows(p), p.num_q_heads, p.head_dim):
        raise ValueError("q shape")
    kshape = (p.num_blocks, p.block_size, p.num_kv_heads, p.head_dim)
    if tuple(k_cache.shape) != kshape or tuple(v_cache.shape) != kshape:
        raise ValueError(f"k/v cache shape must be {kshape}")
    if tuple(block_table.shape) != (p.batch, p.max_blocks_per_seq) or tuple(seq_lens.shape) != (p.batch,):
        raise ValueError("block_table / seq_lens shape")
    if tuple(out.shape) != (_rows(p), p.num_q_heads, p.head_dim) or tuple(lse.shape) != (_rows(p), p.num_q_heads):
        raise ValueError("out/lse shape")
    dev = _req_ws(workspace, q, k_cache, v_cache, block_table, seq_lens, out, lse)
    with torch.cuda.device(dev):
        _abi.check(_abi.dcp_gqa_decode_partial(p, q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                               block_table.data_ptr(), seq_lens.data_ptr(), out.data_ptr(),
                                               lse.data_ptr(), workspace.data_ptr(),
                                               workspace.numel() * workspace.element_size(),
                                               _stream(stream, dev)), "dcp_gqa_decode_partial")


def dcp_combine(partial_out, partial_lse, out_bf16=None, out_f32=None, lse_out=None, stream=None) -> None:
    _req(partial_out, torch.float32, 4, "partial_out")
    _req(partial_lse, torch.float32, 3, "partial_lse")
    n, b, h, dv = partial_out.shape
    if tuple(partial_lse.shape) != (n, b, h):
        raise ValueError("partial_lse shape")
    if out_bf16 is not None:
        _req(out_bf16, torch.bfloat16, 3, "out_bf16")
        if tuple(out_bf16.shape) != (b, h, dv):
            raise ValueError("out_bf16 shape")
    if out_f32 is not None:
        _req(out_f32, torch.float32, 3, "out_f32")
        if tuple(out_f32.shape) != (b, h, dv):
            raise ValueError("out_f32 shape")
    if lse_out is not None:
        _req(lse_out, torch.float32, 2, "lse_out")
        if tuple(lse_out.shape) != (b, h):
            raise ValueError("lse_out shape")
    dev = _one_device(partial_out, partial_lse, out_bf16, out_f32, lse_out)
    ptr = lambda t: 0 if t is None else t.data_ptr()  # noqa: E731
    with torch.cuda.device(dev):
        _abi.check(_abi.dcp_combine(n, b, h, dv, partial_out.data_ptr(), partial_lse.data_ptr(), ptr(out_bf16),
                                    ptr(out_f32), ptr(lse_out), _stream(stream, dev)), "dcp_combine")


def dcp_combine_vproj_gate(partial_out, partial_lse, w_uv_t, gate=None, out_bf16=None, out_f32=None,
                           lse_out=None, stream=None) -> None:
    """Merge + per-head value up-projection + sigmoid gate (include/dcp.h).

    partial_out fp32 [N, b, H, Dv], partial_lse fp32 [N, b, H], w_uv_t bf16
    [H, Dvo, Dv], gate bf16 [b, H, Dvo] or None; outputs [b, H, Dvo]."""
    _req(partial_out, torch.float32, 4, "partial_out")
    _req(partial_lse, torch.float32, 3, "partial_lse")
    _req(w_uv_t, torch.bfloat16, 3, "w_uv_t")
    n, b, h, dv = partial_out.shape
    if tuple(partial_lse.shape) != (n, b, h):
        raise ValueError("partial_lse shape")
    if w_uv_t.shape[0] != h or w_uv_t.shape[2] != dv:
        raise ValueError("w_uv_t shape")
    dvo = w_uv_t.shape[1]
    if gate is not None:
        _req(gate, torch.bfloat16, 3, "gate")
        if tuple(gate.shape) != (b, h, dvo):
            raise ValueError("gate shape")
    for name, t, dt in (("out_bf16", out_bf16, torch.bfloat16), ("out_f32", out_f32, torch.float32)):
        if t is not None:
            _req(t, dt, 3, name)
            if tuple(t.shape) != (b, h, dvo):
                raise ValueError(f"{name} shape")
    if lse_out is not None:
        _req(lse_out, torch.float32, 2, "lse_out")
        if tuple(lse_out.shape) != (b, h):
            raise ValueError("lse_out shape")
    dev = _one_device(partial_out, partial_lse, w_uv_t, gate, out_bf16, out_f32, lse_out)
    ptr = lambda t: 0 if t is None else t.data_ptr()  # noqa: E731
    with torch.cuda.device(dev):
        _abi.check(_abi.dcp_combine_vproj_gate(n, b, h, dv, dvo, partial_out.data_ptr(), partial_lse.data_ptr(),
                                               w_uv_t.data_ptr(), ptr(gate), ptr(out_bf16), ptr(out_f32),
                                               ptr(lse_out), _stream(stream, dev)), "dcp_combine_vproj_gate")
