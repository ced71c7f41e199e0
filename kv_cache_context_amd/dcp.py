"""ctypes binding of libdcp.so (include/dcp.h), same names as the C ABI.

Argument marshalling only: pointers are passed as integers (device addresses,
e.g. ``tensor.data_ptr()``), streams as the raw ``hipStream_t`` value (e.g.
``torch.cuda.current_stream().cuda_stream``).  Every step of the computation
runs in the HIP kernels of the library; there is no fallback.  If the library
is missing, loading fails with an error that says how to build it.

torch is imported first on purpose: its bundled HIP runtime then serves this
library too (both use the soname libamdhip64.so.7), so streams and device
pointers from torch are valid here.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime this library links against)

LIB_PATH = os.environ.get("DCP_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdcp.so")

DCP_OK = 0
DCP_ERR_INVALID_ARGUMENT = 1
DCP_ERR_UNSUPPORTED = 2
DCP_ERR_WORKSPACE = 3
DCP_ERR_HIP = 4
DCP_ERR_SCRATCH = 5
DCP_NOALLOC_SCRATCH_BYTES = 32 << 20
DCP_LAYOUT_ROUND_ROBIN = 0
DCP_LAYOUT_CONTIGUOUS = 1

# every symbol the header declares
EXPORTED = (
    "dcp_mla_workspace_bytes", "dcp_mla_decode_partial", "dcp_mla_decode_partial_fp8",
    "dcp_mla_decode_partial_noalloc",
    "dcp_gqa_workspace_bytes", "dcp_gqa_decode_partial",
    "dcp_combine", "dcp_combine_vproj_gate", "dcp_status_string", "dcp_last_hip_error", "dcp_abi_version",
)


class dcp_mla_params(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32),
        ("kv_lora_rank", ctypes.c_int32), ("rope_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32), ("shard_rank", ctypes.c_int32),
        ("num_shards", ctypes.c_int32), ("layout", ctypes.c_int32),
        ("max_seq_len_hint", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("q_len", ctypes.c_int32),
    ]


class dcp_gqa_params(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32), ("shard_rank", ctypes.c_int32),
        ("num_shards", ctypes.c_int32), ("layout", ctypes.c_int32),
        ("max_seq_len_hint", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("q_len", ctypes.c_int32),
    ]


class DcpError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = status_string(status)
        if status == DCP_ERR_HIP:
            msg += f" (hipError_t {dcp_last_hip_error()})"
        super().__init__(f"{what}: {msg}" if what else msg)


_lib = None
_P = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    """Load libdcp.so once and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m kv_cache_context_amd.build` "
                          "or __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    L.dcp_mla_workspace_bytes.argtypes = [ctypes.POINTER(dcp_mla_params)]
    L.dcp_mla_workspace_bytes.restype = ctypes.c_size_t
    L.dcp_mla_decode_partial.argtypes = [ctypes.POINTER(dcp_mla_params), _P, _P, _P, _P, _P, _P, _P,
                                         ctypes.c_size_t, _P]
    L.dcp_mla_decode_partial.restype = ctypes.c_int
    L.dcp_mla_decode_partial_fp8.argtypes = [ctypes.POINTER(dcp_mla_params), _P, _P, ctypes.c_float, _P, _P, _P,
                                             _P, _P, ctypes.c_size_t, _P]
    L.dcp_mla_decode_partial_fp8.restype = ctypes.c_int
    L.dcp_mla_decode_partial_noalloc.argtypes = [ctypes.POINTER(dcp_mla_params), _P, _P, _P, _P, _P, _P, _P]
    L.dcp_mla_decode_partial_noalloc.restype = ctypes.c_int
    L.dcp_gqa_workspace_bytes.argtypes = [ctypes.POINTER(dcp_gqa_params)]
    L.dcp_gqa_workspace_bytes.restype = ctypes.c_size_t
    L.dcp_gqa_decode_partial.argtypes = [ctypes.POINTER(dcp_gqa_params), _P, _P, _P, _P, _P, _P, _P, _P,
                                         ctypes.c_size_t, _P]
    L.dcp_gqa_decode_partial.restype = ctypes.c_int
    L.dcp_combine.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                              _P, _P, _P, _P, _P, _P]
    L.dcp_combine.restype = ctypes.c_int
    L.dcp_combine_vproj_gate.argtypes = [ctypes.c_int32] * 5 + [_P] * 8
    L.dcp_combine_vproj_gate.restype = ctypes.c_int
    L.dcp_status_string.argtypes = [ctypes.c_int]
    L.dcp_status_string.restype = ctypes.c_char_p
    L.dcp_last_hip_error.argtypes = []
    L.dcp_last_hip_error.restype = ctypes.c_int
    L.dcp_abi_version.argtypes = []
    L.dcp_abi_version.restype = ctypes.c_int
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().dcp_status_string(int(status)).decode()


def dcp_status_string(status: int) -> str:
    return status_string(status)


def dcp_last_hip_error() -> int:
    return int(lib().dcp_last_hip_error())


def dcp_abi_version() -> int:
    return int(lib().dcp_abi_version())


def dcp_mla_workspace_bytes(p: dcp_mla_params) -> int:
    return int(lib().dcp_mla_workspace_bytes(ctypes.byref(p)))


def dcp_gqa_workspace_bytes(p: dcp_gqa_params) -> int:
    return int(lib().dcp_gqa_workspace_bytes(ctypes.byref(p)))


def dcp_mla_decode_partial(p: dcp_mla_params, q: int, kv_cache: int, block_table: int, seq_lens: int,
                           out: int, lse: int, workspace: int, workspace_bytes: int, stream: int) -> int:
    return int(lib().dcp_mla_decode_partial(ctypes.byref(p), q, kv_cache, block_table, seq_lens, out, lse,
                                            workspace, workspace_bytes, stream))


def dcp_mla_decode_partial_fp8(p: dcp_mla_params, q: int, kv_cache: int, kv_scale: float, block_table: int,
                               seq_lens: int, out: int, lse: int, workspace: int, workspace_bytes: int,
                               stream: int) -> int:
    return int(lib().dcp_mla_decode_partial_fp8(ctypes.byref(p), q, kv_cache, kv_scale, block_table, seq_lens,
                                                out, lse, workspace, workspace_bytes, stream))


def dcp_mla_decode_partial_noalloc(p: dcp_mla_params, q: int, kv_cache: int, block_table: int, seq_lens: int,
                                   out: int, lse: int, stream: int) -> int:
    return int(lib().dcp_mla_decode_partial_noalloc(ctypes.byref(p), q, kv_cache, block_table, seq_lens, out, lse,
                                                    stream))


def dcp_gqa_decode_partial(p: dcp_gqa_params, q: int, k_cache: int, v_cache: int, block_table: int,
                           seq_lens: int, out: int, lse: int, workspace: int, workspace_bytes: int,
                           stream: int) -> int:
    return int(lib().dcp_gqa_decode_partial(ctypes.byref(p), q, k_cache, v_cache, block_table, seq_lens,
                                            out, lse, workspace, workspace_bytes, stream))


def dcp_combine(num_shards: int, batch: int, num_heads: int, head_dim_v: int, partial_out: int,
                partial_lse: int, out_bf16: int, out_f32: int, lse_out: int, stream: int) -> int:
    return int(lib().dcp_combine(num_shards, batch, num_heads, head_dim_v, partial_out, partial_lse,
                                 out_bf16, out_f32, lse_out, stream))


def dcp_combine_vproj_gate(num_shards: int, batch: int, num_heads: int, head_dim_v: int, out_dim: int,
                           partial_out: int, partial_lse: int, w_uv_t: int, gate: int, out_bf16: int,
                           out_f32: int, lse_out: int, stream: int) -> int:
    return int(lib().dcp_combine_vproj_gate(num_shards, batch, num_heads, head_dim_v, out_dim, partial_out,
                                            partial_lse, w_uv_t, gate, out_bf16, out_f32, lse_out, stream))


def check(status: int, what: str = "") -> None:
    """Raise DcpError unless status is DCP_OK."""
    if status != DCP_OK:
        raise DcpError(status, what)
