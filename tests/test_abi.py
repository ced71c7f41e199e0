"""The C-ABI library loads on the CPU, exports every declared symbol, and
rejects bad arguments on the host before touching a device."""
import ctypes
import os
import re

import pytest

from kv_cache_context_amd import dcp, ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "dcp.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dcp_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    lib = dcp.lib()
    names = declared_functions()
    assert set(names) == set(dcp.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n
    assert dcp.dcp_abi_version() == 3


def test_struct_layout_matches_header():
    # 11 int32 fields + 1 float + q_len, no padding; q_len last
    assert ctypes.sizeof(dcp.dcp_mla_params) == 52
    assert ctypes.sizeof(dcp.dcp_gqa_params) == 52
    assert dcp.dcp_mla_params.q_len.offset == 48 and dcp.dcp_gqa_params.q_len.offset == 48


def test_workspace_grows_with_query_tokens():
    one = dcp.dcp_mla_workspace_bytes(mla(batch=8))
    assert dcp.dcp_mla_workspace_bytes(mla(batch=8, q_len=0)) == one   # 0 means 1
    assert dcp.dcp_mla_workspace_bytes(mla(batch=8, q_len=4)) == dcp.dcp_mla_workspace_bytes(mla(batch=32))
    assert dcp.dcp_gqa_workspace_bytes(gqa(batch=4, q_len=2)) == dcp.dcp_gqa_workspace_bytes(gqa(batch=8))


def test_status_strings():
    assert dcp.status_string(0) == "ok"
    assert "workspace" in dcp.status_string(3)
    assert "scratch" in dcp.status_string(5)
    assert dcp.status_string(99) == "unknown status"


def mla(**kw):
    base = dict(batch=2, num_heads=64, block_size=64, max_blocks_per_seq=16, num_blocks=64, shard_rank=1,
                num_shards=8, layout=0, max_seq_len_hint=8192, softmax_scale=0.072)
    base.update(kw)
    return ops.mla_params(**base)


def gqa(**kw):
    base = dict(batch=2, num_q_heads=64, num_kv_heads=8, block_size=16, max_blocks_per_seq=64, num_blocks=200,
                shard_rank=1, num_shards=4, layout=0, max_seq_len_hint=4096, softmax_scale=0.088)
    base.update(kw)
    return ops.gqa_params(**base)


FAKE = 1 << 20  # an aligned non-null address; never dereferenced (validation fails first)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=-1), 1), (dict(num_shards=0), 1), (dict(shard_rank=8), 1), (dict(shard_rank=-1), 1),
    (dict(layout=7), 1), (dict(block_size=0), 1), (dict(num_blocks=0), 1), (dict(max_seq_len_hint=0), 1),
    (dict(softmax_scale=0.0), 1), (dict(softmax_scale=float("inf")), 1), (dict(softmax_scale=float("nan")), 1),
    (dict(num_heads=0), 1), (dict(max_seq_len_hint=8 * 16 * 64 + 1), 1),
    (dict(num_heads=17), 2), (dict(num_heads=128), 2), (dict(block_size=8), 2), (dict(block_size=2048), 2),
    (dict(kv_lora_rank=256), 2), (dict(rope_dim=32), 2), (dict(batch=4096), 2),
    (dict(q_len=-1), 1), (dict(q_len=17), 2), (dict(batch=1024, q_len=3), 2),
])
def test_mla_validation(kw, status):
    p = mla(**kw)
    assert dcp.dcp_mla_decode_partial(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, 0) == status
    assert dcp.dcp_mla_workspace_bytes(p) == 0


def test_mla_pointer_and_workspace_checks():
    p = mla()
    need = dcp.dcp_mla_workspace_bytes(p)
    assert need > 0
    assert dcp.dcp_mla_decode_partial(p, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, 0) == 1
    assert dcp.dcp_mla_decode_partial(p, FAKE + 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, 0) == 1
    assert dcp.dcp_mla_decode_partial(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, 0) == 3
    assert dcp.dcp_mla_decode_partial(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, need, 0) == 3
    assert dcp.dcp_mla_decode_partial(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 16, need, 0) == 3
    # batch 0 is a no-op even with null pointers
    assert dcp.dcp_mla_decode_partial(mla(batch=0), 0, 0, 0, 0, 0, 0, 0, 0, 0) == 0
    # workspace grows with batch and heads only
    assert dcp.dcp_mla_workspace_bytes(mla(batch=4)) > need
    assert dcp.dcp_mla_workspace_bytes(mla(max_seq_len_hint=100)) == need


def test_mla_noalloc_validation():
    """The no-allocation entry point validates like dcp_mla_decode_partial
    before it looks at the device (no GPU here: a valid call would need one)."""
    f = dcp.dcp_mla_decode_partial_noalloc
    assert f(mla(num_shards=0), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0) == 1
    assert f(mla(num_heads=17), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0) == 2
    assert f(mla(), 0, FAKE, FAKE, FAKE, FAKE, FAKE, 0) == 1
    assert f(mla(), FAKE, FAKE + 2, FAKE, FAKE, FAKE, FAKE, 0) == 1
    assert f(mla(batch=0), 0, 0, 0, 0, 0, 0, 0) == 0


def test_mla_fp8_validation():
    """The fp8 entry point checks its scale first, then everything the bf16 one does."""
    p = mla()
    need = dcp.dcp_mla_workspace_bytes(p)
    f = dcp.dcp_mla_decode_partial_fp8
    for bad in (0.0, -1.0, float("nan"), float("inf"), 1e-38):
        assert f(p, FAKE, FAKE, bad, FAKE, FAKE, FAKE, FAKE, FAKE, need, 0) == 1, bad
    assert f(mla(num_heads=60), FAKE, FAKE, 0.5, FAKE, FAKE, FAKE, FAKE, FAKE, need, 0) == 2
    assert f(p, FAKE, 0, 0.5, FAKE, FAKE, FAKE, FAKE, FAKE, need, 0) == 1
    assert f(p, FAKE, FAKE + 8, 0.5, FAKE, FAKE, FAKE, FAKE, FAKE, need, 0) == 1   # misaligned cache
    assert f(p, FAKE, FAKE, 0.5, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, 0) == 3
    assert f(mla(batch=0), 0, 0, 0.5, 0, 0, 0, 0, 0, 0, 0) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(num_q_heads=60), 1), (dict(num_kv_heads=0), 1), (dict(shard_rank=4), 1), (dict(batch=-3), 1),
    (dict(head_dim=64), 2), (dict(num_q_heads=128, num_kv_heads=1), 2), (dict(num_q_heads=128, num_kv_heads=128), 2),
    (dict(num_q_heads=1024, num_kv_heads=8), 2),
    (dict(block_size=24), 2), (dict(max_seq_len_hint=4 * 64 * 16 + 1), 1),
])
def test_gqa_validation(kw, status):
    p = gqa(**kw)
    assert dcp.dcp_gqa_decode_partial(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, 0) == status


def test_combine_validation():
    c = dcp.dcp_combine
    assert c(0, 1, 1, 512, FAKE, FAKE, FAKE, 0, 0, 0) == 1
    assert c(65, 1, 1, 512, FAKE, FAKE, FAKE, 0, 0, 0) == 2
    assert c(8, 1, 1, 510, FAKE, FAKE, FAKE, 0, 0, 0) == 2
    assert c(8, 1, 1, 2048, FAKE, FAKE, FAKE, 0, 0, 0) == 2
    assert c(8, 1, 1, 512, FAKE, FAKE, 0, 0, 0, 0) == 1          # no output at all
    assert c(8, 1, 1, 512, 0, FAKE, FAKE, 0, 0, 0) == 1
    assert c(8, 1, 1, 512, FAKE + 4, FAKE, FAKE, 0, 0, 0) == 1   # misaligned partials
    assert c(8, 0, 64, 512, 0, 0, 0, 0, 0, 0) == 0               # empty batch: no-op


def test_combine_vproj_gate_validation():
    c = dcp.dcp_combine_vproj_gate
    ok = (FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0, 0)  # partials, lse, w, gate, out_bf16, out_f32, lse_out, stream
    assert c(0, 1, 1, 512, 128, *ok) == 1
    assert c(65, 1, 1, 512, 128, *ok) == 2
    assert c(8, 1, 1, 500, 128, *ok) == 2           # latent width not a multiple of 32
    assert c(8, 1, 1, 2048, 128, *ok) == 2
    assert c(8, 1, 1, 512, 120, *ok) == 2           # output width not a multiple of 16
    assert c(8, 1, 1, 512, 272, *ok) == 2
    assert c(8, 1, 1, 512, 0, *ok) == 1
    assert c(8, 1, 70000, 512, 128, *ok) == 2
    assert c(8, 1, 1, 512, 128, FAKE, FAKE, 0, FAKE, FAKE, 0, 0, 0) == 1       # no projection
    assert c(8, 1, 1, 512, 128, FAKE, FAKE, FAKE, FAKE, 0, 0, 0, 0) == 1       # no output at all
    assert c(8, 1, 1, 512, 128, FAKE, FAKE, FAKE + 8, FAKE, FAKE, 0, 0, 0) == 1  # misaligned projection
    assert c(8, 1, 1, 512, 128, FAKE, FAKE, FAKE, FAKE + 1, FAKE, 0, 0, 0) == 1  # misaligned gate
    assert c(8, 0, 64, 512, 128, 0, 0, 0, 0, 0, 0, 0, 0) == 0                  # empty batch: no-op


def test_ops_reject_cpu_tensors():
    import torch
    p = mla(batch=1)
    t = torch.zeros((1, 64, 576), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ops.dcp_mla_decode_partial(p, t, t, t, t, t, t, t)


def test_ops_one_device():
    import torch
    a = torch.zeros(1)
    assert ops._one_device(a, None, torch.ones(2)) == torch.device("cpu")
    with pytest.raises(ValueError):
        ops._one_device(a, torch.zeros(1, device="meta"))
