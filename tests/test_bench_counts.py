"""The bench's algorithmic counts (the numerator of the reported HBM rate and
MFMA rate), checked on the CPU against counts built independently from the
oracle's position functions on small seeded workloads: the shard's KV bytes
are its local positions times the row size, a multi-token step attends the
union of the shards' positions below each token's causal limit, and the
flops are 2 x heads x (score width + value width) per attended position."""
import numpy as np
import pytest

import bench
import oracle
import workloads as W


CASES = [
    dict(kind="mla", batch=3, heads=16, seq_lens=(1000, 37, 5), num_shards=4, layout=0, block_size=64),
    dict(kind="mla", batch=2, heads=64, seq_lens=(777, 130), num_shards=3, layout=1, block_size=16),
    dict(kind="mla", batch=2, heads=32, seq_lens=(2, 300), num_shards=8, layout=0, block_size=64),
    dict(kind="gqa", batch=2, heads=64, kv_heads=8, seq_lens=(700, 19), num_shards=4, layout=0, block_size=16),
    dict(kind="gqa", batch=3, heads=8, kv_heads=1, seq_lens=(513, 64, 1), num_shards=2, layout=1, block_size=32),
]


@pytest.mark.parametrize("spec", CASES)
@pytest.mark.parametrize("q_len", [1, 3])
@pytest.mark.parametrize("fp8", [False, True])
def test_algorithmic_counts_match_position_sets(spec, q_len, fp8):
    if fp8 and spec["kind"] != "mla":
        pytest.skip("the fp8 cache is an MLA cache")
    w = W.custom_workload(wid=700, **spec)
    case = W.Case(w, seed=0, kv_fp8_scale=W.FP8_SCALE if fp8 else None)
    n = w.num_shards
    for r in range(n):
        # shard r's positions and their union over the step's tokens
        pos = [oracle.shard_positions(int(L), n, r, w.layout) for L in case.seq_lens]
        held = sum(len(p) for p in pos)
        row = (w.dk * (1 if fp8 else 2)) if w.kind == "mla" else 2 * w.kv_heads * w.head_dim * 2
        blocks = sum(-(-len(p) // w.block_size) for p in pos)
        want = (held * row + w.batch * q_len * w.heads * w.dk * 2 + w.batch * q_len * w.heads * (w.dv + 1) * 4
                + blocks * 4 + w.batch * 4)
        got, kv = bench.algorithmic_bytes(case, r, q_len)
        assert kv == held * row and got == want, (r, got, want)
        # attended (request, token) positions, from the oracle's causal prefix per token
        att = sum(len(oracle.query_positions(int(L), q_len, j, n, r, w.layout)) if q_len > 1 else len(p)
                  for L, p in zip(case.seq_lens, pos) for j in range(q_len))
        assert bench.attended(case, r, q_len) == att
        per = 2 * w.heads * (w.dk + w.dv) if w.kind == "mla" else 4 * w.heads * w.head_dim
        assert bench.algorithmic_flops(case, r, q_len) == att * per


def test_combine_bytes():
    w = W.WORKLOADS["c4b"]
    # N partials of (Dv + 1) fp32 per row in, one bf16 row out
    assert bench.combine_bytes(w) == 8 * 128 * 64 * 513 * 4 + 128 * 64 * 512 * 2
    assert bench.combine_bytes(w, 2) == 2 * bench.combine_bytes(w)


def test_full_config_kv_bytes():
    """The long-context figures quoted for the configurations: C4b shard 1 and
    C4a's eight shards each hold 1,048,576 local tokens of 1,152 bytes."""
    c4b = W.Case(W.WORKLOADS["c4b"])
    assert bench.algorithmic_bytes(c4b, 1)[1] == 128 * 8192 * 1152
    c4a = W.Case(W.WORKLOADS["c4a"])
    assert sum(bench.algorithmic_bytes(c4a, r)[1] for r in range(8)) == (1 << 20) * 1152
    kv1 = W.Case(W.WORKLOADS["c3kv1"])
    assert bench.algorithmic_bytes(kv1, 1)[1] == 16 * 65536 * 512
