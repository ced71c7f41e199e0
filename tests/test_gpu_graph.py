"""Shard partials + combine captured in a HIP graph: every replay gives the
eager result bit for bit (the kernels are deterministic and keep no state
between calls), with eager work and synchronizations between the replays.

The eager result itself is checked against the oracle by the other GPU tests;
here the oracle checks only the combined rows of one request, so that a replay
that matched a wrong eager result would still fail."""
import pytest
import torch

import workloads as W
from tests.gpu_helpers import ShardRun, assert_rows_close, oracle_rows, say
from kv_cache_context_amd import ops

pytestmark = pytest.mark.gpu

CASES = {
    # split requests (reduce kernel in the step) and one finished inside a workgroup
    "mla": (dict(kind="mla", batch=3, heads=64, seq_lens=(5000, 300, 12000), num_shards=2, wid=601), {}),
    "mla_fp8": (dict(kind="mla", batch=2, heads=32, seq_lens=(9000, 64), num_shards=4, wid=602),
                dict(kv_fp8_scale=W.FP8_SCALE)),
    # sharp softmax with planted keys: the overflow rerun path runs inside the graph
    "mla_peaked": (dict(kind="mla", batch=2, heads=64, seq_lens=(3000, 9000), num_shards=4, wid=603),
                   dict(q_scale_pow2=3, needles=[(0, 2500, 5), (1, 8999, 0)])),
    "gqa": (dict(kind="gqa", batch=3, heads=64, kv_heads=8, head_dim=128, seq_lens=(20000, 700, 0),
                 block_size=16, num_shards=4, wid=604), {}),
    # one and two KV heads per workgroup: sub-tile waves merged through LDS
    "gqa_kv1": (dict(kind="gqa", batch=3, heads=8, kv_heads=1, head_dim=128, seq_lens=(20000, 700, 5),
                     block_size=16, num_shards=2, wid=605), {}),
    "gqa_kv2": (dict(kind="gqa", batch=2, heads=32, kv_heads=2, head_dim=128, seq_lens=(9000, 33),
                     block_size=32, num_shards=2, wid=606), {}),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager(dev, name):
    wk, ck = CASES[name]
    w = W.custom_workload(**wk)
    case = W.Case(w, seed=11, **ck)
    n = w.num_shards
    say(f"graph {name}: b={w.batch} H={w.heads} N={n} lens={list(case.seq_lens)}")
    side = torch.cuda.Stream()
    runs = [ShardRun(case, r, dev) for r in range(n)]
    po = torch.empty((n, w.batch, w.heads, w.dv), dtype=torch.float32, device=dev)
    pl = torch.empty((n, w.batch, w.heads), dtype=torch.float32, device=dev)
    out_bf = torch.empty((w.batch, w.heads, w.dv), dtype=torch.bfloat16, device=dev)
    out_f = torch.empty((w.batch, w.heads, w.dv), dtype=torch.float32, device=dev)
    lse = torch.empty((w.batch, w.heads), dtype=torch.float32, device=dev)
    outputs = (po, pl, out_bf, out_f, lse)

    def step():
        for r, sr in enumerate(runs):
            sr.stream = torch.cuda.current_stream()
            sr.run(po[r], pl[r])
        ops.dcp_combine(po, pl, out_bf, out_f, lse, torch.cuda.current_stream())

    def poison():
        for t in outputs:
            t.fill_(float("nan"))

    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        poison()
        step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    assert not torch.isnan(out_f).any()

    heads = list(range(w.heads))
    b = 0
    o_ref, l_ref = oracle_rows(case, b, heads, None)
    assert_rows_close(out_f[b].cpu().numpy(), lse[b].cpu().numpy(), o_ref, l_ref, f"{name} eager combined b={b}")

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step()
    torch.cuda.synchronize()

    scratch_o = torch.empty_like(po[0])
    scratch_l = torch.empty_like(pl[0])
    for rep in range(3):
        poison()
        # eager work between replays: another shard's call on the same workspace
        with torch.cuda.stream(side):
            runs[rep % n].stream = side
            runs[rep % n].run(scratch_o, scratch_l)
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            g.replay()
        torch.cuda.synchronize()
        for i, (t, t_ref) in enumerate(zip(outputs, ref)):
            assert torch.equal(bits(t), bits(t_ref)), f"{name}: replay {rep} output {i} differs from the eager result"
        assert torch.equal(bits(scratch_o), bits(ref[0][rep % n])), f"{name}: eager call between replays differs"
        assert torch.equal(bits(scratch_l), bits(ref[1][rep % n]))


def bits(t):
    """The tensor's bit patterns (NaN from the poisoning never compares equal to a result)."""
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)
