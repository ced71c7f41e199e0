"""dcp_combine on the GPU vs the oracle's LSE-weighted merge (fp64)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import assert_rows_close, say
from workloads.device import f32_tensor
from kv_cache_context_amd import ops

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,b,h,dv,empty", [
    (1, 3, 16, 512, 0.0), (2, 2, 64, 512, 0.2), (4, 16, 64, 128, 0.1), (8, 5, 64, 512, 0.3),
    (8, 1, 16, 512, 1.0), (13, 3, 4, 64, 0.5), (64, 2, 8, 1024, 0.25), (3, 7, 5, 4, 0.0),
])
def test_combine_matches_oracle_merge(dev, n, b, h, dv, empty):
    say(f"combine n={n} b={b} h={h} dv={dv} empty={empty}")
    po, pl = W.random_partials(n, b, h, dv, seed=n * 1000 + dv, empty_frac=empty)
    o_ref, lse_ref = oracle.merge(po.astype(np.float64), pl.astype(np.float64))
    po_d, pl_d = f32_tensor(po, dev), f32_tensor(pl, dev)
    out_bf = torch.empty((b, h, dv), dtype=torch.bfloat16, device=dev)
    out_f = torch.empty((b, h, dv), dtype=torch.float32, device=dev)
    lse = torch.empty((b, h), dtype=torch.float32, device=dev)
    ops.dcp_combine(po_d, pl_d, out_bf, out_f, lse)
    torch.cuda.synchronize()
    o_gpu = out_f.cpu().numpy()
    l_gpu = lse.cpu().numpy()
    # fp32 arithmetic on fp32 inputs: far inside the parity bar
    e_o, e_l = assert_rows_close(o_gpu.reshape(-1, dv), l_gpu.ravel(), o_ref.reshape(-1, dv), lse_ref.ravel(),
                                 "combine")
    assert e_o < 1e-5 and e_l < 1e-5, (e_o, e_l)
    # bf16 output: nearest-even rounding of (a value within fp32 error of) the exact result
    bits = out_bf.view(torch.int16).cpu().numpy().view(np.uint16)
    ref_bits = oracle.bf16_rne_bits(o_ref.astype(np.float32))
    lo = oracle.widen_bf16(bits)
    assert np.all(np.abs(lo - o_ref) <= np.abs(o_ref) * 2.0 ** -8 + 1e-30), "bf16 not a neighbour of the result"
    assert np.mean(bits == ref_bits) > 0.999
    # the f32 result rounded on the host equals the device's cast
    assert np.array_equal(oracle.bf16_rne_bits(o_gpu), bits)


def test_combine_optional_outputs(dev):
    po, pl = W.random_partials(4, 2, 16, 512, seed=7)
    po_d, pl_d = f32_tensor(po, dev), f32_tensor(pl, dev)
    out_bf = torch.empty((2, 16, 512), dtype=torch.bfloat16, device=dev)
    ops.dcp_combine(po_d, pl_d, out_bf, None, None)
    out_f = torch.empty((2, 16, 512), dtype=torch.float32, device=dev)
    ops.dcp_combine(po_d, pl_d, None, out_f, None)
    torch.cuda.synchronize()
    o_ref, _ = oracle.merge(po.astype(np.float64), pl.astype(np.float64))
    assert np.abs(out_f.cpu().numpy() - o_ref).max() < 1e-4
    assert np.array_equal(out_bf.view(torch.int16).cpu().numpy().view(np.uint16),
                          oracle.bf16_rne_bits(out_f.cpu().numpy()))


def test_combine_n1_identity(dev):
    po, pl = W.random_partials(1, 3, 8, 512, seed=3)
    po_d, pl_d = f32_tensor(po, dev), f32_tensor(pl, dev)
    out_f = torch.empty((3, 8, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((3, 8), dtype=torch.float32, device=dev)
    ops.dcp_combine(po_d, pl_d, None, out_f, lse)
    torch.cuda.synchronize()
    assert np.array_equal(out_f.cpu().numpy(), po[0])
    assert np.array_equal(lse.cpu().numpy(), pl[0])
