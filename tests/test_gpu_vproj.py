"""dcp_combine_vproj_gate on the GPU vs the oracle (fp64 merge, per-head value
up-projection, sigmoid gate).

The kernel rounds the merged latent row to bf16 before the projection (one
rounding of relative size 2^-9 per element), so parity is the row-wise bar
(max |y - y_ref| / max |y_ref| <= 1e-2, |lse - lse_ref| <= 1e-3); the bf16
output must be the nearest-even rounding of the kernel's own fp32 output.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import assert_rows_close, say
from workloads.device import bf16_tensor, f32_tensor
from kv_cache_context_amd import ops

pytestmark = pytest.mark.gpu


def _run(dev, n, b, h, dv, dvo, empty, gated=True, seed=0):
    po, pl = W.random_partials(n, b, h, dv, seed=seed + n * 1000 + dv, empty_frac=empty)
    w_bits, g_bits = W.random_vproj(b, h, dvo, dv, seed=seed)
    w = oracle.widen_bf16(w_bits)
    g = oracle.widen_bf16(g_bits) if gated else np.full((b, h, dvo), 80.0)  # sigmoid(80) = 1 in fp64
    y_ref, lse_ref = oracle.combine_vproj_gate(po.astype(np.float64), pl.astype(np.float64), w, g)
    out_bf = torch.empty((b, h, dvo), dtype=torch.bfloat16, device=dev)
    out_f = torch.empty((b, h, dvo), dtype=torch.float32, device=dev)
    lse = torch.empty((b, h), dtype=torch.float32, device=dev)
    ops.dcp_combine_vproj_gate(f32_tensor(po, dev), f32_tensor(pl, dev), bf16_tensor(w_bits, dev),
                               bf16_tensor(g_bits, dev) if gated else None, out_bf, out_f, lse)
    torch.cuda.synchronize()
    return y_ref, lse_ref, out_f.cpu().numpy(), lse.cpu().numpy(), out_bf.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("n,b,h,dv,dvo,empty", [
    (8, 128, 64, 512, 128, 0.1),   # batch-128 step shape: 8 shards, 64 heads
    (8, 32, 64, 512, 128, 0.05),   # batch-32 ragged step shape
    (8, 1, 64, 512, 128, 0.0),     # one request: a 16-row block with 15 rows past the batch
    (4, 19, 5, 64, 48, 0.3),       # ragged batch over two row blocks, odd head count
    (1, 3, 16, 512, 128, 0.0),     # one shard: the merge is the identity
    (64, 17, 2, 1024, 256, 0.25),  # widest shard count, latent and output widths
    (3, 16, 4, 32, 16, 0.5),       # narrowest widths
])
def test_vproj_matches_oracle(dev, n, b, h, dv, dvo, empty):
    say(f"combine_vproj_gate n={n} b={b} h={h} dv={dv} dvo={dvo} empty={empty}")
    y_ref, lse_ref, y, lse, bits = _run(dev, n, b, h, dv, dvo, empty)
    assert_rows_close(y.reshape(-1, dvo), lse.ravel(), y_ref.reshape(-1, dvo), lse_ref.ravel(), "combine_vproj_gate")
    assert np.array_equal(oracle.bf16_rne_bits(y), bits), "bf16 output is not the RNE cast of the fp32 output"


def test_vproj_ungated(dev):
    y_ref, lse_ref, y, lse, _ = _run(dev, 8, 20, 8, 512, 128, 0.1, gated=False, seed=5)
    assert_rows_close(y.reshape(-1, 128), lse.ravel(), y_ref.reshape(-1, 128), lse_ref.ravel(), "ungated")


def test_vproj_all_empty_rows(dev):
    """Rows whose every partial is empty: y = 0 exactly and lse = -inf."""
    y_ref, lse_ref, y, lse, bits = _run(dev, 4, 5, 3, 512, 64, 1.0)
    assert np.all(np.isneginf(lse)) and np.all(y == 0.0) and np.all(bits == 0)


def test_vproj_selection_matches_combine(dev):
    """A projection that picks latent columns and a saturated gate reproduce
    dcp_combine's merged columns (to the bf16 rounding of the operand)."""
    n, b, h, dv, dvo = 8, 24, 4, 512, 32
    po, pl = W.random_partials(n, b, h, dv, seed=77, empty_frac=0.1)
    cols = (np.arange(h)[:, None] * 7 + np.arange(dvo)[None, :] * 13) % dv
    w = np.zeros((h, dvo, dv), dtype=np.float32)
    for hh in range(h):
        w[hh, np.arange(dvo), cols[hh]] = 1.0
    g = np.full((b, h, dvo), 60.0, dtype=np.float32)
    out_f = torch.empty((b, h, dvo), dtype=torch.float32, device=dev)
    ops.dcp_combine_vproj_gate(f32_tensor(po, dev), f32_tensor(pl, dev), bf16_tensor(W.f32_to_bf16_bits(w), dev),
                               bf16_tensor(W.f32_to_bf16_bits(g), dev), None, out_f, None)
    o_c = torch.empty((b, h, dv), dtype=torch.float32, device=dev)
    ops.dcp_combine(f32_tensor(po, dev), f32_tensor(pl, dev), None, o_c, None)
    torch.cuda.synchronize()
    oc = o_c.cpu().numpy()
    picked = np.stack([oc[:, hh, cols[hh]] for hh in range(h)], axis=1)
    # the operand is the bf16 rounding of the merged value (the two kernels merge in
    # different summation orders, so a value may land one bf16 step apart)
    want = oracle.bf16_rne(picked.astype(np.float32))
    got = out_f.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - want) <= np.abs(want) * 2.0 ** -7 + 1e-30)
    assert np.mean(got == want) > 0.99
