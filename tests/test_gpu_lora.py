"""GPU parity of isd_linear, gated_lora_apply and isd_linear_gated.

Pass criteria: outputs within 2e-3 relative of the fp64 oracle (normwise over
each output matrix: max |y - y*| / max |y*|), and clean rows bit-identical to
the base projection.
"""

import numpy as np
import pytest
import torch

import draft_verify_decoding_amd as dvd
import workload
from oracle import lora as ref

pytestmark = pytest.mark.gpu
DEV = "cuda"


def case(seed, M, K, Nout, r, N=4):
    print(f"lora case M={M} K={K} Nout={Nout} r={r}", flush=True)
    x, W, A, B = workload.lora_case(seed, M, K, Nout, r)
    mask = workload.stride_mask(M, N)
    return x, W, A, B, mask


def rel_err(got, want):
    return np.abs(got - want).max() / np.abs(want).max()


def dev(*ts):
    return [t.to(DEV).contiguous() for t in ts]


@pytest.mark.parametrize("Nout", [4096, 1024])
def test_base_projection_8b_shapes(Nout):
    """512 rows (C=64 x 2N=8), hidden 4096, Q/O (4096) and K/V (1024) widths."""
    x, W, A, B, mask = case(1, 512, 4096, Nout, 32)
    xd, Wd = dev(x, W)
    y = dvd.isd_linear(xd, Wd)
    torch.cuda.synchronize()
    want = ref.linear(x.double().numpy(), W.double().numpy())
    e = rel_err(y.cpu().double().numpy(), want)
    print("isd_linear rel err", e)
    assert e < 1e-4


@pytest.mark.parametrize("Nout,r", [(4096, 32), (4096, 128), (6144, 96)])
def test_gated_lora_8b_shapes(Nout, r):
    """O projection (4096) and fused Q|K|V (6144 = 4096 + 2 * 1024, r = 3 * 32)."""
    x, W, A, B, mask = case(2, 512, 4096, Nout, r)
    xd, Wd, Ad, Bd = dev(x, W, A, B)
    md = torch.from_numpy(mask.astype(np.uint8)).to(DEV)
    base = dvd.isd_linear(xd, Wd)
    fused = dvd.isd_linear_gated(xd, Wd, Ad, Bd, md, scale=1.0)
    sep = base.clone()
    dvd.gated_lora_apply(xd, Ad, Bd, md, sep, scale=1.0)
    torch.cuda.synchronize()
    want = ref.gated_lora(x.double().numpy(), W.double().numpy(), A.double().numpy(),
                          B.double().numpy(), mask, 1.0)
    f = fused.cpu()
    assert rel_err(f.double().numpy(), want) < 2e-3
    # the delta itself is small; hold it to the same relative bar on its own
    delta_got = (f - base.cpu()).double().numpy()[mask]
    delta_want = (want - ref.linear(x.double().numpy(), W.double().numpy()))[mask]
    assert rel_err(delta_got, delta_want) < 2e-3
    # clean rows: bit-identical to the base projection, both paths
    m = torch.from_numpy(mask)
    assert torch.equal(f[~m].view(torch.int32), base.cpu()[~m].view(torch.int32))
    assert torch.equal(sep.cpu()[~m].view(torch.int32), base.cpu()[~m].view(torch.int32))
    # fused and separate application agree bit for bit on every row
    assert torch.equal(f.view(torch.int32), sep.cpu().view(torch.int32))


@pytest.mark.parametrize("K,Nout,r", [(5120, 10240, 96), (8192, 5120, 32)])
def test_gated_lora_32b_shapes(K, Nout, r):
    """32B-class projections of a C=16, N=4 step (128 rows, hidden 5120):
    fused Q|K|V (64 + 2 x 8 heads of 128 = 10240 wide, r = 3 x 32) and O
    (8192 -> 5120). These sizes pick other tiles than the 8B ones; a row
    block computed alone (another tile again) keeps the same bits."""
    M = 128
    x, W, A, B, mask = case(7, M, K, Nout, r)
    xd, Wd, Ad, Bd = dev(x, W, A, B)
    md = torch.from_numpy(mask.astype(np.uint8)).to(DEV)
    base = dvd.isd_linear(xd, Wd)
    fused = dvd.isd_linear_gated(xd, Wd, Ad, Bd, md, scale=1.0)
    sep = base.clone()
    dvd.gated_lora_apply(xd, Ad, Bd, md, sep, scale=1.0)
    alone = dvd.isd_linear_gated(xd[40:48].contiguous(), Wd, Ad, Bd, md[40:48].contiguous(), scale=1.0)
    torch.cuda.synchronize()
    want = ref.gated_lora(x.double().numpy(), W.double().numpy(), A.double().numpy(),
                          B.double().numpy(), mask, 1.0)
    f = fused.cpu()
    assert rel_err(f.double().numpy(), want) < 2e-3
    m = torch.from_numpy(mask)
    assert torch.equal(f[~m].view(torch.int32), base.cpu()[~m].view(torch.int32))
    assert torch.equal(f.view(torch.int32), sep.cpu().view(torch.int32))
    assert torch.equal(alone.cpu().view(torch.int32), f[40:48].view(torch.int32))


def test_reduction_order_does_not_depend_on_rows_or_tile():
    """Row results of isd_linear are the same bits whether the row is
    computed with 511 others, alone, or in a small launch that picks the
    other tile size."""
    x, W, A, B, mask = case(3, 512, 4096, 1024, 32)
    xd, Wd = dev(x, W)
    full = dvd.isd_linear(xd, Wd)
    part = dvd.isd_linear(xd[200:237].contiguous(), Wd)
    one = dvd.isd_linear(xd[300:301].contiguous(), Wd)
    torch.cuda.synchronize()
    assert torch.equal(full[200:237], part)
    assert torch.equal(full[300:301], one)


def test_zero_adapter_leaves_values_and_ragged_sizes():
    """B = 0: MASK rows equal the base values (a real +0 add), clean rows
    equal the base bits; M and Nout not multiples of any tile."""
    x, W, A, B, _ = case(4, 77, 256, 130, 16)
    mask = workload.stride_mask(77, 3)
    xd, Wd, Ad = dev(x, W, A)
    Bd = torch.zeros_like(B).to(DEV)
    md = torch.from_numpy(mask.astype(np.uint8)).to(DEV)
    base = dvd.isd_linear(xd, Wd)
    y = dvd.isd_linear_gated(xd, Wd, Ad, Bd, md, scale=3.0)
    torch.cuda.synchronize()
    assert torch.equal(y, base)  # == on values (+0.0 == -0.0)
    m = torch.from_numpy(mask).to(DEV)
    assert torch.equal(y[~m].view(torch.int32), base[~m].view(torch.int32))
    want = ref.linear(x.double().numpy(), W.double().numpy())
    assert rel_err(base.cpu().double().numpy(), want) < 1e-4


def test_scaled_adapter_ragged():
    x, W, A, B, _ = case(5, 100, 192, 200, 48)
    mask = workload.stride_mask(100, 2)
    xd, Wd, Ad, Bd = dev(x, W, A, B)
    md = torch.from_numpy(mask.astype(np.uint8)).to(DEV)
    y = dvd.isd_linear_gated(xd, Wd, Ad, Bd, md, scale=0.5)
    torch.cuda.synchronize()
    want = ref.gated_lora(x.double().numpy(), W.double().numpy(), A.double().numpy(),
                          B.double().numpy(), mask, 0.5)
    assert rel_err(y.cpu().double().numpy(), want) < 2e-3


def test_large_batch_uses_the_wide_tile_with_same_bits():
    """2048 rows (C=256, N=4) pick the 128x128 tile; sampled rows match the
    oracle, and equal bit for bit the same rows computed in a small launch
    (64x64 tile). The fused U columns straddle the last W tile."""
    x, W, A, B, mask = case(6, 2048, 4096, 4096, 32)
    xd, Wd, Ad, Bd = dev(x, W, A, B)
    md = torch.from_numpy(mask.astype(np.uint8)).to(DEV)
    base = dvd.isd_linear(xd, Wd)
    fused = dvd.isd_linear_gated(xd, Wd, Ad, Bd, md, scale=2.0)
    small = dvd.isd_linear_gated(xd[1000:1040].contiguous(), Wd, Ad, Bd, md[1000:1040].contiguous(), scale=2.0)
    torch.cuda.synchronize()
    assert torch.equal(fused[1000:1040], small)
    m = torch.from_numpy(mask).to(DEV)
    assert torch.equal(fused[~m].view(torch.int32), base[~m].view(torch.int32))
    rows = np.array([0, 1, 7, 513, 1000, 1031, 2046, 2047])
    want = ref.gated_lora(x[rows].double().numpy(), W.double().numpy(), A.double().numpy(),
                          B.double().numpy(), mask[rows], 2.0)
    assert rel_err(fused.cpu()[rows].double().numpy(), want) < 2e-3
