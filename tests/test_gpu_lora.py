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


@pytest.mark.parametrize("gated", [False, True])
def test_wide_projection_tile_same_bits(gated):
    """The MLP's fused gate|up width (512 rows, 24,576 outputs) picks the
    128x192 tile; sampled rows match the oracle, clean rows equal the base
    projection, and rows equal bit for bit the same rows computed in a small
    launch (another tile)."""
    x, W, A, B, mask = case(8, 512, 1024, 24576, 32)
    xd, Wd, Ad, Bd = dev(x, W, A, B)
    md = torch.from_numpy(mask.astype(np.uint8)).to(DEV)
    base = dvd.isd_linear(xd, Wd)
    if gated:
        y = dvd.isd_linear_gated(xd, Wd, Ad, Bd, md, scale=1.0)
        small = dvd.isd_linear_gated(xd[100:140].contiguous(), Wd, Ad, Bd, md[100:140].contiguous(), scale=1.0)
    else:
        y = base
        small = dvd.isd_linear(xd[100:140].contiguous(), Wd)
    torch.cuda.synchronize()
    assert torch.equal(y[100:140].view(torch.int32), small.view(torch.int32))
    m = torch.from_numpy(mask).to(DEV)
    assert torch.equal(y[~m].view(torch.int32), base[~m].view(torch.int32))
    rows = np.array([0, 5, 127, 128, 300, 511])
    want = ref.gated_lora(x[rows].double().numpy(), W.double().numpy(), A.double().numpy(), B.double().numpy(),
                          mask[rows], 1.0 if gated else 0.0)
    assert rel_err(y.cpu()[rows].double().numpy(), want) < 2e-3


@pytest.mark.parametrize("M", [1, 8, 13, 32])
@pytest.mark.parametrize("r", [0, 32, 96, 128])
def test_few_rows_same_bits_as_the_tiled_kernel(M, r):
    """Up to 32 rows (a single sequence's stride block and a few more) run
    one wave per 32 output columns over the whole of K; their outputs equal,
    bit for bit, the same rows inside a 512-row launch (the tiled kernel),
    base and gated, and match the oracle. The fused Q|K|V width, 6144."""
    K, Nout = 4096, 6144
    x, W, A, B, mask = case(9, 512, K, Nout, max(r, 16))
    xd, Wd, Ad, Bd = dev(x, W, A, B)
    md = torch.from_numpy(mask.astype(np.uint8)).to(DEV)
    if r:
        full = dvd.isd_linear_gated(xd, Wd, Ad, Bd, md, scale=1.0)
        few = dvd.isd_linear_gated(xd[:M].contiguous(), Wd, Ad, Bd, md[:M].contiguous(), scale=1.0)
    else:
        full = dvd.isd_linear(xd, Wd)
        few = dvd.isd_linear(xd[:M].contiguous(), Wd)
    torch.cuda.synchronize()
    assert torch.equal(few.view(torch.int32), full[:M].view(torch.int32))
    want = ref.gated_lora(x[:M].double().numpy(), W.double().numpy(), A.double().numpy(), B.double().numpy(),
                          mask[:M], 1.0 if r else 0.0)
    assert rel_err(few.cpu().double().numpy(), want) < 2e-3


@pytest.mark.parametrize("M,K,Nout", [(8, 64, 200), (5, 192, 33), (32, 640, 4096), (17, 12288, 96)])
def test_few_rows_ragged_shapes(M, K, Nout):
    """Few-row launches with fewer slabs than stages (K = 64, 192), a ragged
    last column block, 17 rows (32 staged rows) and a long K (12,288): gated
    outputs match the oracle and equal the tiled kernel's rows bit for bit."""
    x, W, A, B, mask = case(10, 256, K, Nout, 32)
    xd, Wd, Ad, Bd = dev(x, W, A, B)
    md = torch.from_numpy(mask.astype(np.uint8)).to(DEV)
    full = dvd.isd_linear_gated(xd, Wd, Ad, Bd, md, scale=0.75)
    few = dvd.isd_linear_gated(xd[:M].contiguous(), Wd, Ad, Bd, md[:M].contiguous(), scale=0.75)
    torch.cuda.synchronize()
    assert torch.equal(few.view(torch.int32), full[:M].view(torch.int32))
    want = ref.gated_lora(x[:M].double().numpy(), W.double().numpy(), A.double().numpy(), B.double().numpy(),
                          mask[:M], 0.75)
    assert rel_err(few.cpu().double().numpy(), want) < 2e-3


@pytest.mark.parametrize("M", [8, 512])
def test_bf16_output_is_the_rounded_fp32_output(M):
    """ydtype bf16: every output is the fp32 result rounded to nearest even,
    in the tiled kernel (512 rows) and the few-row kernel (8 rows), base and
    fused gated; clean rows of the gated call equal the base call's; the
    separate gated_lora_apply on a bf16 y rounds its MASK rows a second time,
    so they stay within one bf16 step of the fused call's."""
    x, W, A, B, mask = case(11, M, 4096, 4096, 32)
    xd, Wd, Ad, Bd = dev(x, W, A, B)
    md = torch.from_numpy(mask.astype(np.uint8)).to(DEV)
    base32 = dvd.isd_linear(xd, Wd)
    base16 = dvd.isd_linear(xd, Wd, ydtype=torch.bfloat16)
    fused32 = dvd.isd_linear_gated(xd, Wd, Ad, Bd, md, scale=1.0)
    fused16 = dvd.isd_linear_gated(xd, Wd, Ad, Bd, md, scale=1.0, ydtype=torch.bfloat16)
    sep16 = base16.clone()
    dvd.gated_lora_apply(xd, Ad, Bd, md, sep16, scale=1.0)
    torch.cuda.synchronize()
    bits = lambda t: t.contiguous().view(torch.int16)
    assert base16.dtype == torch.bfloat16 and fused16.dtype == torch.bfloat16
    assert torch.equal(bits(base16), bits(base32.to(torch.bfloat16)))
    assert torch.equal(bits(fused16), bits(fused32.to(torch.bfloat16)))
    m = torch.from_numpy(mask).to(DEV)
    assert torch.equal(bits(fused16[~m]), bits(base16[~m]))
    assert torch.equal(bits(sep16[~m]), bits(base16[~m]))
    # the separate call rounds the base value before adding the delta: the
    # two differ by at most a rounding of the base value and one of each result
    f, s_, acc = fused16[m].float(), sep16[m].float(), base32[m]
    assert torch.all((f - s_).abs() <= 2.0 ** -8 * (acc.abs() + f.abs() + s_.abs()) + 1e-30)
    want = ref.gated_lora(x.double().numpy(), W.double().numpy(), A.double().numpy(), B.double().numpy(), mask, 1.0)
    got = fused16.float().cpu().double().numpy()
    assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + 1e-4 * np.abs(want).max())


@pytest.mark.parametrize("M,r", [(8, 96), (32, 32)])
def test_few_rows_one_launch_and_two_launch_paths_agree(M, r):
    """With up to 32 rows U's split-K workgroups join the GEMM's launch when
    the whole grid is resident on the GPU at once; a wider output (20,480
    columns: 640 column blocks plus U's) does not fit, and U then has a launch
    of its own. A column block's outputs do not depend on the width, so the
    narrow call (one launch) equals the first columns of the wide call (two
    launches) bit for bit, call after call on one workspace, whose counter
    pair is back at zero after every call; the narrow call matches the
    oracle."""
    K, Nw, Nn = 4096, 20480, 4096
    x, W, A, B, mask = case(12, M, K, Nw, r)
    xd, Wd, Ad, Bd = dev(x, W, A, B)
    md = torch.from_numpy(mask.astype(np.uint8)).to(DEV)
    ws = dvd.lora_workspace(M, r)
    wide = dvd.isd_linear_gated(xd, Wd, Ad, Bd, md, scale=0.5, ws=ws)
    Wn, Bn = Wd[:Nn].contiguous(), Bd[:Nn].contiguous()
    narrow = [dvd.isd_linear_gated(xd, Wn, Ad, Bn, md, scale=0.5, ws=ws) for _ in range(3)]
    torch.cuda.synchronize()
    assert int(ws[:256].count_nonzero()) == 0
    for y in narrow:
        assert torch.equal(y.view(torch.int32), wide[:, :Nn].view(torch.int32))
    want = ref.gated_lora(x.double().numpy(), W[:Nn].double().numpy(), A.double().numpy(), B[:Nn].double().numpy(),
                          mask, 0.5)
    assert rel_err(narrow[0].cpu().double().numpy(), want) < 2e-3


@pytest.mark.parametrize("M,K,Nout,r", [(512, 4096, 6144, 96), (512, 4096, 4096, 32), (200, 4096, 4096, 128),
                                        (128, 5120, 10240, 96), (72, 4096, 1024, 16)])
def test_tiled_fused_call_matches_separate_calls(M, K, Nout, r):
    """Above 32 rows (tiled kernels, every tile shape the picker takes here,
    ragged row counts, ranks 16 to 128): the fused call equals isd_linear
    followed by gated_lora_apply bit for bit on every row, call after call on
    one workspace, whose counter bytes stay zero; it matches the oracle."""
    x, W, A, B, mask = case(13, M, K, Nout, r)
    xd, Wd, Ad, Bd = dev(x, W, A, B)
    md = torch.from_numpy(mask.astype(np.uint8)).to(DEV)
    ws = dvd.lora_workspace(M, r)
    sep = dvd.isd_linear(xd, Wd)
    dvd.gated_lora_apply(xd, Ad, Bd, md, sep, scale=0.75, ws=ws)
    fused = [dvd.isd_linear_gated(xd, Wd, Ad, Bd, md, scale=0.75, ws=ws) for _ in range(3)]
    torch.cuda.synchronize()
    assert int(ws[:256].count_nonzero()) == 0
    for y in fused:
        assert torch.equal(y.view(torch.int32), sep.view(torch.int32))
    want = ref.gated_lora(x.double().numpy(), W.double().numpy(), A.double().numpy(), B.double().numpy(), mask, 0.75)
    assert rel_err(fused[0].cpu().double().numpy(), want) < 2e-3
