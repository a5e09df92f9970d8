"""Layout permutation and positions on the GPU: byte work, so bit-exact
against the oracle's layout maps."""

import numpy as np
import pytest
import torch

import blockwise_online_softmax_amd as ra
from oracle import layouts as OL
from gpu_helpers import log

pytestmark = pytest.mark.gpu

CASES = [(12, 4), (96, 8), (600, 3), (4096, 8), (65536, 8)]


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
@pytest.mark.parametrize("S,N", CASES)
def test_positions(S, N, layout):
    if layout == "zigzag" and S % (2 * N):
        pytest.skip("zigzag needs S % 2N == 0")
    log(f"positions S={S} N={N} {layout}")
    pos = torch.empty(S, dtype=torch.int32, device="cuda")
    ra.ra_positions(pos, S, N, layout, -1)
    want = OL.permuted_positions(S, N, layout)
    got = pos.cpu().numpy()
    assert np.array_equal(got, want)
    # the host copy of the same map (ra_layout_position) agrees with the kernel
    for i in sorted({0, 1, S // 2, S - 2, S - 1}):
        assert ra.ra_layout_position(S, N, layout, -1, i) == got[i]
    for p in (0, N // 2, N - 1):
        pp = torch.empty(S // N, dtype=torch.int32, device="cuda")
        ra.ra_positions(pp, S, N, layout, p)
        assert np.array_equal(pp.cpu().numpy(), OL.device_positions(S, N, layout, p))


@pytest.mark.parametrize("layout", ["striped", "zigzag", "contiguous"])
@pytest.mark.parametrize("S,N,row", [(96, 8, (32,)), (600, 3, (128,)), (4096, 8, (128,)),
                                     (48, 4, ()), (48, 4, (3,))])
def test_permute_bitexact(S, N, row, layout):
    if layout == "zigzag" and S % (2 * N):
        pytest.skip("zigzag needs S % 2N == 0")
    log(f"permute S={S} N={N} row={row} {layout}")
    g = torch.Generator().manual_seed(S + N)
    for dtype in (torch.float32, torch.bfloat16):
        x = torch.randn((3, S) + row, generator=g).to(dtype)
        xd = x.cuda()
        y = torch.empty_like(xd)
        row_bytes = x.element_size() * int(np.prod(row, dtype=np.int64))
        if row_bytes % 4:
            with pytest.raises(RuntimeError, match="RA_ERR_SHAPE"):
                ra.ra_permute(xd, y, N, layout, inverse=False)
            continue
        ra.ra_permute(xd, y, N, layout, inverse=False)
        want = OL.to_device_order(x.float().numpy(), N, layout, axis=1)
        assert np.array_equal(y.cpu().float().numpy(), want)
        z = torch.empty_like(xd)
        ra.ra_permute(y, z, N, layout, inverse=True)
        assert torch.equal(z.cpu(), x)
