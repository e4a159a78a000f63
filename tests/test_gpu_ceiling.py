"""The benchmark's pure-stream kernels move exactly the bytes they are given (needs a
GPU): every output pack is the XOR of the input packs, rows and tails included."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ceil():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench
    return bench.Ceiling()


def _inputs(n, rows, row_bytes, seed):
    g = torch.Generator().manual_seed(seed)
    host = [torch.randint(-2**31, 2**31 - 1, (rows, row_bytes // 4), generator=g, dtype=torch.int32)
            for _ in range(n)]
    return host, [h.cuda() for h in host]


def _expected(host):
    x = host[0].clone()
    for h in host[1:]:
        x ^= h
    return x


@pytest.mark.parametrize("n,rows,row_bytes,w,npk,rpb,grid,half", [
    (3, 37, 10240, 2, 5, 4, 5, True),      # prefill shape, half-size second output, grid-stride
    (9, 16, 8192, 8, 1, 1, 16, False),     # decode shape
    (2, 5, 1040, 1, 2, 2, 3, False),       # ragged: 65 packs, team of 64 lanes x 2
])
def test_rows_stream(ceil, n, rows, row_bytes, w, npk, rpb, grid, half):
    host, dev = _inputs(n, rows, row_bytes, rows + n)
    o1 = torch.zeros(rows, row_bytes // 4, dtype=torch.int32, device="cuda")
    o2 = torch.zeros(rows, row_bytes // (8 if half else 4), dtype=torch.int32, device="cuda")
    orow = torch.zeros(rows + 1, dtype=torch.float32, device="cuda")
    ceil.rows([d.data_ptr() for d in dev], o1.data_ptr(), o2.data_ptr(), half, orow.data_ptr(), rows,
              row_bytes, {"waves_per_row": w, "packs_per_lane": npk, "rows_per_block": rpb,
                          "grid_blocks": grid}, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    x = _expected(host)
    assert torch.equal(o1.cpu(), x)
    xv = x.view(rows, -1, 4)
    if half:
        want = torch.stack([xv[..., 0] ^ xv[..., 2], xv[..., 1] ^ xv[..., 3]], -1).view(rows, -1)
    else:
        want = torch.stack([xv[..., 1], xv[..., 2], xv[..., 3], xv[..., 0]], -1).view(rows, -1)
    assert torch.equal(o2.cpu(), want)
    assert orow[rows].item() == 0.0                   # nothing written past the last row


@pytest.mark.parametrize("n,nbytes,unroll,block,grid,half", [
    (3, 1 << 20, 4, 256, 64, True), (9, 16 * 1000, 2, 512, 3, False), (1, 16, 1, 64, 1, False)])
def test_flat_stream(ceil, n, nbytes, unroll, block, grid, half):
    host, dev = _inputs(n, 1, nbytes, n)
    o1 = torch.zeros(nbytes // 4 + 4, dtype=torch.int32, device="cuda")
    o2 = torch.zeros(nbytes // (8 if half else 4) + 4, dtype=torch.int32, device="cuda")
    ceil.flat([d.data_ptr() for d in dev], o1.data_ptr(), o2.data_ptr(), half, nbytes, unroll, block, grid,
              torch.cuda.current_stream().cuda_stream)
    ceil.empty(4, 64, torch.cuda.current_stream().cuda_stream)
    ceil.sleep(3, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    x = _expected(host).view(-1)
    assert torch.equal(o1.cpu()[:-4], x) and not o1.cpu()[-4:].any()
    xv = x.view(-1, 4)
    want = (torch.stack([xv[:, 0] ^ xv[:, 2], xv[:, 1] ^ xv[:, 3]], -1) if half
            else torch.stack([xv[:, 1], xv[:, 2], xv[:, 3], xv[:, 0]], -1)).view(-1)
    assert torch.equal(o2.cpu()[:-4], want) and not o2.cpu()[-4:].any()


def test_stamps_count_up(ceil):
    out = torch.zeros(4, dtype=torch.int64, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    for i in range(3):
        ceil.stamp(out.data_ptr() + 8 * i, st)
        ceil.sleep(20, st)
    torch.cuda.synchronize()
    t = out.cpu().tolist()
    assert 0 < t[0] < t[1] < t[2] and t[3] == 0
    # 20 sleeps of ~8k clocks are tens of microseconds: thousands of 10 ns ticks
    assert 100 < t[1] - t[0] < 10_000_000
