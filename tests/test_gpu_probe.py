"""The tile-owning stream probe of libdlprobe.so (a benchmark ceiling, not part of the
decode library): its column sums against torch, so that the rate it reports is that of a
stream that delivers every unit whole and in place (direct-to-LDS loads, a ring of
eight LDS buffers reused across many tiles, waits counted by hand)."""
import ctypes
import os

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def probe():
    path = os.path.join(ROOT, "linear_attention_recurrent_amd", "libdlprobe.so")
    if not os.path.exists(path):
        pytest.fail("libdlprobe.so is not built: run `python -m linear_attention_recurrent_amd.build`")
    lib = ctypes.CDLL(path)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.dl_probe_owned_stream.argtypes = [vp, ci, ci, vp, ci, vp]
    return lib


def weights(tiles, device):
    t = torch.arange(tiles, device=device, dtype=torch.float64).view(-1, 1)
    r = torch.arange(128, device=device, dtype=torch.float64).view(1, -1)
    return 1 + torch.remainder(131 * t + r, 7) / 8


@pytest.mark.parametrize("tiles,wgs,order", [(512, 256, 0), (300, 256, 0), (301, 7, 0), (512, 256, 1), (770, 35, 1),
                                              (512, 256, 2), (301, 7, 2), (300, 256, 3), (301, 7, 3)])
def test_owned_stream_column_sums(probe, tiles, wgs, order):
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev).manual_seed(tiles * 131 + wgs + order)
    pool = torch.randn(tiles, 128, 128, device=dev, generator=g)
    out = torch.full((tiles, 128), float("nan"), device=dev)
    print(f"owned stream: tiles {tiles} workgroups {wgs} order {order}", flush=True)
    assert probe.dl_probe_owned_stream(pool.data_ptr(), tiles, order, out.data_ptr(), wgs,
                                       torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    if order != 1:  # whole tiles per workgroup, in any order: each tile's own rows
        rows = pool.double()
    else:  # "tile" T = w + i G gathers units w + (4i + j) G, j < 4, as its rows 32j..32j+31
        T = torch.arange(tiles, device=dev)
        w, i = T % wgs, T // wgs
        idx = w.view(-1, 1) + (4 * i.view(-1, 1) + torch.arange(4, device=dev).view(1, -1)) * wgs
        rows = pool.view(tiles * 4, 32, 128)[idx].reshape(tiles, 128, 128).double()
    ref = (rows * weights(tiles, dev).unsqueeze(-1)).sum(dim=1)
    assert torch.isfinite(out).all()
    err = ((out.double() - ref).abs().max() / ref.abs().max()).item()
    assert err < 1e-5, err


@pytest.mark.parametrize("tiles,exchange", [(512, 0), (300, 1), (2048, 1)])
def test_quarter_split_column_sums(probe, tiles, exchange):
    """Quarter-split partial column sums, and with the exchange the four quarters of each
    tile added up inside the launch by the last workgroup to arrive (counts left zero)."""
    probe.dl_probe_quarter_split.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev).manual_seed(tiles + exchange)
    pool = torch.randn(tiles, 128, 128, device=dev, generator=g)
    part = torch.full((tiles, 4, 256), float("nan"), device=dev)
    cnt = torch.zeros(tiles, dtype=torch.int32, device=dev)
    out = torch.full((tiles, 256), float("nan"), device=dev)
    print(f"quarter split: tiles {tiles} exchange {exchange}", flush=True)
    for _ in range(2):  # the second launch starts from the counts the first left
        assert probe.dl_probe_quarter_split(pool.data_ptr(), tiles, exchange, part.data_ptr(), cnt.data_ptr(),
                                            out.data_ptr(), torch.cuda.current_stream().cuda_stream) == 0
        torch.cuda.synchronize()
    t = torch.arange(tiles, device=dev, dtype=torch.float64).view(-1, 1)
    r = torch.arange(128, device=dev, dtype=torch.float64).view(1, -1)
    w1 = 1 + torch.remainder(131 * t + r, 7) / 8
    w2 = 0.5 + torch.remainder(17 * t + r, 5) / 4
    B = pool.double()
    quarters = [torch.cat([(B[:, 32 * q:32 * q + 32] * w[:, 32 * q:32 * q + 32].unsqueeze(-1)).sum(1)
                           for w in (w1, w2)], dim=1) for q in range(4)]
    ref_part = torch.stack(quarters, dim=1)
    err = ((part.double() - ref_part).abs().max() / ref_part.abs().max()).item()
    assert err < 1e-5, err
    if exchange:
        ref = ref_part.sum(1)
        err = ((out.double() - ref).abs().max() / ref.abs().max()).item()
        assert err < 1e-5, err
        assert bool((cnt == 0).all())
