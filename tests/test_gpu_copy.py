"""rt_copy_from_host(_2d) on the GPU: pinned host memory reaches device
memory bit for bit through the copy kernel (16-byte and 4-byte paths, a word
tail, offsets inside an allocation, column blocks of row-pitched tables), and
pageable memory is refused before any launch."""

import numpy as np
import pytest
import torch

from prefix_shared_kv_rt_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,src_off,dst_off", [(1_000_003, 0, 0), (4096 * 65, 0, 0), (1001, 3, 1), (7, 4, 4),
                                               (1, 0, 5)])
def test_copy_from_pinned_host(n, src_off, dst_off):
    print(f"rt_copy_from_host n={n} src_off={src_off} dst_off={dst_off}", flush=True)
    rng = np.random.default_rng(n + src_off)
    host = torch.from_numpy(rng.integers(-2**31, 2**31 - 1, n + src_off + 8, dtype=np.int64).astype(np.int32))
    host = host.pin_memory()
    dev = torch.full((n + dst_off + 8,), -7, dtype=torch.int32, device="cuda")
    B.rt_copy_from_host(dev[dst_off:dst_off + n], host[src_off:src_off + n])
    torch.cuda.synchronize()
    got = dev.cpu()
    assert torch.equal(got[dst_off:dst_off + n], host[src_off:src_off + n])
    assert bool((got[:dst_off] == -7).all()) and bool((got[dst_off + n:] == -7).all())


@pytest.mark.parametrize("rows,cols,c0,c1", [(69, 1153, 1024, 1153), (64, 1156, 1024, 1156), (3, 40, 4, 36),
                                              (1, 9, 2, 3)])
def test_copy_from_host_2d_column_block(rows, cols, c0, c1):
    print(f"rt_copy_from_host_2d rows={rows} cols={cols} columns {c0}..{c1}", flush=True)
    rng = np.random.default_rng(rows * cols + c0)
    host = torch.from_numpy(rng.integers(-2**31, 2**31 - 1, (rows, cols), dtype=np.int64).astype(np.int32))
    host = host.pin_memory()
    dev = torch.full((rows, cols), -7, dtype=torch.int32, device="cuda")
    B.rt_copy_from_host_2d(dev[:, c0:c1], host[:, c0:c1])
    torch.cuda.synchronize()
    got = dev.cpu()
    assert torch.equal(got[:, c0:c1], host[:, c0:c1])
    assert bool((got[:, :c0] == -7).all()) and bool((got[:, c1:] == -7).all())


def test_copy_from_host_refuses_pageable_memory():
    src = torch.arange(64, dtype=torch.int32)          # ordinary (pageable) host memory
    assert not src.is_pinned()
    dev = torch.full((64,), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(B.RadixRTError):
        B.rt_copy_from_host(dev, src)
    torch.cuda.synchronize()
    assert bool((dev.cpu() == -7).all())


def test_copy_from_host_refuses_host_destination():
    src = torch.arange(64, dtype=torch.int32).pin_memory()
    for dst in (torch.zeros(64, dtype=torch.int32), torch.zeros(64, dtype=torch.int32).pin_memory()):
        with pytest.raises(B.RadixRTError):
            B.rt_copy_from_host(dst, src)
        assert bool((dst == 0).all())


def test_copy_from_host_rejects_bad_sizes():
    host = torch.zeros(16, dtype=torch.int32).pin_memory()
    dev = torch.zeros(16, dtype=torch.int32, device="cuda")
    rc = B.lib().rt_copy_from_host(dev.data_ptr(), host.data_ptr(), 6, None)   # not a multiple of 4
    assert rc == B.RT_ERR_INVALID
    rc = B.lib().rt_copy_from_host(dev.data_ptr(), host.data_ptr() + 2, 8, None)  # misaligned
    assert rc == B.RT_ERR_INVALID


def test_copy_check_launches_nothing_and_follows_the_allocations():
    """rt_copy_from_host_check alone: accepts what the copy accepts, refuses
    pageable sources, ranges past the pinned source allocation, host
    destinations and ranges past the device allocation; no kernel runs."""
    src = torch.arange(1024, dtype=torch.int32).pin_memory()
    dst = torch.full((1024,), -7, dtype=torch.int32, device="cuda")
    B.rt_copy_from_host_check(dst, src)
    B.rt_copy_from_host_check(dst[:512], src[512:])
    B.rt_copy_from_host_check(dst.view(32, 32)[:, 4:12], src.view(32, 32)[:, 4:12], dst_pitch=128, src_pitch=128,
                              width=32, height=32)
    with pytest.raises(B.RadixRTError, match="pinned"):
        B.rt_copy_from_host_check(dst, torch.arange(1024, dtype=torch.int32))     # pageable
    with pytest.raises(B.RadixRTError, match="pinned"):
        B.rt_copy_from_host_check(dst, src, width=64 << 20)                        # past the pinned block
    with pytest.raises(B.RadixRTError, match="destination"):
        B.rt_copy_from_host_check(torch.zeros(1024, dtype=torch.int32).pin_memory(), src)
    big = torch.full((64 << 20,), 0, dtype=torch.uint8)
    with pytest.raises(B.RadixRTError, match="destination"):
        B.rt_copy_from_host_check(dst, big.pin_memory())                           # past the device block
    torch.cuda.synchronize()
    assert bool((dst.cpu() == -7).all())
