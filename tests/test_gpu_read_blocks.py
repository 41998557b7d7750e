"""The read-bandwidth reference (pa_read_blocks): every word of every block
named in the order is read exactly once (the XOR sink equals the XOR over
those blocks computed on the host), ids outside the buffer are skipped, and
every block size it accepts works."""
import numpy as np
import pytest
import torch

import paged_kv_cache_02_amd as pa

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("block_bytes,norder", [(4096, 300), (8192, 300), (16384, 300), (32768, 300),
                                                (4096, 5000)])
def test_read_blocks_folds_every_named_block(block_bytes, norder):
    # 5000 blocks is more than the launch's workgroups, so each one walks
    # several blocks
    rng = np.random.default_rng(block_bytes + norder)
    nblk = 37
    host = rng.integers(0, 2**32, size=nblk * block_bytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.uint8)).cuda()
    # a random order with repeats and ids outside the buffer (skipped)
    order = rng.integers(-3, nblk + 3, size=norder).astype(np.int32)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    print(f"case read blocks {block_bytes} x {norder}", flush=True)
    pa.pa_read_blocks(buf, torch.from_numpy(order).cuda(), block_bytes, sink)
    torch.cuda.synchronize()
    words = host.reshape(nblk, -1)
    want = np.uint32(0)
    for i in order:
        if 0 <= i < nblk:
            want ^= np.bitwise_xor.reduce(words[i])
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(want)


def test_read_blocks_rejects_other_block_sizes():
    buf = torch.zeros(8192, dtype=torch.uint8, device="cuda")
    order = torch.zeros(1, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(pa.PaError):
        pa.pa_read_blocks(buf, order, 2048, sink)
