"""GPU check of the benchmark's read-bandwidth probe (probe.probe_block_read,
built into its own library, libattn_probe.so).

The probe computes nothing but an XOR of every 32-bit word it reads, so its
result has a plain definition: the XOR over all sink words must equal the XOR
of every word of every block listed in `order` (numpy on the host, bit-exact).
Cases cover both cache policies, every block size the entry accepts, a read
count that is not a multiple of the wave count (waves with one block, waves
with none), and repeated block ids (each listed read counts once, so a pair
cancels).
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import probe
    return probe


def host_xor(data, block_bytes, order):
    words = data.numpy().view(np.uint32).reshape(-1, block_bytes // 4)[order.numpy()]
    return int(np.bitwise_xor.reduce(words.ravel())) if words.size else 0


def device_xor(sink):
    return int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)))


@pytest.mark.parametrize("nontemporal", [False, True])
@pytest.mark.parametrize("block_bytes", [1024, 2048, 4096, 8192, 16384])
@pytest.mark.parametrize("n_reads,n_waves", [(77, 8), (5, 8), (200, 4), (96, 256)])
def test_probe_xor_matches_host(api, block_bytes, n_reads, n_waves, nontemporal):
    g = torch.Generator().manual_seed(block_bytes + n_reads)
    nb = 96
    data = torch.randint(0, 256, (nb * block_bytes,), generator=g, dtype=torch.uint8)
    order = torch.randint(0, nb, (n_reads,), generator=g, dtype=torch.int32)
    print(f"[probe test] block_bytes={block_bytes} n_reads={n_reads} n_waves={n_waves} "
          f"nontemporal={nontemporal}", flush=True)
    sink = api.probe_block_read(data.cuda(), block_bytes, order.cuda(), n_waves,
                                     nontemporal=nontemporal)
    torch.cuda.synchronize()
    assert device_xor(sink) == host_xor(data, block_bytes, order)


def test_probe_repeated_ids_cancel(api):
    block_bytes = 4096
    data = torch.randint(0, 256, (8 * block_bytes,), generator=torch.Generator().manual_seed(3),
                         dtype=torch.uint8)
    order = torch.tensor([2, 5, 2, 5], dtype=torch.int32)
    sink = api.probe_block_read(data.cuda(), block_bytes, order.cuda(), 4)
    torch.cuda.synchronize()
    assert device_xor(sink) == 0
