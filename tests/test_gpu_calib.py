"""The measurement probes on the GPU: the read stream touches every 16-byte unit of the buffer exactly
once (needs an MI355X)."""

import numpy as np
import pytest
import torch

import sparse_moe_layer_router_amd as moe

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 1 << 20, (1 << 20) + 16 * 37, 64 << 20, 512 * 1024 * 3 + 1008])
@pytest.mark.parametrize("nontemporal", [True, False])
def test_read_probe_reads_every_unit_once(nbytes, nontemporal):
    """The XOR of the workgroups' sink words equals the XOR of every 32-bit word of the buffer: a unit
    skipped, or read by two lanes, leaves a word of random data out of the fold (or cancels it)."""
    rng = np.random.default_rng(nbytes)
    host = rng.integers(-2**31, 2**31, size=nbytes // 4, dtype=np.int64).astype(np.int32)
    buf = torch.from_numpy(host).cuda()
    sink = torch.zeros(moe.MOE_CALIB_READ_BLOCKS, dtype=torch.int32, device="cuda")
    moe.moe_calib_read_stream(buf, sink, nontemporal)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy())
    assert got == np.bitwise_xor.reduce(host)
