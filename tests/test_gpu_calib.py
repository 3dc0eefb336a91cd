"""The measurement probes on the GPU: the read stream touches every 16-byte unit of the buffer exactly
once, and the MFMA loop executes every instruction it counts (needs an MI355X)."""

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


@pytest.mark.parametrize("iters", [1, 4])
def test_mfma_probe_accumulates_every_instruction(iters):
    """With every operand 1.0 each 32x32x16 MFMA adds 16 to each of a wave's 1,024 outputs, so a
    workgroup's sum is 8 waves x 8 accumulators x 1,024 outputs x 16 x iters (exact in float32 for
    these counts): an instruction dropped or an accumulator left out changes it. The clock counters
    of every wave advance."""
    n = moe.MOE_CALIB_MFMA_BLOCKS * 512 * 16
    ops = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    sink = torch.zeros(moe.MOE_CALIB_MFMA_BLOCKS, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(moe.MOE_CALIB_MFMA_BLOCKS * 8 * 4, dtype=torch.int64, device="cuda")
    moe.moe_calib_mfma(ops, iters, sink, clocks)
    torch.cuda.synchronize()
    assert (sink.cpu().numpy() == 8 * 8 * 1024 * 16 * iters).all()
    c = clocks.view(-1, 4).cpu().numpy()
    assert (c[:, 2] > c[:, 0]).all() and (c[:, 3] >= c[:, 1]).all()
