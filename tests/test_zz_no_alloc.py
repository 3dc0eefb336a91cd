"""moe_layer_forward_noalloc (the layer on the library's fixed per-GPU scratch, no workspace
argument) against moe_layer_forward with a caller workspace, through the C ABI (needs an MI355X).

Two calls in a row on the same GPU, the second with a smaller input, each bitwise equal to the
workspace entry point on the same inputs (the same kernels run; the second call must not see
anything the first left in the shared scratch). Shapes beyond the scratch are refused."""

import pytest
import torch

import synth
from synth import LayerConfig
from tests import gpu_util as G

import sparse_moe_layer_router_amd as moe

pytestmark = pytest.mark.gpu


def run_both(L):
    c = L.cfg
    dt = G.TORCH_DT[c.dtype]
    res = []
    for noalloc in (True, False):
        out = torch.full((c.T, c.d), float("nan"), dtype=dt, device="cuda")
        idx = torch.full((c.T, c.k), -1, dtype=torch.int32, device="cuda")
        w = torch.full((c.T, c.k), float("nan"), dtype=torch.float32, device="cuda")
        counts = torch.full((c.E,), -1, dtype=torch.int32, device="cuda")
        logits = torch.full((c.T, c.E), float("nan"), dtype=torch.float32, device="cuda")
        args = (L.shape, L.x, L.w_router, L.bias, L.w_gate, L.w_up, L.w_down, L.ws_gate, L.ws_up, L.ws_down, out,
                idx, w, counts, logits)
        if noalloc:
            moe.moe_layer_forward_noalloc(*args)
        else:
            moe.moe_layer_forward(*args, workspace=moe.allocate_workspace(L.shape))
        torch.cuda.synchronize()
        res.append([t.cpu() for t in (out, idx, w, counts, logits)])
    return res


def bits(t):
    """Bit patterns, so that equality is exact (NaN included)."""
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else (t.view(torch.int32) if t.dtype == torch.float32 else t)


# a grouped-GEMM layer (about 75 rows per expert, shared expert), then a smaller weight-streaming
# one with the same weights
BIG = LayerConfig("noalloc_gemm", 600, 264, 16, 2, 200, 136, "bf16")


@pytest.mark.parametrize("layout", [moe.MOE_LAYOUT_ROWMAJOR], ids=["rowmajor"])
def test_noalloc_matches_workspace_entry_point_twice(layout):
    small = synth.with_tokens(BIG, 37)
    weights = G.make_weights(BIG, 0, host_copy=True)
    for cfg in (BIG, small):
        print(f"[noalloc] T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} moe_layer_forward_noalloc vs moe_layer_forward",
              flush=True)
        L = G.make_layer(cfg, weights=weights, layout=layout)
        got, ref = run_both(L)
        for name, a, b in zip(("out", "topk_idx", "topk_w", "counts", "logits"), got, ref):
            assert torch.equal(bits(a), bits(b)), name
        assert torch.isfinite(got[0].float()).all()


def test_noalloc_refuses_shapes_beyond_its_scratch():
    s = moe.make_shape(8192, 7168, 256, 8, 2048, 2048, "bf16", moe.MOE_LAYOUT_FRAG16)
    assert moe.moe_workspace_bytes(s) > moe.MOE_NOALLOC_SCRATCH_BYTES
    with pytest.raises(moe.MoeError) as e:
        moe.moe_layer_forward_noalloc(s, 0x100000, 0x100000, None, 0x100000, 0x100000, 0x100000, 0x100000,
                                      0x100000, 0x100000, 0x200000)
    assert e.value.status == moe.MOE_ERR_TOO_LARGE
