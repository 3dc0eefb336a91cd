"""The C-ABI library loads, exports what include/moe.h declares, and validates on the host.

No GPU here: only calls that must fail validation (or do nothing, T == 0) are made. A call that
got past validation would try a kernel launch and report MOE_ERR_HIP, so every expected status
below also shows that nothing was enqueued.
"""

import ctypes
import os
import re

import pytest

import sparse_moe_layer_router_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A = 0x100000          # fake, 256-byte aligned "device" addresses: never dereferenced by validation
B = 0x200000


def header_functions():
    inc = os.path.join(ROOT, "include")
    src = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert {"moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_layer_forward",
            "moe_workspace_bytes", "moe_status_string"} <= set(names)
    lib = ctypes.CDLL(moe.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(moe.EXPORTED)


def dsv3(T=8, **kw):
    s = dict(T=T, d_model=7168, n_experts=256, top_k=8, d_hidden=2048, d_shared_hidden=2048, dtype=moe.MOE_BF16)
    s.update(kw)
    return moe.make_shape(**s)


def test_workspace_bytes():
    s = dsv3()
    n = moe.moe_workspace_bytes(s)
    # at least the hidden rows and outputs of T*k routed + T shared rows
    assert n >= (8 * 8 * 2048 + 8 * 2048) * 2 + (8 * 8 + 8) * 7168 * 2
    assert n % 256 == 0
    assert moe.moe_workspace_bytes(dsv3(T=256)) > n
    assert moe.moe_workspace_bytes(dsv3(top_k=300)) == 0     # invalid shape
    assert moe.moe_workspace_bytes(moe.make_shape(0, 64, 8, 2, 128, 0, "f32")) > 0


def layer(shape, **over):
    args = dict(x=A, w_router=A, logit_bias=None, w_gate=A, w_up=A, w_down=A, w_shared_gate=A, w_shared_up=A,
                w_shared_down=A, out=B, workspace=(A, 1 << 40), stream=0)
    args.update(over)
    return args


def status_of(fn, *a, **k):
    try:
        fn(*a, **k)
        return moe.MOE_OK
    except moe.MoeError as e:
        return e.status


@pytest.mark.parametrize("shape,status", [
    (dict(top_k=257), moe.MOE_ERR_INVALID_ARG),
    (dict(top_k=0), moe.MOE_ERR_INVALID_ARG),
    (dict(T=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(n_experts=2048, top_k=8), moe.MOE_ERR_UNSUPPORTED),
    (dict(d_model=7164), moe.MOE_ERR_ALIGNMENT),
    (dict(d_hidden=2047), moe.MOE_ERR_ALIGNMENT),
    (dict(d_shared_hidden=12), moe.MOE_ERR_ALIGNMENT),
    (dict(dtype=7), moe.MOE_ERR_UNSUPPORTED),
    (dict(T=300_000_000), moe.MOE_ERR_UNSUPPORTED),
    (dict(routing=2), moe.MOE_ERR_UNSUPPORTED),
    (dict(routing=-1), moe.MOE_ERR_UNSUPPORTED),
])
def test_shape_validation(shape, status):
    s = dsv3(**shape)
    assert status_of(moe.moe_layer_forward, s, **layer(s)) == status
    assert status_of(moe.moe_route, s, A, A, None, None, A, A, (A, 1 << 40), 0) == status
    assert status_of(moe.moe_permute, s, A, None, A, A, A, (A, 1 << 40), 0) == status
    assert status_of(moe.moe_grouped_ffn, s, A, A, A, A, A, A, B, (A, 1 << 40), 0) == status
    assert status_of(moe.moe_combine, s, A, A, A, None, B, 0) == status


@pytest.mark.parametrize("name,value,status", [
    ("x", None, moe.MOE_ERR_INVALID_ARG),
    ("x", A + 8, moe.MOE_ERR_ALIGNMENT),
    ("w_router", None, moe.MOE_ERR_INVALID_ARG),
    ("w_gate", None, moe.MOE_ERR_INVALID_ARG),
    ("w_down", A + 4, moe.MOE_ERR_ALIGNMENT),
    ("w_shared_up", None, moe.MOE_ERR_INVALID_ARG),
    ("out", None, moe.MOE_ERR_INVALID_ARG),
    ("logit_bias", A + 2, moe.MOE_ERR_ALIGNMENT),
    ("workspace", None, moe.MOE_ERR_WORKSPACE),
    ("workspace", (A, 1024), moe.MOE_ERR_WORKSPACE),
    ("workspace", (A + 16, 1 << 40), moe.MOE_ERR_ALIGNMENT),
])
def test_pointer_and_workspace_validation(name, value, status):
    s = dsv3()
    assert status_of(moe.moe_layer_forward, s, **layer(s, **{name: value})) == status


def test_shared_pointers_optional_without_shared_expert_and_empty_batch_is_a_no_op():
    s = dsv3(T=0, d_shared_hidden=0)
    assert status_of(moe.moe_layer_forward, s, **layer(s, w_shared_gate=None, w_shared_up=None,
                                                        w_shared_down=None)) == moe.MOE_OK
    assert status_of(moe.moe_route, s, A, A, None, None, A, A, (A, 1 << 40), 0) == moe.MOE_OK
    assert status_of(moe.moe_permute, s, A, None, A, A, A, (A, 1 << 40), 0) == moe.MOE_OK
    assert status_of(moe.moe_grouped_ffn, s, A, None, A, A, A, A, B, (A, 1 << 40), 0) == moe.MOE_OK
    assert status_of(moe.moe_combine, s, A, A, A, None, B, 0) == moe.MOE_OK


def test_route_needs_workspace_only_without_logits_out():
    s = dsv3()
    assert status_of(moe.moe_route, s, A, A, None, None, A, A, None, 0) == moe.MOE_ERR_WORKSPACE
    s0 = dsv3(T=0)
    assert status_of(moe.moe_route, s0, A, A, None, B, A, A, None, 0) == moe.MOE_OK


def test_status_strings_and_stage_names():
    assert moe.moe_status_string(moe.MOE_OK) == "ok"
    assert "workspace" in moe.moe_status_string(moe.MOE_ERR_WORKSPACE)
    assert moe.moe_status_string(99) == "unknown status"
    s = dsv3()
    names = [moe.moe_stage_kernel_name(s, i) for i in range(moe.MOE_NUM_STAGES)]
    assert names[5] == "" and "gate_up" in names[6] and "down" in names[7]     # decode: GEMV, no schedule
    # decode-sized batch: top-k, softmax and dispatch in one launch, the permute stages launch nothing
    assert names[1] == "route_tail_small_kernel<4, 0>" and names[2:5] == ["", "", ""]
    assert moe.moe_stage_kernel_name(dsv3(T=16, top_k=256), 1) == "route_tail_small_kernel<4, 0>"   # 4096 slots
    assert moe.moe_stage_kernel_name(dsv3(T=17), 1) == "route_topk_kernel<4, 0>"
    assert moe.moe_stage_kernel_name(dsv3(T=17), 2) == "permute_count_kernel"
    assert moe.moe_stage_kernel_name(dsv3(T=256), 1) == "route_topk_kernel<4, 0>"
    names = [moe.moe_stage_kernel_name(dsv3(T=8192), i) for i in range(moe.MOE_NUM_STAGES)]
    assert names[0] == "grouped_gemm_kernel<2, 0>" and names[1] == "route_topk_kernel<4, 0>"
    assert names[2:5] == ["permute_count_kernel", "permute_scan_kernel", "permute_scatter_kernel"]
    assert names[5] == "gemm_schedule_kernel"
    sig = moe.MOE_ROUTING_SIGMOID
    assert moe.moe_stage_kernel_name(dsv3(routing=sig), 1) == "route_tail_small_kernel<4, 1>"
    assert moe.moe_stage_kernel_name(dsv3(T=4096, routing=sig), 1) == "route_topk_kernel<4, 1>"
    assert moe.moe_stage_kernel_name(dsv3(T=4096, n_experts=8, top_k=2, routing=sig), 1) == "route_topk_kernel<1, 1>"
    assert names[6] == "grouped_gemm_kernel<0, 0>" and names[7] == "grouped_gemm_kernel<1, 0>"
    packed = dsv3(T=8, weight_layout=moe.MOE_LAYOUT_FRAG16)
    assert moe.moe_stage_kernel_name(packed, 6) == "ffn_gate_up_stream_pair<1, 1>"
    # router logits: one wave per (token, expert) up to 16 tokens, MFMA tiles up to 2047, the GEMM after
    assert moe.moe_stage_kernel_name(dsv3(T=16), 0) == "route_logits_valu<1>"
    assert moe.moe_stage_kernel_name(dsv3(T=256), 0) == "route_logits_mfma"
    assert moe.moe_stage_kernel_name(dsv3(T=2048), 0) == "grouped_gemm_kernel<2, 0>"
    # more than 16 tokens, bf16: two token tiles per pass over the weights (NTT = 2)
    assert moe.moe_stage_kernel_name(dsv3(T=256, weight_layout=moe.MOE_LAYOUT_FRAG16), 6) == "ffn_gate_up_stream<2, 1>"
    assert moe.moe_stage_kernel_name(dsv3(T=256, weight_layout=moe.MOE_LAYOUT_FRAG16), 7) == "ffn_down_stream<2, 1>"
    assert moe.moe_stage_kernel_name(dsv3(top_k=0), 0) == ""


@pytest.mark.parametrize("shape,status", [
    (dict(weight_layout=moe.MOE_LAYOUT_INT8_FRAG), moe.MOE_OK),
    (dict(weight_layout=moe.MOE_LAYOUT_INT8_FRAG, dtype=moe.MOE_F32), moe.MOE_ERR_UNSUPPORTED),
    (dict(weight_layout=moe.MOE_LAYOUT_INT8_FRAG, d_model=7200), moe.MOE_ERR_ALIGNMENT),
    (dict(weight_layout=moe.MOE_LAYOUT_INT8_FRAG, d_hidden=2080), moe.MOE_ERR_ALIGNMENT),
    (dict(weight_layout=moe.MOE_LAYOUT_INT8_FRAG, d_shared_hidden=2080), moe.MOE_ERR_ALIGNMENT),
    (dict(weight_layout=moe.MOE_LAYOUT_FP8_FRAG), moe.MOE_OK),
    (dict(weight_layout=moe.MOE_LAYOUT_FP8_FRAG, dtype=moe.MOE_F32), moe.MOE_ERR_UNSUPPORTED),
    (dict(weight_layout=moe.MOE_LAYOUT_FP8_FRAG, d_model=7200), moe.MOE_ERR_ALIGNMENT),
    (dict(weight_layout=moe.MOE_LAYOUT_FP8_FRAG, d_hidden=2080), moe.MOE_ERR_ALIGNMENT),
    (dict(weight_layout=4), moe.MOE_ERR_UNSUPPORTED),
])
def test_int8_layout_validation(shape, status):
    s = dsv3(**shape)
    assert moe.moe_workspace_bytes(s) > 0 if status == moe.MOE_OK else moe.moe_workspace_bytes(s) == 0
    if status != moe.MOE_OK:
        assert status_of(moe.moe_layer_forward, s, **layer(s)) == status


@pytest.mark.parametrize("layout,code", [(moe.MOE_LAYOUT_INT8_FRAG, 2), (moe.MOE_LAYOUT_FP8_FRAG, 3)])
def test_one_byte_stage_names_follow_the_rows_per_expert(layout, code):
    """One-byte weights stream at decode sizes and take the grouped GEMM at prefill sizes, as bf16."""
    assert moe.moe_stage_kernel_name(dsv3(weight_layout=layout), 6) == f"ffn_gate_up_stream_pair<1, {code}>"
    assert moe.moe_stage_kernel_name(dsv3(weight_layout=layout), 7) == f"ffn_down_stream<1, {code}>"
    big = dsv3(T=8192, weight_layout=layout)
    assert moe.moe_stage_kernel_name(big, 5) == "gemm_schedule_kernel"
    assert moe.moe_stage_kernel_name(big, 6) == f"grouped_gemm_kernel<0, {code}>"
    assert moe.moe_stage_kernel_name(big, 7) == f"grouped_gemm_kernel<1, {code}>"


def test_load_stats_validation():
    s = dsv3()
    assert status_of(moe.moe_load_stats, s, None, 0.01, A, A) == moe.MOE_ERR_INVALID_ARG
    assert status_of(moe.moe_load_stats, s, A + 2, 0.01, A, A) == moe.MOE_ERR_ALIGNMENT
    assert status_of(moe.moe_load_stats, s, A, 0.01, A + 2, A) == moe.MOE_ERR_ALIGNMENT
    assert status_of(moe.moe_load_stats, dsv3(T=0), None, 0.01, None, None) == moe.MOE_OK
    assert status_of(moe.moe_load_stats, dsv3(top_k=0), A, 0.01, A, A) == moe.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("q", [moe.moe_quantize_weights, moe.moe_quantize_weights_fp8])
def test_quantize_weights_validation(q):
    assert moe.moe_quantized_weight_bytes(2, 16, 64) == 2 * 16 * 64 + 2 * 16 * 4
    assert moe.moe_quantized_weight_bytes(-1, 16, 64) == 0
    assert status_of(q, A, B, 1, 8, 64) == moe.MOE_ERR_ALIGNMENT      # rows % 16
    assert status_of(q, A, B, 1, 16, 32) == moe.MOE_ERR_ALIGNMENT     # cols % 64
    assert status_of(q, A, B, -1, 16, 64) == moe.MOE_ERR_INVALID_ARG
    assert status_of(q, None, B, 1, 16, 64) == moe.MOE_ERR_INVALID_ARG
    assert status_of(q, A + 8, B, 1, 16, 64) == moe.MOE_ERR_ALIGNMENT
    assert status_of(q, A, A + 1024, 1, 16, 64) == moe.MOE_ERR_INVALID_ARG   # overlapping
    assert status_of(q, None, None, 0, 16, 64) == moe.MOE_OK                 # nothing to do


@pytest.mark.parametrize("layout", [moe.MOE_LAYOUT_INT8_FRAG, moe.MOE_LAYOUT_FP8_FRAG])
def test_dequantize_weights_validation(layout):
    dq = moe.moe_dequantize_weights
    for other in (moe.MOE_LAYOUT_ROWMAJOR, moe.MOE_LAYOUT_FRAG16, 4):
        assert status_of(dq, A, other, B, 1, 16, 64) == moe.MOE_ERR_UNSUPPORTED
    assert status_of(dq, A, layout, B, 1, 8, 64) == moe.MOE_ERR_ALIGNMENT       # rows % 16
    assert status_of(dq, A, layout, B, 1, 16, 32) == moe.MOE_ERR_ALIGNMENT      # cols % 64
    assert status_of(dq, A, layout, B, -1, 16, 64) == moe.MOE_ERR_INVALID_ARG
    assert status_of(dq, A, layout, None, 1, 16, 64) == moe.MOE_ERR_INVALID_ARG
    assert status_of(dq, A, layout, B + 4, 1, 16, 64) == moe.MOE_ERR_ALIGNMENT
    assert status_of(dq, A, layout, A + 1024, 1, 16, 64) == moe.MOE_ERR_INVALID_ARG   # overlapping
    assert status_of(dq, None, layout, None, 0, 16, 64) == moe.MOE_OK                 # nothing to do


def test_empty_batch_accepts_null_tensors():
    s = dsv3(T=0)
    assert status_of(moe.moe_layer_forward, s, **layer(s, x=None, out=None, workspace=None)) == moe.MOE_OK
    assert status_of(moe.moe_combine, s, None, None, None, None, None, 0) == moe.MOE_OK
    # an invalid shape is still reported when T == 0
    assert status_of(moe.moe_layer_forward, dsv3(T=0, top_k=0), **layer(s)) == moe.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("shape,status", [
    (dict(weight_layout=7), moe.MOE_ERR_UNSUPPORTED),
    (dict(weight_layout=moe.MOE_LAYOUT_FRAG16, dtype=moe.MOE_F32), moe.MOE_ERR_UNSUPPORTED),
    (dict(weight_layout=moe.MOE_LAYOUT_FRAG16, d_model=7176), moe.MOE_ERR_ALIGNMENT),
    (dict(weight_layout=moe.MOE_LAYOUT_FRAG16, d_hidden=2056), moe.MOE_ERR_ALIGNMENT),
    (dict(weight_layout=moe.MOE_LAYOUT_FRAG16, d_shared_hidden=2056), moe.MOE_ERR_ALIGNMENT),
    (dict(weight_layout=moe.MOE_LAYOUT_FRAG16), moe.MOE_ERR_HIP),   # valid: reaches the launch (no GPU here)
])
def test_weight_layout_validation(shape, status):
    s = dsv3(**shape)
    if status == moe.MOE_ERR_HIP:
        assert moe.moe_workspace_bytes(s) > 0
        return
    assert status_of(moe.moe_layer_forward, s, **layer(s)) == status


def test_pack_weights_validation():
    assert status_of(moe.moe_pack_weights, A, B, 2, 24, 64) == moe.MOE_ERR_ALIGNMENT
    assert status_of(moe.moe_pack_weights, A, B, 2, 32, 48) == moe.MOE_ERR_ALIGNMENT
    assert status_of(moe.moe_pack_weights, A, A + 1024, 2, 32, 64) == moe.MOE_ERR_INVALID_ARG   # overlap
    assert status_of(moe.moe_pack_weights, None, B, 2, 32, 64) == moe.MOE_ERR_INVALID_ARG
    assert status_of(moe.moe_pack_weights, A + 8, B, 2, 32, 64) == moe.MOE_ERR_ALIGNMENT
    assert status_of(moe.moe_pack_weights, A, B, 0, 32, 64) == moe.MOE_OK
    assert status_of(moe.moe_pack_weights, A, B, -1, 32, 64) == moe.MOE_ERR_INVALID_ARG


def gelu_args(**over):
    args = dict(x=A, perm_src=A, expert_offsets=A, w1=A, b1=None, w2=A, b2=None, y=B, workspace=(A, 1 << 40),
                stream=0)
    args.update(over)
    return args


@pytest.mark.parametrize("shape,over,status", [
    (dict(dtype=moe.MOE_F32), {}, moe.MOE_ERR_UNSUPPORTED),
    (dict(weight_layout=moe.MOE_LAYOUT_INT8_FRAG), {}, moe.MOE_ERR_UNSUPPORTED),
    (dict(top_k=0), {}, moe.MOE_ERR_INVALID_ARG),
    ({}, dict(w1=None), moe.MOE_ERR_INVALID_ARG),
    ({}, dict(w2=A + 8), moe.MOE_ERR_ALIGNMENT),
    ({}, dict(b1=A + 2), moe.MOE_ERR_ALIGNMENT),
    ({}, dict(b2=A + 1), moe.MOE_ERR_ALIGNMENT),
    ({}, dict(expert_offsets=None), moe.MOE_ERR_INVALID_ARG),
    ({}, dict(y=None), moe.MOE_ERR_INVALID_ARG),
    ({}, dict(workspace=None), moe.MOE_ERR_WORKSPACE),
    ({}, dict(workspace=(A, 1024)), moe.MOE_ERR_WORKSPACE),
    (dict(T=0), dict(x=None, perm_src=None, expert_offsets=None, w1=None, w2=None, y=None, workspace=None), moe.MOE_OK),
])
def test_gelu_ffn_validation(shape, over, status):
    s = dsv3(**dict(dict(d_shared_hidden=0), **shape))
    assert status_of(moe.moe_grouped_ffn_gelu, s, **gelu_args(**over)) == status


def test_gelu_kernel_names():
    assert moe.moe_gelu_kernel_name(dsv3(d_shared_hidden=0), 0) == "ffn_gelu_stream<1, 0, true>"
    assert moe.moe_gelu_kernel_name(dsv3(T=256, weight_layout=moe.MOE_LAYOUT_FRAG16), 1) == \
        "ffn_gelu_stream<2, 1, false>"
    assert moe.moe_gelu_kernel_name(dsv3(), 2) == ""
    assert moe.moe_gelu_kernel_name(dsv3(dtype=moe.MOE_F32), 0) == ""
    assert moe.moe_gelu_kernel_name(dsv3(weight_layout=moe.MOE_LAYOUT_INT8_FRAG), 0) == ""


def test_noalloc_validation():
    """The no-allocation layer refuses shapes beyond its fixed scratch and invalid shapes before
    touching a device, and returns at once for an empty batch."""
    big = dsv3(T=8192, weight_layout=moe.MOE_LAYOUT_FRAG16)
    assert moe.moe_workspace_bytes(big) > moe.MOE_NOALLOC_SCRATCH_BYTES
    args = dict(layer(big))
    del args["workspace"]
    assert status_of(moe.moe_layer_forward_noalloc, big, **args) == moe.MOE_ERR_TOO_LARGE
    assert moe.moe_workspace_bytes(dsv3(T=401)) <= moe.MOE_NOALLOC_SCRATCH_BYTES < moe.moe_workspace_bytes(dsv3(T=402))
    assert status_of(moe.moe_layer_forward_noalloc, dsv3(top_k=300), **args) == moe.MOE_ERR_INVALID_ARG
    empty = {k: None for k in args if k != "stream"}
    assert status_of(moe.moe_layer_forward_noalloc, dsv3(T=0), **empty, stream=0) == moe.MOE_OK
    assert "no-allocation" in moe.moe_status_string(moe.MOE_ERR_TOO_LARGE)


def test_calib_probe_validation():
    """The measurement probes refuse bad arguments on the host (no GPU here: a valid call would
    reach the launch and report MOE_ERR_HIP)."""
    lib = ctypes.CDLL(moe.LIB_PATH)
    lib.moe_calib_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                          ctypes.c_void_p]
    lib.moe_calib_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p]
    assert lib.moe_calib_read_stream(A, 0, B, 1, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_calib_read_stream(None, 1024, B, 1, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_calib_read_stream(A, 1000, B, 1, None) == moe.MOE_ERR_ALIGNMENT
    assert lib.moe_calib_read_stream(A + 8, 1024, B, 1, None) == moe.MOE_ERR_ALIGNMENT
    assert lib.moe_calib_mfma(A, 0, B, None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_calib_mfma(A + 4, 10, B, None, None) == moe.MOE_ERR_ALIGNMENT
    assert lib.moe_calib_mfma(A, 10, B, B + 4, None) == moe.MOE_ERR_ALIGNMENT
