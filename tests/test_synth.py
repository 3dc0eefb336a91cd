"""Seeded input generator: determinism, distribution, layout and bf16 rounding (no GPU)."""

import ctypes

import numpy as np
import pytest
import scipy.stats
import torch

import synth


def test_philox_known_answers():
    """Philox4x32-10 known-answer vectors published with the Random123 library."""
    lib = synth._load()
    kat = [([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
           ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
           ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
            [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1])]
    lib.syn_philox_raw.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.c_uint32, ctypes.c_uint32]
    for ctr, key, want in kat:
        a = (ctypes.c_uint32 * 4)(*ctr)
        lib.syn_philox_raw(a, key[0], key[1])
        assert list(a) == want


def test_deterministic_and_stream_separated():
    a = synth.normal_host((1000,), 0, synth.stream_id(synth.K_X), 1.0, "f32")
    b = synth.normal_host((1000,), 0, synth.stream_id(synth.K_X), 1.0, "f32")
    c = synth.normal_host((1000,), 0, synth.stream_id(synth.K_WG), 1.0, "f32")
    d = synth.normal_host((1000,), 1, synth.stream_id(synth.K_X), 1.0, "f32")
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c) and not np.array_equal(a, d)


def test_standard_normal_distribution():
    a = synth.normal_host((4_000_000,), 7, synth.stream_id(synth.K_X), 1.0, "f32").astype(np.float64)
    assert abs(a.mean()) < 3e-3 and abs(a.std() - 1) < 3e-3
    assert abs(scipy.stats.kurtosis(a, fisher=False) - 3.0) < 0.02
    assert scipy.stats.kstest(a[:1_000_000], "norm").pvalue > 1e-3


def test_weight_std_is_one_over_sqrt_fan_in():
    w = synth.normal_host((256, 7168), 0, synth.stream_id(synth.K_WG), synth.weight_std(7168), "f32")
    assert abs(w.std() - 1 / np.sqrt(7168)) < 2e-4


def test_bf16_is_round_to_nearest_even_of_the_f32_draw():
    f = synth.normal_host((200_000,), 3, synth.stream_id(synth.K_GATE, 5), 0.37, "f32")
    b = synth.normal_host((200_000,), 3, synth.stream_id(synth.K_GATE, 5), 0.37, "bf16")
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(b, ref)


def test_block_layout_matches_per_expert_streams_and_offsets():
    cfg = synth.LayerConfig("t", 4, 16, 3, 2, 8, 0, "bf16")
    g, u, dn = synth.all_expert_weights_host(cfg, 0)
    for e in range(3):
        ge, ue, de = synth.expert_weights_host(cfg, 0, e)
        assert np.array_equal(g[e], ge) and np.array_equal(u[e], ue) and np.array_equal(dn[e], de)
    full = synth.normal_host((999,), 0, synth.stream_id(synth.K_X), 1.0, "f32")
    for first in (1, 2, 5):
        part = synth.normal_host((50,), 0, synth.stream_id(synth.K_X), 1.0, "f32", first=first)
        assert np.array_equal(part, full[first:first + 50])


def test_zipf_bias_matches_scipy_zipfian():
    b = synth.zipf_logit_bias(8, 1.2)
    pmf = scipy.stats.zipfian(1.2, 8).pmf(np.arange(1, 9))
    np.testing.assert_allclose(b, (2 * np.log(pmf)).astype(np.float32), rtol=1e-6)
    np.testing.assert_allclose(b[:3], [-1.694, -3.358, -4.331], atol=1e-3)


def test_redraw_replaces_only_named_rows():
    inp = synth.host_small_inputs(synth.CONFIGS[0], 0)
    x0 = inp.x.copy()
    synth.redraw_rows(inp, [3, 5])
    changed = np.nonzero(np.any(inp.x != x0, axis=1))[0].tolist()
    assert changed == [3, 5] and inp.redraws == {3: 1, 5: 1}


def test_config_table_shapes():
    c = synth.CONFIG_BY_NAME
    assert (c["tiny_fp32"].T, c["tiny_fp32"].d, c["tiny_fp32"].E, c["tiny_fp32"].k) == (16, 64, 8, 2)
    d = c["dsv3_decode_t8"]
    assert (d.T, d.d, d.E, d.k, d.H, d.Hs, d.dtype) == (8, 7168, 256, 8, 2048, 2048, "bf16")
    assert c["dsv3_decode_t256"].T == 256 and c["dsv3_prefill_t8192"].T == 8192
    s = c["skewed_mixtral_t4096"]
    assert (s.T, s.d, s.E, s.k, s.H, s.Hs, s.zipf_s) == (4096, 4096, 8, 2, 14336, 0, 1.2)
