"""CPU-side checks of the C ABI: the library loads and exports every entry
point that include/dmx.h declares; the host bucket rule equals the oracle's
bit for bit over every length; argument validation fails before any launch."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def dmx():
    import masked_gqa_attention_action_amd as m
    m.lib()
    return m


def declared_functions():
    src = open(os.path.join(ROOT, "include", "dmx.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dmx_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol(dmx):
    names = declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(dmx.lib(), n), n
    assert set(names) == set(dmx.EXPORTED)


@pytest.mark.parametrize("buckets,cap,mt", [
    ((576, 704, 768, 896, 1024), 1024, 0), ((576, 704, 768, 896, 1024), 1024, 650), ((2048,), 2048, 0),
    ((576, 704), 1024, 0), ((576, 704, 768, 896, 1024), 2048, 0), ((704, 576), 1024, 0), ((), 1024, 0),
    ((576, 2048), 1024, 0), ((1, 2, 3), 3, 2), ((576, 576), 1024, 0), ((0, 576), 1024, 0),
])
def test_bucket_rule_bit_exact_against_oracle(dmx, buckets, cap, mt):
    for ln in range(-3, cap + 100):
        assert dmx.select_bucket(ln, buckets, cap, mt) == orc.select_bucket(ln, buckets, cap, mt), (ln, buckets)
    for cap2, mt2 in ((0, 0), (cap, -1)):
        assert dmx.select_bucket(10, buckets, cap2, mt2) == orc.select_bucket(10, buckets, cap2, mt2)


def test_workspace_sizes(dmx):
    assert dmx.workspace_bytes(1, 50, 1024) > 0
    assert dmx.workspace_bytes(16, 50, 1024) > dmx.workspace_bytes(1, 50, 1024)
    assert dmx.workspace_bytes(1, 2048, 0) >= 2048 * 4096 * 4
    assert dmx.workspace_bytes(0, 50, 1024) == 0
    assert dmx.workspace_bytes(1, 0, 1024) == 0
    assert dmx.workspace_bytes(1, 50, -1) == 0
    L = dmx.lib()
    assert L.dmx_stack_mod_table_bytes(18, 10, 1) == 10 * 18 * 2 * 1 * 3 * 1024 * 4
    assert L.dmx_stack_mod_table_bytes(18, 10, 4) == 4 * L.dmx_stack_mod_table_bytes(18, 10, 1)
    assert L.dmx_stack_mod_table_bytes(0, 10, 1) == 0
    assert L.dmx_stack_mod_table_bytes(18, 0, 1) == 0
    assert L.dmx_stack_mod_table_bytes(18, 10, 0) == 0


FAKE = ctypes.c_void_p(0x10000)      # aligned, never dereferenced: validation fails first
ODD = ctypes.c_void_p(0x10001)


def test_validation_errors_before_launch(dmx):
    L = dmx.lib()
    st = L.dmx_adarms_prenorm(None, FAKE, FAKE, FAKE, 1, 50, FAKE, FAKE, None)
    assert st == dmx.ERR_INVALID_ARG and b"x is null" in L.dmx_last_error_string()
    assert L.dmx_adarms_prenorm(ODD, FAKE, FAKE, FAKE, 1, 50, FAKE, FAKE, None) == dmx.ERR_MISALIGNED
    assert L.dmx_adarms_prenorm(FAKE, FAKE, FAKE, FAKE, 0, 50, FAKE, FAKE, None) == dmx.ERR_UNSUPPORTED
    assert L.dmx_qkv_qknorm_rope(FAKE, FAKE, FAKE, FAKE, 1, 50, 2048, FAKE, 10000.0, FAKE, FAKE, FAKE, 50, 0,
                                 FAKE, 1 << 30, None) == dmx.ERR_UNSUPPORTED
    assert L.dmx_qkv_qknorm_rope(FAKE, FAKE, FAKE, FAKE, 1, 50, 1024, FAKE, 10000.0, FAKE, FAKE, FAKE, 60, 20,
                                 FAKE, 1 << 30, None) == dmx.ERR_INVALID_ARG
    assert L.dmx_qkv_qknorm_rope(FAKE, FAKE, FAKE, FAKE, 1, 50, 1024, FAKE, 10000.0, FAKE, FAKE, FAKE, 50, 0,
                                 FAKE, 1024, None) == dmx.ERR_WORKSPACE
    assert L.dmx_suffix_attention(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 65, 1024, FAKE, FAKE, 1 << 30,
                                  None) == dmx.ERR_UNSUPPORTED
    assert L.dmx_suffix_attention(FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 50, 1024, FAKE, FAKE, 1 << 30,
                                  None) == dmx.ERR_INVALID_ARG
    assert L.dmx_suffix_attention(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 50, 5000, FAKE, FAKE, 1 << 30,
                                  None) == dmx.ERR_UNSUPPORTED
    assert L.dmx_oproj_gated_residual(FAKE, FAKE, FAKE, FAKE, 1, 50, FAKE, None, 1 << 30,
                                      None) == dmx.ERR_INVALID_ARG
    assert L.dmx_geglu_mlp(FAKE, FAKE, FAKE, FAKE, FAKE, 65, 50, FAKE, FAKE, 1 << 30, None) == dmx.ERR_UNSUPPORTED
    assert L.dmx_suffix_layer_forward(None, None, FAKE, FAKE, FAKE, 1, 50, FAKE, FAKE, 1 << 30,
                                      None) == dmx.ERR_INVALID_ARG
    lw = dmx.LayerWeights(*([0x10000] * 9 + [0x10008]))
    kv = dmx.PrefixKV(0x10000, 0x10000, 0x10000, 1024)
    assert L.dmx_suffix_layer_forward(ctypes.byref(lw), ctypes.byref(kv), FAKE, FAKE, FAKE, 1, 50, FAKE, FAKE,
                                      1 << 30, None) == dmx.ERR_MISALIGNED
    assert b"w_down" in L.dmx_last_error_string()
    assert L.dmx_pack_weight(None, 16, 32, FAKE, None) == dmx.ERR_INVALID_ARG
    assert L.dmx_pack_weight(FAKE, 24, 32, ctypes.c_void_p(0x90000), None) == dmx.ERR_UNSUPPORTED
    assert L.dmx_pack_weight(FAKE, 16, 48, ctypes.c_void_p(0x90000), None) == dmx.ERR_UNSUPPORTED
    assert L.dmx_pack_weight(FAKE, 16, 32, ctypes.c_void_p(0x10200), None) == dmx.ERR_INVALID_ARG  # overlap
    assert b"overlaps" in L.dmx_last_error_string()
    g = ctypes.c_void_p()
    assert L.dmx_stack_graph_create(None, FAKE, ctypes.byref(g)) == dmx.ERR_INVALID_ARG
    assert L.dmx_stack_mod_table_fill(None, FAKE, None) == dmx.ERR_INVALID_ARG
    assert L.dmx_prefix_workspace_bytes(0) == 0 and L.dmx_prefix_workspace_bytes(5000) == 0
    assert L.dmx_prefix_workspace_bytes(2048) > L.dmx_prefix_workspace_bytes(96) > 0
    assert L.dmx_prefix_attention(None, FAKE, FAKE, FAKE, 10, 10, FAKE, FAKE, 1 << 30, None) == dmx.ERR_INVALID_ARG
    assert L.dmx_prefix_attention(FAKE, FAKE, FAKE, FAKE, 20, 10, FAKE, FAKE, 1 << 30, None) == dmx.ERR_UNSUPPORTED
    assert L.dmx_prefix_attention(FAKE, FAKE, FAKE, None, 10, 10, FAKE, FAKE, 1 << 30, None) == dmx.ERR_INVALID_ARG
    assert L.dmx_prefix_attention(FAKE, FAKE, FAKE, FAKE, 2048, 2048, FAKE, FAKE, 1024, None) == dmx.ERR_WORKSPACE
    assert L.dmx_prefix_attention_workspace_bytes(0) == 0
    assert L.dmx_prefix_attention_workspace_bytes(2048) > L.dmx_prefix_attention_workspace_bytes(64) > 0
    assert L.dmx_image_merge(FAKE, FAKE, FAKE, 4, 2, 12, FAKE, None) == dmx.ERR_UNSUPPORTED
    assert L.dmx_image_merge(FAKE, FAKE, None, 4, 2, 16, FAKE, None) == dmx.ERR_INVALID_ARG
    assert L.dmx_prefix_layer_forward(None, FAKE, FAKE, 8, FAKE, FAKE, 8, FAKE, FAKE, 1 << 30,
                                      None) == dmx.ERR_INVALID_ARG
    pw = dmx.PrefixLayerWeights(*([0x10000] * 10))
    assert L.dmx_prefix_layer_forward(ctypes.byref(pw), FAKE, FAKE, 8, FAKE, FAKE, 4, ctypes.c_void_p(0x20000),
                                      FAKE, 1 << 30, None) == dmx.ERR_UNSUPPORTED  # kv_rows < tokens
    assert L.dmx_prefix_layer_forward(ctypes.byref(pw), FAKE, FAKE, 8, FAKE, FAKE, 8, ctypes.c_void_p(0x20000),
                                      FAKE, 1024, None) == dmx.ERR_WORKSPACE
    assert L.dmx_sampler_schedule_bytes(0) == 0 and L.dmx_sampler_schedule_bytes(1001) == 0
    assert L.dmx_sampler_schedule_bytes(10) > L.dmx_sampler_schedule_bytes(1) > 0
    sw = dmx.SamplerWeights(32, *([0x10000] * 10))
    assert L.dmx_sampler_schedule_fill(None, 10, 1, FAKE, FAKE, 1 << 30, None) == dmx.ERR_INVALID_ARG
    assert L.dmx_sampler_schedule_fill(ctypes.byref(sw), 0, 1, FAKE, FAKE, 1 << 30, None) == dmx.ERR_INVALID_ARG
    assert L.dmx_sampler_schedule_fill(ctypes.byref(sw), 10, 0, FAKE, FAKE, 1 << 30, None) == dmx.ERR_INVALID_ARG
    assert L.dmx_sampler_schedule_fill(ctypes.byref(sw), 10, 1, FAKE, FAKE, 64, None) == dmx.ERR_WORKSPACE
    sw_bad = dmx.SamplerWeights(24, *([0x10000] * 10))
    assert L.dmx_sampler_schedule_fill(ctypes.byref(sw_bad), 10, 1, FAKE, FAKE, 1 << 30, None) == dmx.ERR_UNSUPPORTED
    sw_mis = dmx.SamplerWeights(32, *([0x10000] * 9 + [0x10008]))
    assert L.dmx_sampler_schedule_fill(ctypes.byref(sw_mis), 10, 1, FAKE, FAKE, 1 << 30, None) == dmx.ERR_MISALIGNED
    assert L.dmx_sampler_forward(None, None) == dmx.ERR_INVALID_ARG
    assert L.dmx_sampler_graph_create(None, FAKE, ctypes.byref(g)) == dmx.ERR_INVALID_ARG
    assert L.dmx_graph_launch(None, None) == dmx.ERR_INVALID_ARG
    L.dmx_graph_destroy(None)
    for s in (0, 1, -1, -2, -3, -4, -5, -6, -7, -99):
        assert L.dmx_status_string(s)


def test_noalloc_layer_validates_before_any_device_call(dmx):
    """The allocation-free layer call refuses null pointers and sizes beyond
    its fixed scratch on the host, before it touches the device."""
    L = dmx.lib()
    lw = dmx.LayerWeights(*([0x10000] * 10))
    assert L.dmx_suffix_layer_forward_noalloc(None, None, FAKE, FAKE, FAKE, 1, 50, FAKE, None) == dmx.ERR_INVALID_ARG
    kv = dmx.PrefixKV(0x10000, 0x10000, 0x10000, 2048)
    st = L.dmx_suffix_layer_forward_noalloc(ctypes.byref(lw), ctypes.byref(kv), FAKE, FAKE, FAKE, 2, 64, FAKE, None)
    assert st == dmx.ERR_WORKSPACE and b"scratch" in L.dmx_last_error_string()
    assert L.dmx_workspace_bytes(1, 64, 2048) <= dmx.NOALLOC_SCRATCH_BYTES < L.dmx_workspace_bytes(2, 64, 2048)


def test_stack_checks_x_and_pos0_against_the_batch(dmx):
    """Stack() names x and pos0 when their shape or dtype does not match the
    batch cond gives (the layers write x in place and read pos0 per request);
    checked before anything touches a device."""
    import torch
    B, C, P = 2, 50, 64
    cond = torch.zeros((3, B, 1024), dtype=torch.bfloat16)
    mask = torch.zeros((B, P), dtype=torch.uint8)
    pos0 = torch.zeros((B,), dtype=torch.int32)
    x_short = torch.zeros((1, C, 1024), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=r"^x: expected .*\(2, 50, 1024\)"):
        dmx.Stack([{}], [], [], mask, cond, pos0, x_short)
    x = torch.zeros((B, C, 1024), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=r"^pos0: expected .*torch.int32 \(2,\)"):
        dmx.Stack([{}], [], [], mask, cond, pos0.long(), x)
