"""CPU checks of the C-ABI library: it loads, exports every function include/beamattn.h
declares, and its host-only functions behave. No GPU work is launched here: the
argument checks fail before any HIP call."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "beamattn.h")
LIB = os.path.join(ROOT, "nope_gqa_attention_amd", "libbeamattn.so")
DEBUG_LIB = os.path.join(ROOT, "nope_gqa_attention_amd", "libbeamattn_debug.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(beam_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libbeamattn.so is not built (python -m nope_gqa_attention_amd.build)")
    import torch  # noqa: F401  (torch's HIP runtime first, as in real use)
    return ctypes.CDLL(LIB)


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("beam_qknorm_rope_ssmax_kvwrite", "beam_attn_prefill", "beam_attn_decode",
              "beam_head_gate"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_debug_library_loads_and_exports_every_declared_symbol():
    """The BEAMATTN_DEBUG build (device-side batch-metadata checks) is built beside the
    library and exports the same interface."""
    if not os.path.exists(DEBUG_LIB):
        pytest.fail("libbeamattn_debug.so is not built (python -m nope_gqa_attention_amd.build --debug)")
    import torch  # noqa: F401
    dbg = ctypes.CDLL(DEBUG_LIB)
    missing = [n for n in declared_functions() if not hasattr(dbg, n)]
    assert not missing, missing


def test_binding_names_match_header():
    from nope_gqa_attention_amd import beamattn as ba
    assert sorted(ba.ENTRY_POINTS) == declared_functions()
    for n in declared_functions():
        assert callable(getattr(ba, n))


def test_host_only_functions(lib):
    from nope_gqa_attention_amd import beamattn as ba
    ba.load(LIB)
    assert ba.beam_abi_version() == ba.BEAM_ABI_VERSION
    assert ba.beam_kv_bytes_per_token(9, 8, 128, ba.BEAM_KV_BF16) == 36 * 1024
    assert ba.beam_kv_bytes_per_token(9, 8, 128, ba.BEAM_KV_FP8_E4M3) == 18 * 1024
    assert ba.beam_kv_bytes_per_token(52, 8, 128, ba.BEAM_KV_BF16) == 208 * 1024
    assert ba.beam_kv_bytes_per_token(9, 8, 128, 7) == 0
    assert ba.beam_status_string(ba.BEAM_ERR_WORKSPACE) == "workspace too small"
    layer = ba.layer_desc("full")
    # one split: no workspace; long contexts: a workspace that grows with the split count
    assert ba.beam_attn_decode_workspace_bytes(layer, 1, 1, 512) == 0
    w = ba.beam_attn_decode_workspace_bytes(layer, 1, 1, 100000)
    assert w > 0 and w % (48 * 130 * 4) == 0
    assert ba.beam_attn_decode_workspace_bytes(layer, 1, 17, 100000) == 0   # invalid q_len
    swa = ba.layer_desc("swa")
    assert ba.beam_attn_decode_workspace_bytes(swa, 1, 1, 10 ** 6) == 0     # window fits one split


def test_invalid_descriptor_fails_before_any_launch(lib):
    from nope_gqa_attention_amd import beamattn as ba
    ba.load(LIB)
    layer = ba.layer_desc("full")
    layer.num_kv_heads = 5     # 48 % 5 != 0
    st = lib.beam_attn_prefill(ctypes.byref(layer), None, None, None, 0, None, 0, None, None, 0, None)
    assert st == ba.BEAM_ERR_INVALID_ARG
    assert "multiple" in ba.beam_last_error()
    layer = ba.layer_desc("swa", window=0)
    st = lib.beam_head_gate(ctypes.byref(layer), 0, None, 0, None, 0, None, None, 0, None)
    assert st == ba.BEAM_ERR_INVALID_ARG and "window" in ba.beam_last_error()
    layer = ba.layer_desc("full")
    st = lib.beam_attn_decode(ctypes.byref(layer), None, None, None, 0, None, 0, None, None, 0,
                              None, 0, None)
    assert st == ba.BEAM_ERR_INVALID_ARG and "batch" in ba.beam_last_error()
