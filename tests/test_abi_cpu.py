"""The C-ABI library without a GPU: it loads, exports every symbol include/rlt.h declares,
and validates arguments before touching the device."""
import ctypes
import os
import re
from ctypes import byref, c_void_p

import pytest

import stateful_decoding_amd as sd
from stateful_decoding_amd.binding import RLT_BF16, RLT_F32, rlt_config
from synth import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "rlt.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rlt_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sd.LIB_PATH):
        pytest.fail("librlt.so is not built: run __graft_entry__.build()")
    return sd.load_library()


CORE = ("rlt_memproj", "rlt_decoder_step", "rlt_run_sequence", "rlt_state_create",
        "rlt_state_export", "rlt_state_import", "rlt_model_create", "rlt_run_parallel",
        "rlt_bptt", "rlt_encode", "rlt_readout", "rlt_head_create", "rlt_last_error")


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(CORE) <= set(names) and len(names) >= 37, names
    raw = ctypes.CDLL(sd.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def good(**kw):
    c = sd.make_config(CONFIGS["s140m_bf16"], version=5)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("field,value,status", [
    ("dtype", 7, 3), ("d", 0, 2), ("head_dim", 48, 2), ("n_heads", 11, 2), ("ffn", 100, 2),
    ("window", 0, 2), ("window", 2000, 2), ("n_groups", 3, 2), ("alpha", float("nan"), 1),
    ("eps", -1.0, 1),
])
def test_config_validation(lib, field, value, status):
    assert lib.rlt_config_check(byref(good())) == 0
    c = good(**{field: value})
    assert lib.rlt_config_check(byref(c)) == status
    assert lib.rlt_last_error()
    assert lib.rlt_model_ws_bytes(byref(c)) == 0


def test_config_presets_are_valid(lib):
    for cfg in CONFIGS.values():
        c = sd.make_config(cfg)
        assert lib.rlt_config_check(byref(c)) == 0, lib.rlt_last_error()


def test_buffer_sizes(lib):
    c = good()
    d, L, F, G, H, hd, W = 768, 12, 3072, 12, 12, 64, 128
    # packed matrices, plus the fused output + cross-query matrices (4 d^2 per layer) and one
    # d^2 scratch block used while building them
    weights = 2 * (2 * d * d + L * (6 * d * d + 3 * d * F) + G * 2 * d * d + L * 4 * d * d + d * d)
    ws = lib.rlt_model_ws_bytes(byref(c))
    assert weights <= ws <= weights + 64 * 256 + 4 * (2 * d + 3 * L * d) + 4096
    mem = lib.rlt_memory_bytes(byref(c), 256, 1024)
    assert mem == 2 * G * 256 * H * 1024 * hd * 2
    st = lib.rlt_state_bytes(byref(c), 256)
    assert st >= 2 * L * 256 * H * W * hd * 2
    assert lib.rlt_memory_bytes(byref(c), 256, 0) == 0
    assert lib.rlt_memory_bytes(byref(c), 256, (1 << 20) + 1) == 0
    assert lib.rlt_state_bytes(byref(c), 0) == 0
    # token-parallel workspace: f32 residual stream + bf16 operands per token (at least)
    par = lib.rlt_parallel_ws_bytes(byref(c), 16, 8192)
    rows = 16 * 8192
    assert par >= rows * d * 4 + rows * (5 * d + F) * 2
    assert lib.rlt_parallel_ws_bytes(byref(c), 16, 0) == 0
    assert lib.rlt_parallel_ws_bytes(byref(c), 0, 8) == 0
    # backward workspace: five fp32 and five dtype rows per (token, sequence, layer) at least
    bw = lib.rlt_bptt_ws_bytes(byref(c), 4, 64)
    assert bw >= 4 * 64 * c.n_layers * d * (5 * 4 + 5 * 2)
    assert lib.rlt_bptt_ws_bytes(byref(c), 4, 0) == 0
    assert lib.rlt_bptt_ws_bytes(byref(c), 0, 8) == 0
    # head: embedding and readout matrix in bf16 plus the gains; vocabularies of 64k only
    V = 32768
    hw = lib.rlt_head_ws_bytes(byref(c), V)
    assert 2 * V * d * 2 + 4 * (2 * L * d + 2 * d) <= hw <= 2 * V * d * 2 + 4 * (2 * L * d + 2 * d) + 5 * 256
    for bad in (0, 100, 1000, (1 << 22) + 64):
        assert lib.rlt_head_ws_bytes(byref(c), bad) == 0
    assert lib.rlt_encode_ws_bytes(byref(c), 16, 1024) == lib.rlt_parallel_ws_bytes(byref(c), 16,
                                                                                    1024)
    assert lib.rlt_encode_ws_bytes(byref(good(dtype=RLT_F32)), 16, 1024) == 0
    ro = lib.rlt_readout_ws_bytes(byref(c), V, 256)
    assert ro >= 256 * V * 4  # logits
    assert lib.rlt_readout_ws_bytes(byref(c), V, 0) == 0


def test_null_arguments_rejected_without_gpu(lib):
    c = good()
    out = c_void_p()
    assert lib.rlt_model_create(byref(c), None, None, 0, None, byref(out)) == 1
    assert lib.rlt_state_create(None, 4, None, 0, None, byref(out)) == 1
    assert lib.rlt_memory_create(None, 4, 16, None, 0, byref(out)) == 1
    assert lib.rlt_memproj(None, None, None, 0, 1, None) == 1
    assert lib.rlt_decoder_step(None, None, None, None, None, None) == 1
    assert lib.rlt_run_sequence(None, None, None, None, 1, None, None) == 1
    assert lib.rlt_run_parallel(None, None, None, None, 1, None, None, 0, None) == 1
    assert lib.rlt_bptt(None, None, 1, 1, None, None, None, None, None, 0, None, None, None,
                         None) == 1
    assert lib.rlt_state_export(None, None, None, None, None, None, None, None) == 1
    assert lib.rlt_state_import(None, None, None, None, 0, 0, None) == 1
    assert lib.rlt_state_reset(None, None) == 1
    assert lib.rlt_profile_clock(None, None, 0) == 1
    assert lib.rlt_head_create(None, 32768, None, None, 0, None, byref(out)) == 1
    assert lib.rlt_encode(None, None, None, 1, 1, None, None, 0, None) == 1
    assert lib.rlt_readout(None, None, None, 1, None, None, None, None, None, None, None, 0,
                           None) == 1
    assert lib.rlt_state_position(None) == -1
    assert lib.rlt_memory_length(None) == -1
    assert b"NULL" in lib.rlt_last_error()


def test_dtype_codes():
    assert (RLT_F32, RLT_BF16) == (0, 1)
    assert ctypes.sizeof(rlt_config) == 48
