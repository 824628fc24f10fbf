"""The C ABI library: it loads, exports every declared symbol, and rejects bad
arguments before touching the GPU (these run on a machine without one)."""
import ctypes
import os
import re
import subprocess

import pytest

from sparse_moe_transformer_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ffn.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_ffn_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libmoe_ffn.so is not built (run python -m sparse_moe_transformer_amd.build)")
    return binding.lib()


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert set(binding.EXPORTS) == set(names), names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (moe_ffn_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_header_constants_match_binding():
    """Every MOE_FFN_* enum value in the header equals the binding's constant."""
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    consts = dict(re.findall(r"\b(MOE_FFN_[A-Z0-9_]+)\s*=\s*(-?\d+)", src))
    assert "MOE_FFN_NUM_STAGES" in consts and "MOE_FFN_STAGE_GEGLU" in consts
    for name, val in consts.items():
        assert getattr(binding, name) == int(val), name


def cfg(**kw):
    base = dict(hidden=2816, num_experts=128, top_k=8, expert_dim=704, dense_dim=2112, max_tokens=16)
    base.update(kw)
    return binding.make_config(**base)


def test_workspace_bytes_valid_config(lib):
    rc, n = binding.moe_ffn_workspace_bytes(cfg())
    assert rc == binding.MOE_FFN_OK
    # at least y = T*k*H bf16 and h = T*k*I bf16
    assert n >= 16 * 8 * (2816 + 704) * 2


@pytest.mark.parametrize("kw,code", [
    (dict(hidden=2800), binding.MOE_FFN_ERR_UNSUPPORTED),
    (dict(hidden=4352), binding.MOE_FFN_ERR_UNSUPPORTED),
    (dict(expert_dim=4160), binding.MOE_FFN_ERR_UNSUPPORTED),
    # no experts (a dense FFN) needs top_k = expert_dim = 0 and dense_dim > 0
    (dict(num_experts=0), binding.MOE_FFN_ERR_INVALID_ARG),
    (dict(num_experts=0, top_k=0), binding.MOE_FFN_ERR_INVALID_ARG),
    (dict(num_experts=0, top_k=0, expert_dim=0, dense_dim=0), binding.MOE_FFN_ERR_INVALID_ARG),
    (dict(dense_dim=16448), binding.MOE_FFN_ERR_UNSUPPORTED),
    (dict(num_experts=126), binding.MOE_FFN_ERR_UNSUPPORTED),
    (dict(num_experts=300), binding.MOE_FFN_ERR_UNSUPPORTED),
    (dict(top_k=0), binding.MOE_FFN_ERR_UNSUPPORTED),
    (dict(top_k=17), binding.MOE_FFN_ERR_UNSUPPORTED),
    (dict(num_experts=4, top_k=5), binding.MOE_FFN_ERR_UNSUPPORTED),
    (dict(expert_dim=700), binding.MOE_FFN_ERR_UNSUPPORTED),
    (dict(dense_dim=-64), binding.MOE_FFN_ERR_UNSUPPORTED),
    (dict(dense_dim=100), binding.MOE_FFN_ERR_UNSUPPORTED),
    (dict(max_tokens=0), binding.MOE_FFN_ERR_INVALID_ARG),
    # 2^20 tokens: h [T*8, 704] bf16 would reach 11.8 GB (32-bit operand offsets)
    (dict(max_tokens=1 << 20), binding.MOE_FFN_ERR_UNSUPPORTED),
    (dict(weight_format=7), binding.MOE_FFN_ERR_UNSUPPORTED),
    (dict(weight_format=3), binding.MOE_FFN_ERR_UNSUPPORTED),
    (dict(flags=2), binding.MOE_FFN_ERR_UNSUPPORTED),
])
def test_bad_configs_rejected(lib, kw, code):
    rc, _ = binding.moe_ffn_workspace_bytes(cfg(**kw))
    assert rc == code
    assert binding.moe_ffn_last_error() != ""
    rc, h = binding.moe_ffn_create(cfg(**kw))
    assert rc == code and not h


def test_dense_ffn_configs_accepted(lib):
    """A config without experts is the dense FFN of the E4B model (2560 ->
    10240 -> 2560); wide dense branches are accepted with experts too."""
    rc, n = binding.moe_ffn_workspace_bytes(cfg(hidden=2560, num_experts=0, top_k=0, expert_dim=0,
                                                dense_dim=10240, max_tokens=4096))
    assert rc == binding.MOE_FFN_OK
    assert n >= 4096 * 10240 * 2 + 4096 * 2560 * 2  # h_d and y_d rows
    rc, _ = binding.moe_ffn_workspace_bytes(cfg(dense_dim=16384))
    assert rc == binding.MOE_FFN_OK


def test_fp8_config_accepted(lib):
    rc, _ = binding.moe_ffn_workspace_bytes(cfg(weight_format=binding.MOE_FFN_W_FP8))
    assert rc == binding.MOE_FFN_OK


def test_largest_addressable_token_count(lib):
    # T*k*I*2 < 2^31 at the 26B shape: up to 190,650 tokens
    rc, _ = binding.moe_ffn_workspace_bytes(cfg(max_tokens=190650))
    assert rc == binding.MOE_FFN_OK
    rc, _ = binding.moe_ffn_workspace_bytes(cfg(max_tokens=190651))
    assert rc == binding.MOE_FFN_ERR_UNSUPPORTED


def test_null_arguments(lib):
    assert lib.moe_ffn_workspace_bytes(None, None) == binding.MOE_FFN_ERR_INVALID_ARG
    assert lib.moe_ffn_create(None, None) == binding.MOE_FFN_ERR_INVALID_ARG
    assert binding.moe_ffn_forward(None, 8, *([None] * 11)) == binding.MOE_FFN_ERR_INVALID_ARG
    assert binding.moe_ffn_forward_nvfp4(None, 8, *([None] * 11)) == binding.MOE_FFN_ERR_INVALID_ARG
    assert binding.moe_ffn_forward_fp8(None, 8, *([None] * 11)) == binding.MOE_FFN_ERR_INVALID_ARG
    assert binding.moe_ffn_get_routing(None, *([None] * 7)) == binding.MOE_FFN_ERR_INVALID_ARG
    assert binding.moe_ffn_get_intermediates(None, *([None] * 5)) == binding.MOE_FFN_ERR_INVALID_ARG
    assert binding.moe_ffn_align_only(None, 4, None, None) == binding.MOE_FFN_ERR_INVALID_ARG
    assert binding.moe_ffn_set_variant(None, 0) == binding.MOE_FFN_ERR_INVALID_ARG
    assert binding.moe_ffn_destroy(None) == binding.MOE_FFN_OK
    assert "NULL" in binding.moe_ffn_last_error()


def test_last_error_never_null(lib):
    assert isinstance(lib.moe_ffn_last_error(), bytes)


def test_noalloc_validation_before_any_gpu_call(lib):
    """The no-allocation forward validates its config, T and pointers before
    any HIP call: NULL config, a non-bf16 format, T out of range and a
    workspace beyond the static scratch are refused; T = 0 is a no-op."""
    f = binding.moe_ffn_forward_noalloc
    ptrs = [256 * (i + 1) for i in range(11)]  # never dereferenced: each call is refused or T == 0
    assert f(None, 8, *ptrs) == binding.MOE_FFN_ERR_INVALID_ARG
    assert f(cfg(weight_format=binding.MOE_FFN_W_NVFP4), 8, *ptrs) == binding.MOE_FFN_ERR_UNSUPPORTED
    assert f(cfg(max_tokens=16), 17, *ptrs) == binding.MOE_FFN_ERR_INVALID_ARG
    assert f(cfg(max_tokens=16), -1, *ptrs) == binding.MOE_FFN_ERR_INVALID_ARG
    # 64 MiB of scratch: at the 26B shape T = 446 fits, T = 447 does not
    assert f(cfg(max_tokens=447), 447, *ptrs) == binding.MOE_FFN_ERR_UNSUPPORTED
    assert "static scratch" in binding.moe_ffn_last_error()
    rc, n = binding.moe_ffn_workspace_bytes(cfg(max_tokens=446))
    assert rc == binding.MOE_FFN_OK and n <= 64 << 20
    assert f(cfg(max_tokens=446), 0, *ptrs) == binding.MOE_FFN_OK
