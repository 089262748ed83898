"""Host-side boundary checks of the C ABI (CPU only: no call here touches a GPU).

Gates and error names: "Model-agnostic LLM inference", sections "Supported models"
(gate table), "Errors" and "Long context" (65,536-token ceiling).  The cache sizes in
the section "The quantized load cache" (0.598 GB / 1.724 GB) pin the packed size.
"""
import dataclasses
import os
import re

import pytest

import int8_weight_only_amd as qd
from workloads import SHAPES

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    lib = qd.load_library()
    header = open(os.path.join(ROOT, "include", "qd.h")).read()
    declared = set(re.findall(r"\b(qd_[a-z0-9_]+)\s*\(", header))
    assert {"qd_load_weights", "qd_prefill", "qd_decode_step", "qd_generate_greedy",
            "qd_free"} <= declared
    for name in declared:
        assert hasattr(lib, name), name
    assert declared == set(qd.EXPORTS)


GOOD = SHAPES["tiny"]


@pytest.mark.parametrize("field,value,needle", [
    ("n_kv_heads", 3, "% num_key_value_heads"),
    ("hidden", 100, "hidden_size 100 not divisible by 32"),
    ("intermediate", 300, "intermediate_size 300 not divisible by 32"),
    ("head_dim", 20, "num_attention_heads * head_dim = 80 not divisible by 32"),
    ("tie_word_embeddings", False, "tie_word_embeddings must be true"),
    ("attention_bias", True, "attention_bias must be false"),
])
def test_each_gate_alone(field, value, needle):
    bad = dataclasses.replace(GOOD, **{field: value})
    with pytest.raises(qd.UnsupportedArchitectureError) as e:
        qd.check_shape(bad)
    assert e.value.code == "unsupported_architecture"
    assert needle in str(e.value)


def test_all_failing_gates_are_named_together():
    bad = dataclasses.replace(GOOD, n_kv_heads=3, hidden=100, intermediate=300,
                              tie_word_embeddings=False, attention_bias=True)
    with pytest.raises(qd.UnsupportedArchitectureError) as e:
        qd.check_shape(bad)
    msg = str(e.value)
    for needle in ("% num_key_value_heads", "hidden_size 100", "intermediate_size 300",
                   "tie_word_embeddings", "attention_bias"):
        assert needle in msg


def test_own_kernel_gates():
    with pytest.raises(qd.UnsupportedArchitectureError, match="power of two"):
        qd.check_shape(dataclasses.replace(GOOD, head_dim=96, n_heads=4))
    with pytest.raises(qd.UnsupportedArchitectureError, match="> 8"):
        qd.check_shape(dataclasses.replace(GOOD, n_heads=32, n_kv_heads=2))
    with pytest.raises(qd.UnsupportedArchitectureError, match="must be > 0"):
        qd.check_shape(dataclasses.replace(GOOD, n_layers=0))


@pytest.mark.parametrize("name", ["tiny", "qwen3-0.6b", "qwen3-1.7b"])
def test_supported_shapes_pass(name):
    qd.check_shape(SHAPES[name])


def test_packed_size_matches_the_pages_cache_sizes():
    s06 = qd.query_sizes(SHAPES["qwen3-0.6b"], 1, 512, 512)
    s17 = qd.query_sizes(SHAPES["qwen3-1.7b"], 1, 512, 512)
    assert round(s06["packed_model_bytes"] / 1e9, 3) == 0.598
    assert round(s17["packed_model_bytes"] / 1e9, 3) == 1.724
    # the device arena holds exactly that plus alignment padding and the RoPE table
    rope = 512 * 64 * 8
    assert 0 <= s06["weight_bytes"] - s06["packed_model_bytes"] - rope < 256 * 400


def test_kv_bytes_formula():
    s = SHAPES["qwen3-0.6b"]
    sz = qd.query_sizes(s, 4, 1024, 1024)
    assert sz["kv_bytes"] == s.n_layers * 2 * 4 * s.n_kv_heads * 1024 * s.head_dim * 2


def test_context_ceiling_and_limits():
    with pytest.raises(qd.QdError) as e:
        qd.query_sizes(GOOD, 1, 65537, 16)
    assert e.value.code == "context_ceiling"
    qd.query_sizes(GOOD, 1, 65536, 16)
    with pytest.raises(qd.QdError) as e:
        qd.query_sizes(GOOD, 0, 512, 16)
    assert e.value.code == "invalid_arguments"
    with pytest.raises(qd.QdError) as e:
        qd.query_sizes(GOOD, 65, 512, 16)
    assert e.value.code == "invalid_arguments"
    with pytest.raises(qd.QdError) as e:
        qd.query_sizes(GOOD, 1, 512, 0)
    assert e.value.code == "invalid_arguments"
    with pytest.raises(qd.QdError) as e:  # prefill attention takes at most 65535 row tiles
        qd.query_sizes(GOOD, 1, 512, 4000001)
    assert e.value.code == "invalid_arguments"


def test_prefill_tokens_bounded_by_32_bit_gemm_offsets():
    """The prefill GEMM reads each [tokens, width] bf16 operand through 32-bit byte offsets:
    tokens x widest row x 2 must stay below 2 GiB (tiny: widest row 384, the intermediate)."""
    cap = (2 ** 31 - 1) // (2 * 384)
    qd.query_sizes(GOOD, 1, 512, cap)
    with pytest.raises(qd.QdError) as e:
        qd.query_sizes(GOOD, 1, 512, cap + 1)
    assert e.value.code == "invalid_arguments" and "32-bit" in str(e.value)
    # Qwen3-1.7B: the widest row is the 6144-wide intermediate
    cap17 = (2 ** 31 - 1) // (2 * 6144)
    qd.query_sizes(SHAPES["qwen3-1.7b"], 1, 512, cap17)
    with pytest.raises(qd.QdError):
        qd.query_sizes(SHAPES["qwen3-1.7b"], 1, 512, cap17 + 1)


def test_run_op_rejects_a_null_model_on_the_host():
    import ctypes
    lib = qd.load_library()
    st = lib.qd_run_op(None, 1, 0, 1, None, None, None, None, None)
    assert st == 2 and b"model is NULL" in lib.qd_last_error()


def test_binding_count_mismatches_are_argument_errors():
    """A slot or seed list whose length differs from the batch is an argument error
    ("Model-agnostic LLM inference", section "Errors": invalid_arguments), raised by the
    binding before any library call."""
    torch = pytest.importorskip("torch")
    m = object.__new__(qd.Model)          # no device buffers: only the argument checks run
    m.shape, m.device, m._h = GOOD, torch.device("cpu"), None
    with pytest.raises(qd.QdError) as e:
        m.decode_step(torch.zeros(2, dtype=torch.int32), slots=[0, 1, 2])
    assert e.value.code == "invalid_arguments"
    logits = torch.zeros((2, GOOD.vocab), dtype=torch.float32)
    with pytest.raises(qd.QdError) as e:
        m.sample(logits, seeds=[1, 2, 3])
    assert e.value.code == "invalid_arguments"
    with pytest.raises(qd.QdError) as e:
        m.sample(logits, seeds=[1, 2], slots=[0])
    assert e.value.code == "invalid_arguments"
