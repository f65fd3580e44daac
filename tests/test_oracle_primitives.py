"""Pins of the oracle's primitives against things other than the oracle itself:
torch's bf16 cast, hand-worked rounding cases, a complex-number statement of RoPE,
torch's scaled-dot-product attention, and the mathematical properties of each."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import dflash_oracle as O


# ---------------------------------------------------------------- bf16 rounding
def test_round_bf16_matches_torch_cast_on_fp32_inputs():
    g = np.random.default_rng(1)
    x = np.concatenate([
        g.standard_normal(200_000).astype(np.float32),
        (g.standard_normal(20_000) * 1e-39).astype(np.float32),  # subnormal range
        (g.standard_normal(20_000) * 1e30).astype(np.float32),
        np.float32([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-45, np.inf, -np.inf]),
    ])
    # exact ties: bf16 keeps the top 16 bits; set the dropped 16 bits to 0x8000
    bits = g.integers(0, 2**32, size=50_000, dtype=np.uint64).astype(np.uint32)
    bits = (bits & np.uint32(0x7F7F0000)) | np.uint32(0x8000)
    x = np.concatenate([x, bits.view(np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    got = O.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)


def test_round_bf16_hand_cases():
    # spacing of bf16 just above 1 is 2^-7
    assert O.round_bf16(1 + 2**-8) == 1.0  # tie -> even (mantissa ...0)
    assert O.round_bf16(1 + 3 * 2**-8) == 1 + 2**-6  # tie -> even (mantissa ...10)
    assert O.round_bf16(1 + 2**-8 + 2**-30) == 1 + 2**-7  # above the tie
    assert O.round_bf16(-(1 + 2**-8)) == -1.0
    assert O.round_bf16(2**-133) == 2**-133  # smallest subnormal
    assert O.round_bf16(2**-135) == 0.0  # below half of it
    assert np.isinf(O.round_bf16(3.5e38))


def test_round_f32_is_ieee_single():
    assert O.round_f32(1 + 2**-24) == 1.0
    assert O.round_f32(1 + 3 * 2**-24) == 1 + 2**-22
    x = np.random.default_rng(2).standard_normal(1000)
    assert np.array_equal(O.round_f32(x), torch.from_numpy(x).float().double().numpy())


# ---------------------------------------------------------------- RMSNorm
def test_rms_norm_matches_torch_functional():
    g = np.random.default_rng(3)
    x = g.standard_normal((7, 96))
    w = 1 + 0.1 * g.standard_normal(96)
    want = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(w), eps=1e-6)
    np.testing.assert_allclose(O.rms_norm(x, w, 1e-6), want.numpy(), rtol=1e-12, atol=1e-12)


def test_rms_norm_scale_invariance_and_unit_rms():
    g = np.random.default_rng(4)
    x = g.standard_normal((5, 64))
    y = O.rms_norm(x, np.ones(64), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-13)
    np.testing.assert_allclose(O.rms_norm(37.5 * x, np.ones(64), 0.0), y, rtol=1e-12)


# ---------------------------------------------------------------- RoPE
def _rope_complex(x, pos, theta):
    """RoPE as complex multiplication: z_i = x_i + 1j*x_{i+D/2} turned by pos * theta^(-2i/D)."""
    D = x.shape[-1]
    z = x[..., : D // 2] + 1j * x[..., D // 2:]
    freq = np.exp(-np.log(theta) * np.arange(0, D, 2) / D)
    z = z * np.exp(1j * np.asarray(pos, np.float64)[..., None] * freq)
    return np.concatenate([z.real, z.imag], axis=-1)


@pytest.mark.parametrize("D,theta", [(64, 1e6), (128, 1e6), (128, 5e5), (8, 10000.0)])
def test_rope_equals_complex_rotation(D, theta):
    g = np.random.default_rng(5)
    x = g.standard_normal((11, 3, D))
    pos = g.integers(0, 40000, size=(11, 1))
    np.testing.assert_allclose(O.apply_rope(x, pos, theta), _rope_complex(x, pos, theta),
                               rtol=1e-9, atol=1e-9)


def test_rope_properties():
    g = np.random.default_rng(6)
    D = 128
    q, k = g.standard_normal(D), g.standard_normal(D)
    # position 0 is the identity
    np.testing.assert_array_equal(O.apply_rope(q, 0, 1e6), q)
    # each (i, i + D/2) pair keeps its norm
    r = O.apply_rope(q, 12345, 1e6)
    np.testing.assert_allclose(r[:64] ** 2 + r[64:] ** 2, q[:64] ** 2 + q[64:] ** 2, rtol=1e-12)
    # the score depends only on the position difference
    s1 = O.apply_rope(q, 1000, 1e6) @ O.apply_rope(k, 990, 1e6)
    s2 = O.apply_rope(q, 31000, 1e6) @ O.apply_rope(k, 30990, 1e6)
    np.testing.assert_allclose(s1, s2, rtol=1e-9)


# ---------------------------------------------------------------- attention
def _sdpa(q, k, v):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v))[0, 0].numpy()


def test_attention_matches_torch_sdpa_noncausal():
    g = np.random.default_rng(7)
    for tq, tk, d in [(16, 16, 64), (16, 300, 128), (10, 1, 128), (4, 2063, 32)]:
        q, k, v = g.standard_normal((tq, d)), g.standard_normal((tk, d)), g.standard_normal((tk, d))
        np.testing.assert_allclose(O.attention(q, k, v), _sdpa(q, k, v), rtol=1e-10, atol=1e-12)


def test_attention_special_cases():
    g = np.random.default_rng(8)
    q = g.standard_normal((5, 16))
    k1, v1 = g.standard_normal((1, 16)), g.standard_normal((1, 16))
    np.testing.assert_allclose(O.attention(q, k1, v1), np.repeat(v1, 5, 0), rtol=1e-14)
    k = np.repeat(g.standard_normal((1, 16)), 9, 0)
    v = g.standard_normal((9, 16))
    np.testing.assert_allclose(O.attention(q, k, v), np.repeat(v.mean(0, keepdims=True), 5, 0),
                               rtol=1e-12)
    # permuting keys together with their values changes nothing
    k, v = g.standard_normal((30, 16)), g.standard_normal((30, 16))
    perm = g.permutation(30)
    np.testing.assert_allclose(O.attention(q, k[perm], v[perm]), O.attention(q, k, v), rtol=1e-12)


# ---------------------------------------------------------------- paged slots
def test_paged_slots_hand_worked(golden_dir):
    with open(os.path.join(golden_dir, "paged_slots_examples.json")) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        got = O.paged_slots(case["block_table"], case["req"], case["pos"], case["page_size"])
        assert got.tolist() == case["slot"]


# ---------------------------------------------------------------- query block
def test_query_block_matches_vllm_worked_example(golden_dir):
    with open(os.path.join(golden_dir, "vllm_first_pass_example.json")) as f:
        gold = json.load(f)
    K = gold["num_speculative_tokens"]
    M = 128002
    ids, pos, keep, qsl = O.build_query_block(gold["next_token_ids"], gold["seq_lens"], K + 1, M)
    want_ids = [M if t == "M" else t for t in gold["expected_input_ids"]]
    assert ids.tolist() == want_ids
    assert pos.tolist() == gold["expected_query_positions"]
    assert keep.tolist() == gold["expected_token_indices_to_sample"]
    assert qsl.tolist() == gold["expected_query_start_loc"]
    assert int(np.max(np.diff(qsl))) == gold["expected_max_query_len"]
    assert ids.size == gold["expected_num_tokens"]
    # the context rows of that step are the last query_len positions before each seq_len
    ctx = np.concatenate([np.arange(s - q, s) for s, q in zip(gold["seq_lens"], gold["query_lens"])])
    assert ctx.tolist() == gold["target_positions"]
