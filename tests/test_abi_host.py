"""CPU-only checks of the C ABI library: it loads, exports every entry point declared in
include/dflash.h, and its host-side validation and workspace sizing behave as documented.
No call here reaches the GPU."""
import ctypes
import os
import re
from dataclasses import replace

import pytest

from block_diffusion_drafting_concat_amd import binding, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "dflash.h")).read()
    return sorted(set(re.findall(r"\b(dflash_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = binding.lib()
    names = _declared()
    assert len(names) >= 8
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    L = binding.lib()
    assert L.dflash_status_string(0) == b"ok"
    assert L.dflash_status_string(-3) == b"workspace too small"


@pytest.mark.parametrize("bad", [
    dict(head_dim=96), dict(n_kv_heads=3), dict(block_size=1), dict(vocab=4100),
    dict(hidden=200), dict(mask_token_id=4096), dict(block_size=40),
])
def test_invalid_configs_are_rejected_without_gpu(bad):
    spec = replace(synth.WORKLOADS["tiny_fp32_b1"].spec, **bad)
    cfg = binding.make_config(spec)
    assert binding.workspace_bytes(cfg, binding.DFLASH_OP_PROPOSE, 1, 128) == 0
    L = binding.lib()
    st = L.dflash_propose_block(ctypes.byref(cfg), None, None, 1, None, None, 0, None, None, None, None, 0, None)
    assert st < 0
    assert L.dflash_last_error() != b""


def test_argument_errors_and_empty_calls():
    spec = synth.WORKLOADS["tiny_fp32_b1"].spec
    cfg = binding.make_config(spec)
    L = binding.lib()
    # batch 0 / n_rows 0 are no-ops that succeed before touching any pointer
    assert L.dflash_propose_block(ctypes.byref(cfg), None, None, 0, None, None, 0, None, None, None, None, 0,
                                  None) == 0
    assert L.dflash_inject_context_kv(ctypes.byref(cfg), None, None, None, 256, 0, None, None, None, 0, None) == 0
    assert L.dflash_greedy_verify(0, 7, None, None, None, None, None, None) == 0
    # NULL weights with work to do
    assert L.dflash_propose_block(ctypes.byref(cfg), None, None, 1, None, None, 0, None, None, None, None, 0,
                                  None) == -1
    assert L.dflash_greedy_verify(1, 0, None, None, None, None, None, None) == -2
    assert L.dflash_greedy_verify(1, 64, None, None, None, None, None, None) == -2
    assert L.dflash_greedy_verify(1, 7, None, None, None, None, None, None) == -1
    assert L.dflash_build_rope_table(63, 1e6, 10, None, None, None) == -1
    # verify with counters: stats is required; prepare: argument ranges and empty calls
    assert L.dflash_greedy_verify_stats(0, 7, None, None, None, None, None, None, None) == 0
    assert L.dflash_greedy_verify_stats(1, 7, None, None, None, None, None, None, None) == -1
    assert L.dflash_greedy_verify_stats(1, 64, None, None, None, None, None, None, None) == -1
    assert L.dflash_prepare_proposal_inputs(0, 3, None, 10, None, 0, None, None, None, 4, 16, None, None, None,
                                            None, None) == 0
    assert L.dflash_prepare_proposal_inputs(0, 3, None, 10, None, 2, None, None, None, 4, 16, None, None, None,
                                            None, None) == -1
    assert L.dflash_prepare_proposal_inputs(1, 64, None, 10, None, 0, None, None, None, 4, 16, None, None, None,
                                            None, None) == -2
    assert L.dflash_prepare_proposal_inputs(1, 3, None, 10, None, 0, None, None, None, 4, 0, None, None, None,
                                            None, None) == -1
    assert L.dflash_prepare_proposal_inputs(1, 3, None, 10, None, 0, None, None, None, 4, 16, None, None, None,
                                            None, None) == -1


def test_workspace_sizes_grow_with_work_and_are_bounded():
    spec = synth.QWEN3_8B_DRAFTER
    cfg = binding.make_config(spec)
    p1 = binding.workspace_bytes(cfg, binding.DFLASH_OP_PROPOSE, 1, 2048)
    p32 = binding.workspace_bytes(cfg, binding.DFLASH_OP_PROPOSE, 32, 8192)
    assert 0 < p1 < p32 < 2 << 30
    i16 = binding.workspace_bytes(cfg, binding.DFLASH_OP_INJECT, 16)
    ibig = binding.workspace_bytes(cfg, binding.DFLASH_OP_INJECT, 1 << 20)
    assert 0 < i16 < ibig < 1 << 30  # rows are processed in bounded chunks
