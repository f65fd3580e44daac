"""dflash_propose_block_noalloc, the proposal on the library's static device scratch (for
callers that cannot allocate), against dflash_propose_block with a caller workspace: the same
kernels on the same inputs, so draft ids, drafts and final hidden rows must be bit-identical.
Two calls in a row share the scratch, the second on a smaller input (a Qwen3-8B-shaped batch-1
proposal over a 2048-token context, then a small drafter's), so stale scratch contents from the
first call must not leak into the second."""
import numpy as np
import pytest
import torch

from block_diffusion_drafting_concat_amd import binding, synth
from tests.gpu_helpers import Setup

pytestmark = pytest.mark.gpu

SMALL_BF16 = synth.DrafterSpec(hidden=256, n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=128,
                               intermediate=512, vocab=2048, n_aux=2, target_hidden=192, block_size=16,
                               mask_token_id=2047, rope_theta=1e6, dtype="bf16")


def _both(st, bonus):
    spec = st.spec
    K = spec.block_size - 1
    bonus_d = torch.from_numpy(np.asarray(bonus, np.int32)).cuda()
    ctx_d = torch.from_numpy(st.ctx).cuda()
    res = []
    for noalloc in (False, True):
        out = (torch.full((st.B, K + 1), -7, dtype=torch.int32, device="cuda"),
               torch.full((st.B, K), -7, dtype=torch.int32, device="cuda"))
        hid = torch.full((st.B * K, spec.hidden), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            st.dev.propose_noalloc(st.cache, bonus_d, ctx_d, st.max_ctx, out=out, hidden_out=hid)
        else:
            st.dev.propose(st.cache, bonus_d, ctx_d, st.max_ctx, st.ws_prop, out=out, hidden_out=hid)
        torch.cuda.synchronize()
        res.append((out[0].cpu(), out[1].cpu(), hid.cpu()))
    return res


def test_noalloc_matches_the_workspace_entry_point_on_two_calls():
    wl = synth.WORKLOADS["qwen3_8b_b1_ctx2048"]
    cases = [(wl.spec, synth.context_lengths(wl), wl.seed), (SMALL_BF16, np.array([40], np.int32), 8)]
    need = []
    for spec, ctx, seed in cases:
        print(f"\n[case] noalloc {spec.hidden}x{spec.n_layers} ctx {ctx.tolist()}", flush=True)
        st = Setup(spec, ctx, seed=seed)
        need.append(binding.workspace_bytes(st.dev.cfg, binding.DFLASH_OP_PROPOSE, st.B, st.max_ctx))
        (i0, d0, h0), (i1, d1, h1) = _both(st, (np.arange(st.B) * 53 + 11) % spec.vocab)
        assert torch.equal(i0, i1) and torch.equal(d0, d1)
        assert torch.equal(h0.view(torch.int32), h1.view(torch.int32)), "hidden rows differ"
        assert not torch.isnan(h1).any()
        del st
    assert need[1] < need[0] <= 64 << 20

