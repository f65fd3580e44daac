"""GPU parity (through the C ABI) of the step's integer bookkeeping against the CPU oracle:
greedy verification with the fused acceptance counters, and the proposal-input preparation
that corrects an optimistic schedule. Both are bit-exact integer work."""
import numpy as np
import pytest
import torch

from block_diffusion_drafting_concat_amd import binding
from oracle import dflash_oracle as O

pytestmark = pytest.mark.gpu


def _rounds(rng, B, K, V):
    d = rng.integers(0, V, size=(B, K)).astype(np.int32)
    t = rng.integers(0, V, size=(B, K + 1)).astype(np.int32)
    for b in range(B):
        n = rng.integers(0, K + 1)
        t[b, :n] = d[b, :n]
    t[0, :K] = d[0]  # one full acceptance
    return d, t


def test_verify_stats_accumulate_the_acceptance_counters():
    rng = np.random.default_rng(5)
    for K, V in [(15, 151936), (9, 128256), (1, 3), (63, 7)]:
        stats = torch.zeros(3, dtype=torch.int64, device="cuda")
        all_a = []
        for B in (1, 37, 256):
            d, t = _rounds(rng, B, K, V)
            acc, out, nb = binding.verify_with_stats(torch.from_numpy(d).cuda(), torch.from_numpy(t).cuda(), stats)
            ra, ro, rn = O.greedy_verify(d, t)
            assert np.array_equal(acc.cpu().numpy(), ra) and np.array_equal(out.cpu().numpy(), ro)
            assert np.array_equal(nb.cpu().numpy(), rn)
            all_a.append(ra)
        m = O.acceptance_metrics(np.concatenate(all_a), K)
        got = stats.cpu().numpy()
        assert got.tolist() == [m["num_drafts"], m["num_draft_tokens"], m["num_accepted_tokens"]], (K, got, m)
        print(f"[case] K={K}: acceptance rate {got[2] / got[1]:.3f}, length {1 + got[2] / got[0]:.3f}", flush=True)


def _prepare_case(rng, B, K, V, P, maxb, neg=False):
    prev = rng.integers(0, V, size=(B, K + 1)).astype(np.int32)
    for b in range(B):
        a = rng.integers(0 if neg else 1, K + 2)
        prev[b, a:] = -1
        if rng.random() < 0.2 and a > 0:
            prev[b, rng.integers(0, a)] = V + rng.integers(0, 3)  # out-of-vocabulary entries are invalid
    opt_seq = rng.integers(0 if neg else K + 1, 4000, size=B).astype(np.int32)
    per = rng.integers(0, 5, size=B)
    req = np.repeat(np.arange(B), per).astype(np.int32)
    opt_pos = np.concatenate([opt_seq[b] + np.arange(per[b]) for b in range(B)] or [np.zeros(0)]).astype(np.int32)
    bt = rng.permutation(B * maxb).reshape(B, maxb).astype(np.int32)
    return prev, opt_seq, req, opt_pos, bt


@pytest.mark.parametrize("B,K,V,P,maxb", [(1, 15, 151936, 16, 256), (32, 15, 151936, 16, 512),
                                          (128, 9, 128256, 16, 256), (7, 0, 50, 1, 4000), (64, 63, 1000, 64, 64)])
def test_prepare_matches_oracle(B, K, V, P, maxb):
    rng = np.random.default_rng(B * 100 + K)
    for neg in (False, True):
        prev, opt_seq, req, opt_pos, bt = _prepare_case(rng, B, K, V, P, maxb, neg)
        ref = O.prepare_proposal_inputs(prev, V, opt_seq, req, opt_pos, bt, P)
        cu = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
        seq, pos, slots, bonus = binding.prepare(cu(prev), V, cu(opt_seq), cu(req), cu(opt_pos), cu(bt), P)
        torch.cuda.synchronize()
        assert np.array_equal(seq.cpu().numpy(), ref["seq_lens"]), (B, K, neg)
        assert np.array_equal(pos.cpu().numpy(), ref["positions"]), (B, K, neg)
        assert np.array_equal(slots.cpu().numpy(), ref["slot_mapping"]), (B, K, neg)
        assert np.array_equal(bonus.cpu().numpy(), ref["bonus"]), (B, K, neg)


def test_verify_then_prepare_recovers_the_synchronous_schedule():
    """On the device, verification followed by preparation gives the true post-verify lengths,
    the verify's next bonus, and the slots of the true context positions (the valid-count
    identity of [N] "Async Rejection and Position Correction")."""
    rng = np.random.default_rng(11)
    B, K, V, P, maxb = 48, 15, 151936, 16, 300
    d, t = _rounds(rng, B, K, V)
    dd, tt = torch.from_numpy(d).cuda(), torch.from_numpy(t).cuda()
    acc, out, nb = binding.verify(dd, tt)
    c = rng.integers(0, 4000, size=B).astype(np.int32)
    opt_seq = torch.from_numpy(c + K + 1).cuda()
    per = np.full(B, K + 1)
    req = np.repeat(np.arange(B), per).astype(np.int32)
    opt_pos = np.concatenate([c[b] + K + 1 + np.arange(per[b]) for b in range(B)]).astype(np.int32)
    bt = rng.permutation(B * maxb).reshape(B, maxb).astype(np.int32)
    seq, pos, slots, bonus = binding.prepare(out, V, opt_seq, torch.from_numpy(req).cuda(),
                                             torch.from_numpy(opt_pos).cuda(), torch.from_numpy(bt).cuda(), P)
    a = acc.cpu().numpy()
    true_seq = c + a
    true_pos = np.concatenate([true_seq[b] + np.arange(per[b]) for b in range(B)])
    assert np.array_equal(seq.cpu().numpy(), true_seq)
    assert np.array_equal(bonus.cpu().numpy(), nb.cpu().numpy())
    assert np.array_equal(pos.cpu().numpy(), true_pos)
    assert np.array_equal(slots.cpu().numpy(), O.paged_slots(bt, req, true_pos, P))
