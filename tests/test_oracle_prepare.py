"""Pins of the oracle's proposal-input preparation ([N] "Async Rejection and Position
Correction"): it must undo an optimistic schedule exactly, in agreement with the independently
written greedy verification (the valid-count identity: the previous output holds a valid
tokens, so (1 + K) - valid is the number of rejected positions)."""
import numpy as np
import pytest

from oracle import greedy_verify, paged_slots, prepare_proposal_inputs


def _random_round(rng, B, K, V):
    drafts = rng.integers(0, V, size=(B, K))
    target = rng.integers(0, V, size=(B, K + 1))
    # copy a random-length prefix so that every acceptance length occurs
    for b in range(B):
        n = rng.integers(0, K + 1)
        target[b, :n] = drafts[b, :n]
    return drafts, target


@pytest.mark.parametrize("K", [1, 3, 9, 15])
def test_prepare_undoes_the_optimistic_schedule(K):
    rng = np.random.default_rng(K)
    B, V, P = 7, 50, 4
    max_blocks = 64
    block_table = rng.permutation(B * max_blocks).reshape(B, max_blocks)
    c = rng.integers(0, 100, size=B)  # context length before the verified block
    drafts, target = _random_round(rng, B, K, V)
    a, out, next_bonus = greedy_verify(drafts, target)
    # the next step injects n_b new context rows per request, right after the accepted ones
    n_rows_per = rng.integers(1, 4, size=B)
    row_req = np.repeat(np.arange(B), n_rows_per)
    true_seq = c + a
    true_pos = np.concatenate([true_seq[b] + np.arange(n_rows_per[b]) for b in range(B)])
    # the optimistic schedule assumed all K drafts plus the bonus were accepted
    opt_seq = c + K + 1
    opt_pos = np.concatenate([opt_seq[b] + np.arange(n_rows_per[b]) for b in range(B)])
    r = prepare_proposal_inputs(out, V, opt_seq, row_req, opt_pos, block_table, P)
    np.testing.assert_array_equal(r["seq_lens"], true_seq)
    np.testing.assert_array_equal(r["positions"], true_pos)
    np.testing.assert_array_equal(r["bonus"], next_bonus)
    np.testing.assert_array_equal(r["num_rejected"], K + 1 - a)
    np.testing.assert_array_equal(r["slot_mapping"], paged_slots(block_table, row_req, true_pos, P))


def test_full_acceptance_is_the_identity_and_out_of_vocab_entries_are_invalid():
    V, P = 10, 16
    bt = np.arange(8).reshape(2, 4)
    prev = np.array([[3, 4, 5, 6], [7, 8, 9, 10]])  # 10 == V: not a valid token
    r = prepare_proposal_inputs(prev, V, [40, 50], [0, 1], [40, 50], bt, P)
    np.testing.assert_array_equal(r["num_rejected"], [0, 1])
    np.testing.assert_array_equal(r["seq_lens"], [40, 49])
    np.testing.assert_array_equal(r["bonus"], [6, 9])
    np.testing.assert_array_equal(r["slot_mapping"], [bt[0, 2] * P + 8, bt[1, 3] * P + 1])


def test_worked_example_positions_after_full_acceptance():
    """[V]'s worked example: seq_lens [10, 8, 12] with K = 3. A fully accepted previous round
    leaves the block positions seq_len + j unchanged, and their slots follow the page table."""
    K, V, P = 3, 1000, 16
    bt = np.array([[0, 1], [2, 3], [4, 5]])
    prev = np.array([[1, 2, 3, 100], [4, 5, 6, 200], [7, 8, 9, 300]])
    seq = np.array([10, 8, 12])
    req = np.repeat(np.arange(3), K + 1)
    pos = np.concatenate([s + np.arange(K + 1) for s in seq])
    r = prepare_proposal_inputs(prev, V, seq, req, pos, bt, P)
    np.testing.assert_array_equal(r["positions"], [10, 11, 12, 13, 8, 9, 10, 11, 12, 13, 14, 15])
    np.testing.assert_array_equal(r["bonus"], [100, 200, 300])
    np.testing.assert_array_equal(r["slot_mapping"], bt[req, 0] * P + pos)


def test_negative_corrected_position_is_skipped():
    r = prepare_proposal_inputs(np.array([[-1, -1, -1]]), 5, [1], [0], [1], np.array([[3]]), 4)
    assert r["num_rejected"][0] == 3 and r["positions"][0] == -2 and r["slot_mapping"][0] == -1
    assert r["bonus"][0] == 0
