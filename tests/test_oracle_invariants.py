"""Invariant pins of the oracle's injection, block proposal and verification."""
import itertools

import numpy as np
import pytest

from block_diffusion_drafting_concat_amd import synth
from oracle import dflash_oracle as O
from tests.oracle_helpers import SMALL, empty_cache, filled_context, numpy_weights

W_SMALL = numpy_weights(synth.make_weights(SMALL, seed=5))


def _aux(spec, seq, n, seed=5):
    return [synth.as_f32(a) for a in synth.aux_states(spec, seed, seq, 0, n)]


# ---------------------------------------------------------------- injection
@pytest.mark.parametrize("mode", ["exact", "f32", "bf16"])
def test_incremental_injection_equals_full_recompute(mode):
    spec, W, P, n = SMALL, W_SMALL, 4, 37
    aux = _aux(spec, 0, n)
    pos = np.arange(n)
    slots = np.random.default_rng(0).permutation(12 * P)[:n]  # any distinct slots
    kf, vf = empty_cache(spec, 12, P)
    O.inject_context_kv(spec, W, kf, vf, aux, pos, slots, mode)
    ki, vi = empty_cache(spec, 12, P)
    order = np.random.default_rng(1).permutation(n)
    for chunk in np.array_split(order, 5):  # any chunking, any order
        O.inject_context_kv(spec, W, ki, vi, [a[chunk] for a in aux], pos[chunk], slots[chunk], mode)
    for l in range(spec.n_layers):
        np.testing.assert_array_equal(ki[l], kf[l])
        np.testing.assert_array_equal(vi[l], vf[l])


def test_injection_skips_negative_slots_and_touches_nothing_else():
    spec, W, P, n = SMALL, W_SMALL, 4, 10
    aux = _aux(spec, 0, n)
    kc, vc = empty_cache(spec, 6, P)
    for c in kc + vc:
        c[...] = 7.25  # canary
    slots = np.array([3, -1, 8, 9, -5, 0, 1, 2, 23, 22])
    O.inject_context_kv(spec, W, kc, vc, aux, np.arange(n), slots, "f32")
    written = np.zeros(6 * P, bool)
    written[slots[slots >= 0]] = True
    for c in kc + vc:
        flat = c.reshape(6 * P, -1)
        assert np.all(flat[~written] == 7.25)
        assert np.all(flat[written] != 7.25)


def test_injection_concat_is_block_matrix_product():
    """fc(concat(aux)) = sum_j fc[:, j-th block] aux_j: aux_j pairs with the j-th block of
    fc's input features, in ascending target-layer order."""
    spec, W, n = SMALL, W_SMALL, 6
    aux = _aux(spec, 1, n)
    kc, vc = empty_cache(spec, 4, 4)
    y = O.inject_context_kv(spec, W, kc, vc, aux, np.arange(n), np.arange(n), "exact")["y"]
    Ht = spec.target_hidden
    want = sum(aux[j].astype(np.float64) @ W["fc"][:, j * Ht:(j + 1) * Ht].T.astype(np.float64)
               for j in range(spec.n_aux))
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12)


def test_hidden_norm_makes_injection_scale_invariant():
    """Scaling every aux state by s > 0 scales fc's output by s, and hidden_norm removes it
    (the Qualcomm transform pre-scales fc for fp16 range on this basis)."""
    from dataclasses import replace
    spec, W, n = replace(SMALL, rms_eps=0.0), W_SMALL, 8  # eps = 0: exact invariance
    aux = _aux(spec, 2, n)
    k1, v1 = empty_cache(spec, 4, 4)
    k2, v2 = empty_cache(spec, 4, 4)
    O.inject_context_kv(spec, W, k1, v1, aux, np.arange(n), np.arange(n), "exact")
    O.inject_context_kv(spec, W, k2, v2, [a * 64.0 for a in aux], np.arange(n), np.arange(n), "exact")
    for l in range(spec.n_layers):
        np.testing.assert_allclose(k1[l], k2[l], rtol=1e-6, atol=1e-7)
        np.testing.assert_allclose(v1[l], v2[l], rtol=1e-6, atol=1e-7)


def test_injected_keys_at_position_zero_have_unit_rms_with_unit_norm_weight():
    from dataclasses import replace
    spec, n = replace(SMALL, rms_eps=0.0), 5
    W = dict(W_SMALL)
    for l in range(spec.n_layers):
        W[f"layers.{l}.k_norm"] = np.ones(spec.head_dim, np.float32)
    kc, vc = empty_cache(spec, 2, 4)
    O.inject_context_kv(spec, W, kc, vc, _aux(spec, 3, n), np.zeros(n, int), np.arange(n), "exact")
    k = kc[0].reshape(-1, spec.n_kv_heads, spec.head_dim)[:n].astype(np.float64)
    np.testing.assert_allclose(np.sqrt(np.mean(k * k, axis=-1)), 1.0, rtol=1e-6)


# ---------------------------------------------------------------- proposal
def _propose(spec, W, ctx, mode="f32", P=4, shuffle=False, bonus=None, seed=5):
    kc, vc, bt = filled_context(spec, W, ctx, P, mode, seed=seed, shuffle=shuffle)
    bonus = np.arange(len(ctx)) * 7 + 3 if bonus is None else bonus
    return O.propose_block(spec, W, kc, vc, bt, bonus, ctx, mode)


def test_batch_invariance():
    ctx = [13, 0, 29]
    full = _propose(SMALL, W_SMALL, ctx)
    K = SMALL.block_size - 1
    for b, c in enumerate(ctx):
        kc, vc, bt = filled_context(SMALL, W_SMALL, ctx, 4, "f32", seed=5)
        one = O.propose_block(SMALL, W_SMALL, kc, vc, bt[b:b + 1], [b * 7 + 3], [c], "f32")
        np.testing.assert_array_equal(one["draft_token_ids"][0], full["draft_token_ids"][b])
        np.testing.assert_allclose(one["hidden"], full["hidden"][b * K:(b + 1) * K], rtol=1e-12)


@pytest.mark.parametrize("P", [1, 4, 16, 64])
def test_page_size_and_page_permutation_invariance(P):
    ctx = [21, 34]
    ref = _propose(SMALL, W_SMALL, ctx, P=4)
    got = _propose(SMALL, W_SMALL, ctx, P=P, shuffle=True)
    np.testing.assert_array_equal(got["draft_token_ids"], ref["draft_token_ids"])
    np.testing.assert_allclose(got["hidden"], ref["hidden"], rtol=1e-12, atol=1e-12)


def test_zero_layers_closed_form():
    """With no layers every kept row is the mask embedding, so all K drafts equal
    argmax(U rho(rms(E[mask]) w_fn)) whatever the context and bonus."""
    from dataclasses import replace
    spec = replace(SMALL, n_layers=0)
    W = numpy_weights(synth.make_weights(spec, seed=8))
    kc, vc = empty_cache(SMALL, 4, 4)
    res = O.propose_block(spec, W, kc[:0], vc[:0], np.zeros((2, 4), np.int32), [1, 2], [0, 0], "f32",
                          page_size=4, return_logits=True)
    e = W["embed"][spec.mask_token_id].astype(np.float64)
    f = e / np.sqrt(np.mean(e * e) + spec.rms_eps) * W["final_norm"]
    f = f.astype(np.float32).astype(np.float64)
    z = W["lm_head"].astype(np.float64) @ f
    best = [i for i in range(spec.vocab) if z[i] == z.max()][0]  # brute-force scan
    assert np.all(res["drafts_only"] == best)


def test_argmax_ties_take_lowest_index():
    spec = SMALL
    W = dict(W_SMALL)
    U = W["lm_head"].copy()
    kc, vc, bt = filled_context(spec, W, [6], 4, "f32", seed=5)
    first = O.propose_block(spec, W, kc, vc, bt, [3], [6], "f32")["drafts_only"][0]
    # duplicate each drafted row of U into a lower and a higher index
    for t in set(first.tolist()):
        U[0] = U[t]
        U[spec.vocab - 1] = U[t]
        W["lm_head"] = U
        again = O.propose_block(spec, W, kc, vc, bt, [3], [6], "f32")["drafts_only"][0]
        assert np.all(again[first == t] == 0)
        U = W_SMALL["lm_head"].copy()


# ---------------------------------------------------------------- verification
@pytest.mark.parametrize("K", [1, 2, 3])
def test_verify_brute_force_tiny_vocab(K):
    V = 3
    for d in itertools.product(range(V), repeat=K):
        for t in itertools.product(range(V), repeat=K + 1):
            a, out, nb = O.greedy_verify(np.array([d]), np.array([t]))
            a = int(a[0])
            assert 1 <= a <= K + 1
            # a - 1 drafts are accepted: exactly the matching prefix
            assert all(d[i] == t[i] for i in range(a - 1))
            assert a == K + 1 or d[a - 1] != t[a - 1]
            assert out[0, :a].tolist() == list(t[:a]) and np.all(out[0, a:] == -1)
            assert nb[0] == t[a - 1]
            # valid count (!= -1 and < V) equals a, so (1 + K) - valid = rejected drafts
            valid = int(np.sum((out[0] != -1) & (out[0] < V)))
            assert valid == a and (1 + K) - valid == K + 1 - a


def test_speculative_greedy_decoding_is_lossless():
    """Drafting + greedy verification emits exactly the target's greedy sequence, whatever
    the drafts (the frozen target verifies, so output equals standard decoding)."""
    V, K, steps = 5, 4, 60
    rng = np.random.default_rng(0)
    table = rng.integers(0, V, size=(V,) * 3)  # target's greedy next token given 3 last tokens

    def target_next(seq):
        return int(table[seq[-3], seq[-2], seq[-1]])

    ref = [0, 1, 2]
    while len(ref) < 3 + steps:
        ref.append(target_next(ref))
    for trial in range(20):
        seq = [0, 1, 2]
        while len(seq) < 3 + steps:
            # drafts: sometimes right, sometimes random
            drafts, s = [], list(seq)
            for _ in range(K):
                tok = target_next(s) if rng.random() < 0.6 else int(rng.integers(0, V))
                drafts.append(tok)
                s.append(tok)
            tgt = [target_next(seq + drafts[:i]) for i in range(K + 1)]
            a, out, nb = O.greedy_verify(np.array([drafts]), np.array([tgt]))
            seq.extend(out[0, : a[0]].tolist())
            assert seq[-1] == nb[0]
        assert seq[: 3 + steps] == ref[: 3 + steps]


def test_acceptance_metrics_identities():
    a = np.array([1, 4, 16, 2, 7])
    m = O.acceptance_metrics(a, 15)
    assert m["num_drafts"] == 5 and m["num_draft_tokens"] == 75
    assert m["num_accepted_tokens"] == int((a - 1).sum())
    assert m["acceptance_length"] == pytest.approx(a.mean())
    assert m["acceptance_rate"] == pytest.approx((a - 1).sum() / 75)
