"""Helpers shared by the CPU tests: small drafters and the oracle's cache setup."""
import numpy as np
import torch

from block_diffusion_drafting_concat_amd import synth
from oracle import dflash_oracle as O

# Deliberately non-square: hidden != q_heads*head_dim != intermediate, so that a transposed
# operand anywhere changes a shape or a value.
SMALL = synth.DrafterSpec(hidden=48, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=16,
                          intermediate=80, vocab=97, n_aux=3, target_hidden=40, block_size=5,
                          mask_token_id=96, rope_theta=1e4, dtype="f32")


def numpy_weights(W):
    return {k: synth.as_f32(v) for k, v in W.items()}


def empty_cache(spec, num_pages, page_size):
    shape = (num_pages, page_size, spec.n_kv_heads, spec.head_dim)
    return ([np.zeros(shape, np.float32) for _ in range(spec.n_layers)],
            [np.zeros(shape, np.float32) for _ in range(spec.n_layers)])


def filled_context(spec, W, ctx_lens, page_size, mode, seed=0, shuffle=False):
    """Oracle caches holding every sequence's injected context, plus the block table."""
    B = len(ctx_lens)
    maxb = (int(max(ctx_lens)) + spec.block_size + page_size - 1) // page_size
    ids = np.arange(B * maxb)
    if shuffle:
        ids = np.random.default_rng(seed + 99).permutation(B * maxb + 3)[: B * maxb]
    bt = ids.reshape(B, maxb).astype(np.int32)
    kc, vc = empty_cache(spec, B * maxb + 3, page_size)
    for b, c in enumerate(ctx_lens):
        if c == 0:
            continue
        aux = [synth.as_f32(a) for a in synth.aux_states(spec, seed, b, 0, c)]
        pos = np.arange(c)
        slots = O.paged_slots(bt, np.full(c, b), pos, page_size)
        O.inject_context_kv(spec, W, kc, vc, aux, pos, slots, mode)
    return kc, vc, bt
