"""Seeded synthetic inputs for the DFlash draft-proposal path.

This module draws random numbers and lays them out: drafter weights, the target's auxiliary
hidden states, context lengths, page tables, bonus tokens and the target's argmax tokens used
by greedy verification. It holds none of the method's arithmetic. Both the CPU oracle (through
the tests) and the GPU path consume exactly the arrays it returns.

Every tensor has its own counter-keyed Philox stream, keyed by (seed, tensor id, chunk).
Tensors can therefore be drawn lazily, in parallel, and per sequence: a test can regenerate
one sequence's context rows without drawing the whole batch.

Value recipe:
  * dense weights ~ N(0, 0.02);
  * norm weights ~ 1 + N(0, 0.01);
  * auxiliary states ~ N(0, 1).
In bf16 drafters each value is drawn in fp32 and rounded to nearest-even bf16 by torch's cast.
"""
from __future__ import annotations

import hashlib
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np
import torch

_CHUNK = 1 << 22  # elements per independent Philox stream


# --------------------------------------------------------------------------------------------
# Shapes
# --------------------------------------------------------------------------------------------
@dataclass(frozen=True)
class DrafterSpec:
    """Shape of a Qwen3-style DFlash drafter (Neuron design doc, "Draft Model")."""

    hidden: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    n_aux: int  # number of target layers whose states are concatenated
    target_hidden: int
    block_size: int  # [bonus, mask x (block_size-1)]
    mask_token_id: int
    rope_theta: float
    rms_eps: float = 1e-6
    dtype: str = "bf16"  # storage type of weights, auxiliary states, the KV cache and the block's q/k/v

    @property
    def n_drafts(self) -> int:
        return self.block_size - 1

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


@dataclass(frozen=True)
class Workload:
    """One synthetic drafting workload: a drafter, a batch and its context-length mix."""

    name: str
    spec: DrafterSpec
    batch: int
    ctx_lo: int  # context lengths are uniform integers in [ctx_lo, ctx_hi]
    ctx_hi: int
    inject_rows: int  # new context rows injected per sequence per step
    accept: tuple  # ("geometric", p) or ("per_position", q_lo, q_hi)
    page_size: int = 16
    shuffle_pages: bool = False
    seed: int = 0


QWEN3_8B_DRAFTER = DrafterSpec(
    hidden=4096, n_layers=5, n_q_heads=32, n_kv_heads=8, head_dim=128, intermediate=12288,
    vocab=151936, n_aux=5, target_hidden=4096, block_size=16, mask_token_id=151935,
    rope_theta=1e6, dtype="bf16")

WORKLOADS = {
    # tiny fp32 drafter: parity at a size the oracle finishes in well under a second
    "tiny_fp32_b1": Workload(
        "tiny_fp32_b1",
        DrafterSpec(hidden=256, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=64,
                    intermediate=768, vocab=4096, n_aux=3, target_hidden=256, block_size=8,
                    mask_token_id=4095, rope_theta=1e6, dtype="f32"),
        batch=1, ctx_lo=128, ctx_hi=128, inject_rows=8, accept=("geometric", 0.3)),
    # Qwen3-8B-shaped drafter, batch 1, 2048-token context (the headline throughput workload)
    "qwen3_8b_b1_ctx2048": Workload(
        "qwen3_8b_b1_ctx2048", QWEN3_8B_DRAFTER, batch=1, ctx_lo=2048, ctx_hi=2048,
        inject_rows=16, accept=("geometric", 0.15)),
    "qwen3_8b_b32_ragged": Workload(
        "qwen3_8b_b32_ragged", QWEN3_8B_DRAFTER, batch=32, ctx_lo=512, ctx_hi=8192,
        inject_rows=64, accept=("geometric", 0.15), shuffle_pages=True),
    "qwen3_8b_b1_ctx32768": Workload(
        "qwen3_8b_b1_ctx32768", QWEN3_8B_DRAFTER, batch=1, ctx_lo=32768, ctx_hi=32768,
        inject_rows=16, accept=("geometric", 0.15)),
    "llama31_8b_b128": Workload(
        "llama31_8b_b128",
        replace(QWEN3_8B_DRAFTER, intermediate=14336, vocab=128256, block_size=10,
                mask_token_id=128002, rope_theta=5e5),
        batch=128, ctx_lo=256, ctx_hi=4096, inject_rows=10,
        accept=("per_position", 0.5, 0.95)),
}


# --------------------------------------------------------------------------------------------
# Random streams
# --------------------------------------------------------------------------------------------
def _key(seed: int, *parts) -> int:
    h = hashlib.blake2b(repr((seed,) + parts).encode(), digest_size=8).digest()
    return int.from_bytes(h, "little")


def _normal_f32(n: int, seed: int, *tag) -> np.ndarray:
    """n standard normals (fp32), drawn from independent Philox streams per _CHUNK slice."""
    out = np.empty(n, dtype=np.float32)
    k = _key(seed, *tag)

    def work(i: int) -> None:
        g = np.random.Generator(np.random.Philox(key=[k, i]))
        g.standard_normal(out=out[i * _CHUNK:(i + 1) * _CHUNK], dtype=np.float32)

    nchunks = (n + _CHUNK - 1) // _CHUNK
    if nchunks <= 1:
        if n:
            work(0)
    else:
        with ThreadPoolExecutor(min(16, os.cpu_count() or 4)) as ex:
            list(ex.map(work, range(nchunks)))
    return out


def _rng(seed: int, *tag) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=[_key(seed, *tag), 0]))


def _to_storage(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(a)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


# --------------------------------------------------------------------------------------------
# Weights
# --------------------------------------------------------------------------------------------
def weight_shapes(spec: DrafterSpec) -> list[tuple[str, tuple[int, ...], str]]:
    """(name, shape, kind) in the fixed generation order; kind is 'dense' or 'norm'.

    Dense weights are row-major [out_features, in_features] (the F.linear convention)."""
    H, D = spec.hidden, spec.head_dim
    qd, kvd = spec.n_q_heads * D, spec.n_kv_heads * D
    out = [("fc", (H, spec.n_aux * spec.target_hidden), "dense"),
           ("hidden_norm", (H,), "norm"),
           ("embed", (spec.vocab, H), "dense"),
           ("lm_head", (spec.vocab, H), "dense"),
           ("final_norm", (H,), "norm")]
    for l in range(spec.n_layers):
        p = f"layers.{l}."
        out += [(p + "in_norm", (H,), "norm"),
                (p + "wq", (qd, H), "dense"),
                (p + "wk", (kvd, H), "dense"),
                (p + "wv", (kvd, H), "dense"),
                (p + "q_norm", (D,), "norm"),
                (p + "k_norm", (D,), "norm"),
                (p + "wo", (H, qd), "dense"),
                (p + "post_norm", (H,), "norm"),
                (p + "w_gate", (spec.intermediate, H), "dense"),
                (p + "w_up", (spec.intermediate, H), "dense"),
                (p + "w_down", (H, spec.intermediate), "dense")]
    return out


def make_weights(spec: DrafterSpec, seed: int = 0) -> dict[str, torch.Tensor]:
    """All drafter weights as CPU tensors of the storage dtype (bf16 or fp32)."""
    w = {}
    for name, shape, kind in weight_shapes(spec):
        n = math.prod(shape)
        a = _normal_f32(n, seed, "w", name)
        if kind == "dense":
            a *= np.float32(0.02)
        else:
            a *= np.float32(0.01)
            a += np.float32(1.0)
        w[name] = _to_storage(a.reshape(shape), spec.dtype)
    return w


def as_f32(t: torch.Tensor) -> np.ndarray:
    """Exact fp32 numpy copy of a CPU storage tensor (bf16 -> fp32 is exact)."""
    return t.float().numpy()


# --------------------------------------------------------------------------------------------
# Context
# --------------------------------------------------------------------------------------------
def context_lengths(wl: Workload) -> np.ndarray:
    if wl.ctx_lo == wl.ctx_hi:
        return np.full(wl.batch, wl.ctx_lo, dtype=np.int32)
    return _rng(wl.seed, "ctx").integers(wl.ctx_lo, wl.ctx_hi + 1, size=wl.batch).astype(np.int32)


def aux_states(spec: DrafterSpec, seed: int, seq: int, row0: int, nrows: int) -> list[torch.Tensor]:
    """The n_aux auxiliary target states of rows [row0, row0+nrows) of sequence `seq`.

    Returns n_aux CPU tensors [nrows, target_hidden] in ascending target-layer order. Each
    (sequence, row) has its own stream, so any row range is reproducible on its own."""
    Ht, A = spec.target_hidden, spec.n_aux
    out = np.empty((nrows, A, Ht), dtype=np.float32)
    for r in range(nrows):
        g = np.random.Generator(np.random.Philox(key=[_key(seed, "aux", seq), row0 + r]))
        g.standard_normal(out=out[r].reshape(-1), dtype=np.float32)
    return [_to_storage(np.ascontiguousarray(out[:, j, :]), spec.dtype) for j in range(A)]


def aux_states_fast(spec: DrafterSpec, seed: int, seq: int, row0: int, nrows: int) -> list[torch.Tensor]:
    """Same values as aux_states, drawn with one thread per row block (for long contexts)."""
    if nrows <= 256:
        return aux_states(spec, seed, seq, row0, nrows)
    Ht, A = spec.target_hidden, spec.n_aux
    out = np.empty((nrows, A, Ht), dtype=np.float32)
    k = _key(seed, "aux", seq)

    def work(lo: int) -> None:
        for r in range(lo, min(nrows, lo + 256)):
            g = np.random.Generator(np.random.Philox(key=[k, row0 + r]))
            g.standard_normal(out=out[r].reshape(-1), dtype=np.float32)

    with ThreadPoolExecutor(min(16, os.cpu_count() or 4)) as ex:
        list(ex.map(work, range(0, nrows, 256)))
    return [_to_storage(np.ascontiguousarray(out[:, j, :]), spec.dtype) for j in range(A)]


@dataclass
class PageLayout:
    block_table: np.ndarray  # [batch, max_blocks_per_seq] int32 physical page ids
    num_pages: int
    page_size: int

    @property
    def max_blocks(self) -> int:
        return self.block_table.shape[1]


def page_layout(wl: Workload, ctx: np.ndarray, extra_pages: int = 2) -> PageLayout:
    """Per-sequence page tables covering context + block positions.

    Pages are contiguous per sequence, or a seeded random permutation of all pages when the
    workload shuffles them. `extra_pages` physical pages are never referenced; tests fill them
    with a canary and check that they stay untouched."""
    P = wl.page_size
    maxb = (int(ctx.max()) + wl.spec.block_size + P - 1) // P
    used = wl.batch * maxb
    ids = np.arange(used, dtype=np.int64)
    if wl.shuffle_pages:
        ids = _rng(wl.seed, "pages").permutation(used + extra_pages)[:used]
    return PageLayout(ids.reshape(wl.batch, maxb).astype(np.int32), used + extra_pages, P)


def bonus_tokens(wl: Workload, step: int = 0) -> np.ndarray:
    return _rng(wl.seed, "bonus", step).integers(0, wl.spec.vocab, size=wl.batch).astype(np.int32)


def target_tokens(wl: Workload, drafts: np.ndarray, step: int = 0) -> np.ndarray:
    """Synthetic target argmax tokens [B, K+1] for greedy verification of `drafts` [B, K].

    ("geometric", p): copy the drafts up to a geometric(p) first mismatch.
    ("per_position", lo, hi): each sequence draws q ~ U(lo, hi); each position copies its
    draft with probability q. A mismatching token is (draft + 1 + U[0, V-2]) mod V, so it
    always differs; target[K] (the token after the last draft) is uniform."""
    drafts = np.asarray(drafts, dtype=np.int64)
    B, K = drafts.shape
    V = wl.spec.vocab
    g = _rng(wl.seed, "target", step)
    tgt = np.empty((B, K + 1), dtype=np.int64)
    for b in range(B):
        if wl.accept[0] == "geometric":
            m = int(g.geometric(wl.accept[1])) - 1  # matches before the first mismatch
            match = np.arange(K) < m
        else:
            q = g.uniform(wl.accept[1], wl.accept[2])
            match = g.random(K) < q
        other = (drafts[b] + 1 + g.integers(0, V - 1, size=K)) % V
        tgt[b, :K] = np.where(match, drafts[b], other)
        tgt[b, K] = g.integers(0, V)
    return tgt.astype(np.int32)
